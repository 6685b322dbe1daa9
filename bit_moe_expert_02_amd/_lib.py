"""ctypes binding of libmoe.so: argument marshalling only.

Function names follow include/moe.h.  Device buffers are torch tensors on the
current HIP device; the stream is torch's current stream.  Nothing here
computes any part of the layer: every step runs in the library.  If the
library is missing the import fails loudly -- there is no fallback path.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EFORMAT, MOE_EWORKSPACE, MOE_EDEVICE, MOE_ECODE, MOE_ETIMEOUT = \
    0, -1, -2, -3, -4, -5, -6, -7
MOE_ACT_MXFP8 = 1
FMT = {"TERN160": 1, "Q2_0": 2, "Q3": 3, "MXFP4": 4, "Q8": 5}
FMT_NAME = {v: k for k, v in FMT.items()}
MAX_DECODE_ROWS = 8
MAX_TOP_K = 8

# every symbol include/moe.h declares
EXPORTS = ("moe_status_string", "moe_packed_bytes", "moe_pack", "moe_unpack",
           "moe_workspace_bytes", "moe_check_experts", "moe_route", "moe_expert_ffn",
           "moe_layer", "moe_layer_profiled", "moe_stack_decode", "moe_quant_mxfp8",
           "moe_stream_read", "moe_set_spin_limit", "moe_workspace_status", "moe_layer_noalloc",
           "moe_allocate_formats", "moe_cache_create", "moe_cache_destroy", "moe_cache_plan",
           "moe_copy_share", "moe_cpu_expert_ffn", "moe_add_chain")


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status} ({status_string(status)})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("sel_bias", ctypes.c_void_p),
                ("weights", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("shared", ctypes.c_void_p)]


class ExpertRef(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("gate", ctypes.c_uint64), ("up", ctypes.c_uint64), ("down", ctypes.c_uint64)]


EXPERT_REF_DTYPE = np.dtype([("fmt", "<u4"), ("reserved", "<u4"), ("gate", "<u8"),
                             ("up", "<u8"), ("down", "<u8")])
assert EXPERT_REF_DTYPE.itemsize == ctypes.sizeof(ExpertRef) == 32

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_moe_expert_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dims_p = ctypes.POINTER(Dims)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_packed_bytes.restype = sz
        L.moe_packed_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.moe_pack.restype = ctypes.c_int
        L.moe_pack.argtypes = [ctypes.c_int, vp, i64, i64, vp, sz, ctypes.c_int]
        L.moe_unpack.restype = ctypes.c_int
        L.moe_unpack.argtypes = [ctypes.c_int, vp, sz, i64, i64, vp, ctypes.c_int]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [dims_p, i32]
        L.moe_check_experts.restype = ctypes.c_int
        L.moe_check_experts.argtypes = [dims_p, vp, i32, sz]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [dims_p, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [dims_p, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_layer.restype = ctypes.c_int
        L.moe_layer.argtypes = [dims_p, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_layer_noalloc.restype = ctypes.c_int
        L.moe_layer_noalloc.argtypes = [dims_p, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_layer_profiled.restype = ctypes.c_int
        L.moe_layer_profiled.argtypes = [dims_p, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         vp, vp, i32]
        L.moe_quant_mxfp8.restype = ctypes.c_int
        L.moe_quant_mxfp8.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_set_spin_limit.restype = ctypes.c_int32
        L.moe_set_spin_limit.argtypes = [i32]
        L.moe_stream_read.restype = ctypes.c_int
        L.moe_stream_read.argtypes = [vp, sz, vp, i32, i32, vp]
        L.moe_workspace_status.restype = ctypes.c_int
        L.moe_workspace_status.argtypes = [vp, sz, vp]
        L.moe_allocate_formats.restype = ctypes.c_int
        L.moe_allocate_formats.argtypes = [i32, i32, vp, vp, vp, vp, ctypes.c_double, i32, i32, i32, vp,
                                           vp, vp]
        L.moe_stack_decode.restype = ctypes.c_int
        L.moe_stack_decode.argtypes = [dims_p, i32, ctypes.POINTER(LayerWeights), i32, vp, vp, vp,
                                       vp, vp, vp, sz, vp]
        L.moe_cache_create.restype = ctypes.c_int
        L.moe_cache_create.argtypes = [i32, i32, i32, ctypes.POINTER(vp)]
        L.moe_cache_destroy.restype = None
        L.moe_cache_destroy.argtypes = [vp]
        L.moe_cache_plan.restype = ctypes.c_int
        L.moe_cache_plan.argtypes = [vp, i32, i32, i32, vp, ctypes.c_double, vp, vp, vp, vp, vp, vp, vp]
        L.moe_copy_share.restype = ctypes.c_double
        L.moe_copy_share.argtypes = [ctypes.c_double, ctypes.c_double]
        L.moe_cpu_expert_ffn.restype = ctypes.c_int
        L.moe_cpu_expert_ffn.argtypes = [dims_p, i32, vp, vp, vp, vp, i32, vp, vp, vp, i32]
        L.moe_add_chain.restype = ctypes.c_int
        L.moe_add_chain.argtypes = [vp, vp, vp, vp, i32, i32, vp]
        _lib = L
    return _lib


def status_string(status):
    return lib().moe_status_string(int(status)).decode()


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


# ----------------------------------------------------------------------------- host packer
def packed_bytes(fmt, n, k):
    return int(lib().moe_packed_bytes(FMT[fmt], int(n), int(k)))


def pack(fmt, w, nthreads=0):
    """fp32 [n, k] (numpy) -> packed uint8 array (numpy), via moe_pack."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    nbytes = packed_bytes(fmt, n, k)
    if nbytes == 0:
        raise MoeError("moe_packed_bytes", MOE_ESHAPE)
    out = np.empty(nbytes, np.uint8)
    _check("moe_pack", lib().moe_pack(FMT[fmt], w.ctypes.data, n, k, out.ctypes.data, nbytes,
                                      int(nthreads)))
    return out


def pack_into(fmt, w, out, nthreads=0):
    """Packs into a preallocated uint8 numpy array view (for large buffers)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    _check("moe_pack", lib().moe_pack(FMT[fmt], w.ctypes.data, n, k, out.ctypes.data, out.size,
                                      int(nthreads)))


def unpack(fmt, buf, n, k, nthreads=0):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    out = np.empty((n, k), np.float32)
    _check("moe_unpack", lib().moe_unpack(FMT[fmt], buf.ctypes.data, buf.size, int(n), int(k),
                                          out.ctypes.data, int(nthreads)))
    return out


def allocate_formats(err, tokens, energy, fmt_bytes, max_tern_frac=0.5, min_tokens=8, edge_first=2,
                     edge_last=3):
    """moe_allocate_formats: err [L, E, 3] (TERN160, Q2_0, Q3), tokens [L, E],
    energy [L], fmt_bytes [3] -> (format names [L, E], total cost, total bytes)."""
    err = np.ascontiguousarray(err, np.float64)
    tokens = np.ascontiguousarray(tokens, np.int32)
    energy = np.ascontiguousarray(energy, np.float64)
    fb = np.ascontiguousarray(fmt_bytes, np.uint64)
    L_, E_ = tokens.shape
    out = np.empty((L_, E_), np.uint8)
    cost = ctypes.c_double()
    nbytes = ctypes.c_uint64()
    _check("moe_allocate_formats", lib().moe_allocate_formats(
        L_, E_, err.ctypes.data, tokens.ctypes.data, energy.ctypes.data, fb.ctypes.data,
        float(max_tern_frac), int(min_tokens), int(edge_first), int(edge_last), out.ctypes.data,
        ctypes.byref(cost), ctypes.byref(nbytes)))
    names = np.vectorize(FMT_NAME.get)(out)
    return names, cost.value, int(nbytes.value)


# ----------------------------------------------------------------------------- device calls
def dims(hidden, inter, n_experts, top_k, flags=0):
    return Dims(hidden, inter, n_experts, top_k, flags)


def workspace_bytes(d, rows):
    return int(lib().moe_workspace_bytes(ctypes.byref(d), int(rows)))


def check_experts(d, table, weights_bytes):
    table = np.ascontiguousarray(table, dtype=EXPERT_REF_DTYPE)
    return int(lib().moe_check_experts(ctypes.byref(d), table.ctypes.data, len(table),
                                       int(weights_bytes)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def moe_route(d, x, rows, w_router, bias, idx, wts, ws, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(d), _ptr(x), int(rows), _ptr(w_router),
                                        _ptr(bias), _ptr(idx), _ptr(wts), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_ffn(d, x, rows, idx, wts, weights, experts, shared, y, ws, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(d), _ptr(x), int(rows), _ptr(idx), _ptr(wts), _ptr(weights), _ptr(experts),
        _ptr(shared), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer(d, x, rows, w_router, bias, weights, experts, shared, idx, wts, y, ws, stream=None):
    _check("moe_layer", lib().moe_layer(
        ctypes.byref(d), _ptr(x), int(rows), _ptr(w_router), _ptr(bias), _ptr(weights),
        _ptr(experts), _ptr(shared), _ptr(idx), _ptr(wts), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_noalloc(d, x, rows, w_router, bias, weights, experts, shared, idx, wts, y, stream=None):
    """moe_layer on the library's fixed per-GPU workspace (no allocation)."""
    _check("moe_layer_noalloc", lib().moe_layer_noalloc(
        ctypes.byref(d), _ptr(x), int(rows), _ptr(w_router), _ptr(bias), _ptr(weights),
        _ptr(experts), _ptr(shared), _ptr(idx), _ptr(wts), _ptr(y), _stream(stream)))


def moe_layer_profiled(d, x, rows, w_router, bias, weights, experts, shared, idx, wts, y, ws,
                       events, stream=None):
    arr = (ctypes.c_void_p * len(events))(*events)
    _check("moe_layer_profiled", lib().moe_layer_profiled(
        ctypes.byref(d), _ptr(x), int(rows), _ptr(w_router), _ptr(bias), _ptr(weights),
        _ptr(experts), _ptr(shared), _ptr(idx), _ptr(wts), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream), arr, len(events)))


def layer_weights(layers):
    """ctypes array of LayerWeights for objects with router, bias, weights, experts, shared."""
    arr = (LayerWeights * len(layers))()
    for i, dl in enumerate(layers):
        addr = [None if t is None else t.data_ptr()
                for t in (dl.router, dl.bias, dl.weights, dl.experts, dl.shared)]
        arr[i] = LayerWeights(*addr)
    return arr


def moe_stack_decode(d, layers, rows, x_all, noise, y_all, idx_all, wts_all, ws, stream=None):
    """layers: a LayerWeights array (layer_weights()); the other buffers are torch tensors."""
    _check("moe_stack_decode", lib().moe_stack_decode(
        ctypes.byref(d), len(layers), layers, int(rows), _ptr(x_all), _ptr(noise), _ptr(y_all),
        _ptr(idx_all), _ptr(wts_all), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_quant_mxfp8(x, rows, k, codes, scales, stream=None):
    _check("moe_quant_mxfp8", lib().moe_quant_mxfp8(_ptr(x), int(rows), int(k), _ptr(codes),
                                                    _ptr(scales), _stream(stream)))


def moe_stream_read(buf, nbytes, sink, grid, unroll, stream=None):
    """Measurement aid: the streaming-read kernel over the first nbytes of buf."""
    _check("moe_stream_read", lib().moe_stream_read(_ptr(buf), int(nbytes), _ptr(sink), int(grid),
                                                    int(unroll), _stream(stream)))


def moe_workspace_status(ws, stream=None):
    """MOE_OK or MOE_ETIMEOUT (a fused call's hand-off wait gave up since the
    last query); synchronises the stream and clears the workspace's error word."""
    st = lib().moe_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if st not in (MOE_OK, MOE_ETIMEOUT):
        raise MoeError("moe_workspace_status", st)
    return st


def moe_set_spin_limit(polls):
    """Polls before a hand-off wait of the fused launch gives up; returns the previous limit."""
    prev = lib().moe_set_spin_limit(int(polls))
    if prev < 0:
        raise MoeError("moe_set_spin_limit", prev)
    return prev


# ----------------------------------------------------------------------------- stacks larger than HBM
class SlotCache:
    """moe_cache_create / moe_cache_plan / moe_cache_destroy (host only)."""

    def __init__(self, n_layers, n_experts, n_slots):
        h = ctypes.c_void_p()
        _check("moe_cache_create", lib().moe_cache_create(int(n_layers), int(n_experts), int(n_slots),
                                                          ctypes.byref(h)))
        self.h, self.n_experts, self.n_slots = h, int(n_experts), int(n_slots)

    def plan(self, layer, idx, copy_share):
        """idx: host int32 [rows, top_k] -> dict(slot_of [E], copies [(expert, slot)],
        cpu [experts], idx_gpu [rows, top_k])."""
        idx = np.ascontiguousarray(idx, np.int32)
        rows, k = idx.shape
        n = rows * k
        slot_of = np.empty(self.n_experts, np.int32)
        ce, cs, cpu, idx_gpu = (np.empty(max(n, 1), np.int32) for _ in range(4))
        nc, nu = ctypes.c_int32(), ctypes.c_int32()
        _check("moe_cache_plan", lib().moe_cache_plan(
            self.h, int(layer), rows, k, idx.ctypes.data, float(copy_share), slot_of.ctypes.data,
            ce.ctypes.data, cs.ctypes.data, ctypes.byref(nc), cpu.ctypes.data, ctypes.byref(nu),
            idx_gpu.ctypes.data))
        return {"slot_of": slot_of,
                "copies": [(int(ce[i]), int(cs[i])) for i in range(nc.value)],
                "cpu": [int(cpu[i]) for i in range(nu.value)],
                "idx_gpu": idx_gpu[:n].reshape(rows, k).copy()}

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def copy_share(pcie_bytes_per_s, cpu_bytes_per_s):
    return float(lib().moe_copy_share(float(pcie_bytes_per_s), float(cpu_bytes_per_s)))


def cpu_expert_ffn(d, fmt, gate, up, down, x_bf16, row_ids, row_w, y, nthreads=0):
    """moe_cpu_expert_ffn on host numpy arrays: y [rows, H] fp32 accumulates
    row_w[j] * FFN(x[row_ids[j]])."""
    for a in (gate, up, down, x_bf16, y):
        assert a.flags.c_contiguous
    assert y.dtype == np.float32
    rid = np.ascontiguousarray(row_ids, np.int32)
    rw = np.ascontiguousarray(row_w, np.float32)
    _check("moe_cpu_expert_ffn", lib().moe_cpu_expert_ffn(
        ctypes.byref(d), FMT[fmt] if isinstance(fmt, str) else int(fmt), gate.ctypes.data,
        up.ctypes.data, down.ctypes.data, x_bf16.ctypes.data, len(rid), rid.ctypes.data,
        rw.ctypes.data, y.ctypes.data, int(nthreads)))


def moe_add_chain(y, add, noise, x_next, stream=None):
    """y [rows, hidden] fp32 device tensor; add / noise likewise or None; x_next
    [rows, hidden] int16 (bf16 bits) or None."""
    rows, hidden = y.shape
    _check("moe_add_chain", lib().moe_add_chain(_ptr(y), _ptr(add), _ptr(noise), _ptr(x_next),
                                                int(rows), int(hidden), _stream(stream)))
