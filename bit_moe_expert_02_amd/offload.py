"""Decode over a stack larger than HBM: routed experts in a pinned host store,
a device slot cache in front of it, misses copied over PCIe or computed on the
host CPU.

"DeepSeek-V4.1-Flash served three ways on 4xL20", section 3C (a pinned host
expert store, a device slot cache, misses split between copies and the CPU by
the ratio of measured bandwidths) and section 5 (f / (1 - f) = effective
PCIe rate / effective CPU rate); "[Strata] DeepSeek V4.1 Flash on a single
4090", section 5.2 (a device LRU in front of a pinned host arena).

One layer step (rows <= 8):
  1. moe_route on the device -> idx, wts; both copied to the host (the step's
     one synchronisation: the plan needs the selection);
  2. moe_cache_plan: hits, copies (expert -> slot, LRU) and CPU experts;
  3. the copies, pinned host -> device slots, queued on the stream; the
     expert table of the resident experts queued after them;
  4. moe_expert_ffn on the device with the CPU's pairs marked -1, while the
     host computes the CPU's experts with moe_cpu_expert_ffn;
  5. the CPU's sum copied to the device and added by moe_add_chain, which
     also rounds x for the next layer.
The router weights, selection biases and shared experts stay resident: only
routed experts move.  Every arithmetic step runs in the library (device
kernels or its host FFN); this module moves bytes and marshals arguments.
"""

import time

import numpy as np

from . import _lib as L

ALIGN = 256


def _align(v):
    return (v + ALIGN - 1) // ALIGN * ALIGN


def blob_layout(fmt, hidden, inter):
    """(gate, up, down, total) byte offsets of one expert's matrices in a blob."""
    gu = L.packed_bytes(fmt, inter, hidden)
    dn = L.packed_bytes(fmt, hidden, inter)
    up = _align(gu)
    down = _align(up + gu)
    return 0, up, down, _align(down + dn)


class OffloadStack:
    """A stack of n_layers routed-MoE layers whose routed experts live in pinned
    host memory.

    routers   list of device fp32 [E, H] tensors;  biases  list of device fp32
              [E] tensors or None
    shared    list of (fmt, gate, up, down) host uint8 arrays or None per layer
    fmts      [n_layers][E] format names of the routed experts
    fill      fill(layer, expert, dst) writes the expert's blob (blob_layout)
              into the host uint8 array dst
    n_slots   device expert slots (each sized for the largest format present)
    copy_share  share of misses copied (0..1), or None: measured at set-up from
              one pinned copy and one CPU expert (moe_copy_share)
    """

    def __init__(self, hidden, inter, n_experts, top_k, routers, biases, shared, fmts, fill, n_slots,
                 copy_share=None, cpu_threads=0, device="cuda"):
        import torch
        self.H, self.I, self.E, self.k = hidden, inter, n_experts, top_k
        self.n_layers = len(routers)
        self.dims = L.dims(hidden, inter, n_experts, top_k)
        self.routers, self.biases = routers, biases
        self.fmts = [list(f) for f in fmts]
        self.cpu_threads = cpu_threads
        present = sorted({f for row in self.fmts for f in row})
        self.slot_bytes = max(blob_layout(f, hidden, inter)[3] for f in present)
        # host store: every routed expert's blob, pinned
        self.host_off = np.zeros((self.n_layers, n_experts), np.int64)
        self.blob_size = np.zeros((self.n_layers, n_experts), np.int64)
        off = 0
        for li in range(self.n_layers):
            for e in range(n_experts):
                size = blob_layout(self.fmts[li][e], hidden, inter)[3]
                self.host_off[li, e] = off
                self.blob_size[li, e] = size
                off += size
        self.store = torch.empty(off, dtype=torch.uint8, pin_memory=True)
        self.store_np = self.store.numpy()
        for li in range(self.n_layers):
            for e in range(n_experts):
                o = int(self.host_off[li, e])
                fill(li, e, self.store_np[o:o + int(self.blob_size[li, e])])
        # device weights: the slot pool, then every layer's shared expert
        self.n_slots = int(n_slots)
        pool_bytes = self.n_slots * self.slot_bytes
        sh_refs, sh_parts, soff = [], [], pool_bytes
        for sh in shared:
            if sh is None:
                sh_refs.append(None)
                continue
            f, g, u, d = sh
            lay = blob_layout(f, hidden, inter)
            ref = np.zeros(1, L.EXPERT_REF_DTYPE)
            ref[0] = (L.FMT[f], 0, soff + lay[0], soff + lay[1], soff + lay[2])
            sh_refs.append(ref)
            sh_parts.append((soff, lay, (g, u, d)))
            soff += lay[3]
        self.weights = torch.zeros(soff, dtype=torch.uint8, device=device)
        for base, lay, mats in sh_parts:
            for o, m in zip(lay[:3], mats):
                self.weights[base + o: base + o + m.size].copy_(torch.from_numpy(m))
        self.shared = [None if r is None else torch.from_numpy(r.view(np.uint8).copy()).to(device)
                       for r in sh_refs]
        self.cache = L.SlotCache(self.n_layers, n_experts, self.n_slots)
        # per-step staging: pinned host buffers the device reads asynchronously
        self.table_h = torch.empty(n_experts * L.EXPERT_REF_DTYPE.itemsize, dtype=torch.uint8,
                                   pin_memory=True)
        self.table_d = torch.empty_like(self.table_h, device=device)
        self.device = device
        self.stats = {"hits": 0, "copies": 0, "cpu": 0, "copy_bytes": 0, "cpu_bytes": 0,
                      "cpu_seconds": 0.0, "steps": 0}
        self.rates = None
        self.copy_share = copy_share if copy_share is not None else self.measure_share()

    # ------------------------------------------------------------------ set-up
    def measure_share(self):
        """Times one pinned host -> device copy and one CPU expert at one row
        (packed bytes per second each), then moe_copy_share."""
        import torch
        n = min(int(self.store.numel()), 256 << 20)
        dst = torch.empty(n, dtype=torch.uint8, device=self.device)
        dst.copy_(self.store[:n], non_blocking=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dst.copy_(self.store[:n], non_blocking=True)
        torch.cuda.synchronize()
        pcie = n / (time.perf_counter() - t0)
        del dst
        x = np.zeros((1, self.H), np.uint16)
        y = np.zeros((1, self.H), np.float32)
        li, e = 0, 0
        t0 = time.perf_counter()
        self._cpu_expert(li, e, x, [0], [1.0], y)
        cpu = float(self.blob_size[li, e]) / (time.perf_counter() - t0)
        self.rates = {"pcie_bytes_per_s": pcie, "cpu_bytes_per_s": cpu}
        return L.copy_share(pcie, cpu)

    def _views(self, li, e):
        o = int(self.host_off[li, e])
        f = self.fmts[li][e]
        g0, u0, d0, _ = blob_layout(f, self.H, self.I)
        gu = L.packed_bytes(f, self.I, self.H)
        dn = L.packed_bytes(f, self.H, self.I)
        s = self.store_np
        return f, s[o + g0:o + g0 + gu], s[o + u0:o + u0 + gu], s[o + d0:o + d0 + dn]

    def _cpu_expert(self, li, e, x_host, row_ids, row_w, y_host):
        f, g, u, d = self._views(li, e)
        L.cpu_expert_ffn(self.dims, f, g, u, d, x_host, row_ids, row_w, y_host, self.cpu_threads)

    # ------------------------------------------------------------------ one step
    def layer_step(self, li, x, rows, idx, wts, y, ws, noise=None, x_next=None):
        """Layer li on device x [rows, H] bf16 bits -> device y [rows, H] fp32
        (and x_next when given).  idx / wts: device int32 / fp32 [rows, k]
        outputs of the routing."""
        import torch
        L.moe_route(self.dims, x, rows, self.routers[li], self.biases[li], idx, wts, ws)
        idx_h = idx.cpu().numpy()           # waits for the routing
        wts_h = wts.cpu().numpy()
        p = self.cache.plan(li, idx_h, self.copy_share)
        # the CPU's rows of x, taken now so that nothing below waits for the
        # device part
        x_h = x.cpu().numpy().view(np.uint16).reshape(rows, self.H) if p["cpu"] else None
        st = self.stats
        st["steps"] += 1
        st["copies"] += len(p["copies"])
        st["cpu"] += len(p["cpu"])
        st["hits"] += len(set(idx_h.reshape(-1).tolist())) - len(p["copies"]) - len(p["cpu"])
        for e, s in p["copies"]:
            o, n = int(self.host_off[li, e]), int(self.blob_size[li, e])
            self.weights[s * self.slot_bytes: s * self.slot_bytes + n].copy_(self.store[o:o + n],
                                                                             non_blocking=True)
            st["copy_bytes"] += n
        table = np.zeros(self.E, L.EXPERT_REF_DTYPE)
        for e in range(self.E):
            s = int(p["slot_of"][e])
            f = self.fmts[li][e]
            g0, u0, d0, _ = blob_layout(f, self.H, self.I)
            base = max(s, 0) * self.slot_bytes   # a non-resident expert is never read
            table[e] = (L.FMT[f], 0, base + g0, base + u0, base + d0)
        self.table_h.numpy()[:] = table.view(np.uint8)
        self.table_d.copy_(self.table_h, non_blocking=True)
        idx_gpu = torch.from_numpy(p["idx_gpu"]).to(self.device, non_blocking=False)
        L.moe_expert_ffn(self.dims, x, rows, idx_gpu, wts, self.weights, self.table_d,
                         self.shared[li], y, ws)
        add = None
        if p["cpu"]:
            t0 = time.perf_counter()
            y_cpu = np.zeros((rows, self.H), np.float32)
            for e in p["cpu"]:
                pairs = np.argwhere(idx_h == e)
                self._cpu_expert(li, e, x_h, pairs[:, 0], wts_h[pairs[:, 0], pairs[:, 1]], y_cpu)
                st["cpu_bytes"] += int(self.blob_size[li, e])
            st["cpu_seconds"] += time.perf_counter() - t0
            add = torch.from_numpy(y_cpu).to(self.device)
        L.moe_add_chain(y, add, noise, x_next)
        return p

    def decode(self, x0, rows, noise=None, ws=None):
        """All layers chained: x_{l+1} = bf16(y_l + noise_l).  x0 device int16
        [rows, H]; noise device fp32 [n_layers, rows, H] or None.  Returns
        (x_all [n_layers + 1, rows, H], y_all, idx_all)."""
        import torch
        from . import layer as LY
        n = self.n_layers
        x_all = torch.zeros((n + 1, rows, self.H), dtype=torch.int16, device=self.device)
        x_all[0].copy_(x0)
        y_all = torch.zeros((n, rows, self.H), dtype=torch.float32, device=self.device)
        idx_all = torch.zeros((n, rows, self.k), dtype=torch.int32, device=self.device)
        wts = torch.zeros((rows, self.k), dtype=torch.float32, device=self.device)
        ws = ws if ws is not None else LY.workspace(self.dims, rows, self.device)
        for li in range(n):
            self.layer_step(li, x_all[li], rows, idx_all[li], wts, y_all[li], ws,
                            None if noise is None else noise[li], x_all[li + 1])
        return x_all, y_all, idx_all

    def close(self):
        self.cache.close()
