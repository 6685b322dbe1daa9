/*
 * moe.h -- C ABI of libmoe: a low-bit routed-MoE expert FFN for one AMD
 * MI355X (gfx950).
 *
 * The computation (sources cited by page title and section):
 *   - "DeepSeek-V4.1-Flash served three ways on 4xL20" (lcz.me/topic/2356),
 *     section 1: the decoder layer -- hidden 5120, moe_intermediate 2304,
 *     384 routed experts, top-6, one shared expert; section 2: an expert is
 *     three 5120x2304 matrices and decode cost is the expert bytes a token
 *     selects.
 *   - "[Strata] DeepSeek V4.1 Flash on a single 4090" (lcz.me/post/25274),
 *     section 5.1: per-expert mixed low-bit formats (ternary, Q2_0, Q3);
 *     section 5.3: a selection-only route bias that leaves mixing weights exact;
 *     section 2: the int8 (Q8_0) dense half.
 *
 * Per layer and per row r of x:
 *     logits[r,e] = sum_h x[r,h] * Wr[e,h]                 (router GEMV, fp64 sums)
 *     S_r         = the top_k experts by logits[r,e] + bias[e],
 *                   ties toward the lower expert id, ordered by key desc
 *     w[r,e]      = softmax over S_r of the UNBIASED logits
 *     y[r]        = sum_{e in S_r, ascending e} w[r,e] * FFN_e(x[r]) + FFN_shared(x[r])
 *     FFN(x)      = W_down (silu(W_gate x) * (W_up x)),  silu(z) = z / (1 + e^-z)
 *
 * Weight formats (block layouts are this library's definitions; the pages
 * give the formats' names and bit rates only):
 *   MOE_FMT_Q2_0    64 w/block: 16 code bytes (weight i = bits [2i,2i+2) of the
 *                   128-bit LE code word) + fp16 d;  value d*(c-2).     2.25 bpw
 *   MOE_FMT_TERN160 160 w/block: 32 bytes, byte j = sum_m (t_{5j+m}+1)*3^m
 *                   (values 243..255 invalid) + fp16 d; value d*t.  Rows whose
 *                   length is not a multiple of 160 are padded with zero trits.
 *   MOE_FMT_Q3      256 w/block, 16 sub-blocks of 16: 96 code bytes of 3-bit
 *                   q, fp16 d, 12 bytes of sixteen 6-bit u_j at bits
 *                   [6j,6j+6);  value d*(u_j-32)*(q-4).  3.4375 bpw.  Codes
 *                   by quarter block (six little-endian words at byte 24u):
 *                   weight t of the quarter's sub-block j is in half h = t/8
 *                   of pair p = t%8; field f = the 3 bits at 16h+1+3f of a
 *                   word; p < 6: q = 3j + p%3, field p/3 (+3 if q >= 6) of
 *                   word q%6; p >= 6: q = 2j + p-6, field 2 of word q (q < 6),
 *                   else code bit b is bit 16h of word 3(q-6)+b
 *   MOE_FMT_MXFP4   32 w/block: 16 bytes of e2m1 (element i in byte i/2, low
 *                   nibble for even i) + e8m0 E (255 invalid);
 *                   value 2^(E-127)*e2m1 (OCP MX v1.0).                 4.25 bpw
 *   MOE_FMT_Q8      32 w/block: 32 int8 + fp16 d; value d*q.           8.5 bpw
 * Every matrix W[N x K] is planar: codes of all blocks in (row, block) order,
 * then the scales in the same order (Q3: all fp16 d, then all 12-byte u records).
 *
 * Conventions for every entry point:
 *   - Return value: MOE_OK (0) or a negative moe_status.  Argument, shape and
 *     format errors are detected on the host before anything is launched.
 *   - Device pointers are HIP device (or managed) memory on the current device.
 *     The caller owns every buffer; the library never allocates or frees.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls are
 *     asynchronous on it; nothing synchronises the host.  Device faults surface
 *     at the caller's next synchronisation.
 *   - The library's only mutable global state is a thread-safe counter that
 *     gives every moe_layer call a process-unique tag, and per device the
 *     number of fused-layer workgroups the device holds at once (looked up
 *     on the first call).  Calls on different streams with different
 *     workspaces may run concurrently.
 */
#ifndef BIT_MOE_H
#define BIT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,      /* null pointer, negative size, bad flag            */
  MOE_ESHAPE = -2,      /* dims the kernels do not support / K not a block multiple */
  MOE_EFORMAT = -3,     /* unknown format tag                                */
  MOE_EWORKSPACE = -4,  /* workspace smaller than moe_workspace_bytes()      */
  MOE_EDEVICE = -5,     /* a HIP launch or runtime call failed               */
  MOE_ECODE = -6,       /* moe_unpack met an invalid code (ternary byte > 242, e8m0 255) */
  MOE_ETIMEOUT = -7     /* moe_workspace_status: a hand-off wait of a fused call gave up */
} moe_status;

typedef enum {
  MOE_FMT_TERN160 = 1,
  MOE_FMT_Q2_0 = 2,
  MOE_FMT_Q3 = 3,
  MOE_FMT_MXFP4 = 4,
  MOE_FMT_Q8 = 5
} moe_format;

/* Largest number of rows the decode kernels take in one call (one token or
 * one speculative-verify window of up to 8 candidates). */
#define MOE_MAX_DECODE_ROWS 8
/* Largest top_k the selection kernel takes. */
#define MOE_MAX_TOP_K 8
/* Largest row count of moe_expert_ffn's many-row (prefill) path. */
#define MOE_MAX_PREFILL_ROWS 8192

const char* moe_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Host-side packer.  Pure functions of their arguments, thread-safe, touch  */
/* no device.                                                                */
/* ------------------------------------------------------------------------ */

/* Bytes of one packed N x K matrix in `fmt`: N * ceil(K/B) * (code + scale
 * bytes).  Returns 0 for an unknown format, n <= 0, k <= 0, or (except
 * TERN160) K not a multiple of the block size. */
size_t moe_packed_bytes(int fmt, int64_t n, int64_t k);

/* Round-to-nearest packing of a row-major fp32 matrix w[n x k] (host memory)
 * into dst (host, dst_bytes >= moe_packed_bytes).  Arithmetic is IEEE fp32
 * with ties to even; fp16 scales round to nearest even and saturate at
 * +-65504.  Per-format rules:
 *   Q2_0    m = block element of largest |w| (first on ties), d = fp16(m/-2),
 *           c = clamp(rint(w/d)+2, 0, 3)           (d == 0: c = 2)
 *   TERN160 d = fp16(max|w|), t = clamp(rint(w/d), -1, 1)   (d == 0: t = 0)
 *   Q3      sigma_j = m_j/-4 per sub-block, d = fp16(max|sigma_j|/31),
 *           u_j = clamp(rint(sigma_j/d), -31, 31) + 32,
 *           q = clamp(rint(w/(d*(u_j-32))) + 4, 0, 7)  (zero divisor: u=32, q=4)
 *   MXFP4   E = clamp(floor(log2 amax) - 2 + 127, 0, 254) (amax 0: E 0),
 *           element = e2m1 nearest-even of w/2^(E-127), saturating at 6;
 *           the sign bit is the sign bit of w
 *   Q8      d = fp16(max|w|/127), q = clamp(rint(w/d), -127, 127)
 * nthreads <= 0 uses the hardware concurrency.  Non-finite inputs give
 * unspecified (but valid) codes. */
int moe_pack(int fmt, const float* w, int64_t n, int64_t k, void* dst, size_t dst_bytes,
             int nthreads);

/* Exact decode of a packed matrix (host) to fp32 w[n x k] (host).  TERN160
 * padding columns are dropped.  Returns MOE_ECODE on an invalid code.
 * Every decoded value is exact in fp32, except MXFP4 values of magnitude
 * 2^128 and above (E = 254 with |e2m1| >= 2), which decode to +-inf. */
int moe_unpack(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k, float* w,
               int nthreads);

/* Per-expert format allocation for a stack of n_layers x n_experts routed
 * experts ("[Strata] DeepSeek V4.1 Flash on a single 4090", section 5.1):
 * each expert gets TERN160, Q2_0 or Q3 so that the stack's bytes stay within
 * those of the whole stack in Q2_0, by a Lagrangian relaxation (bisection on
 * the multiplier) and a greedy fill of the bytes left over.
 *   err        [n_layers x n_experts x 3] host: held-out output error of the
 *              expert in TERN160, Q2_0, Q3 (>= 0)
 *   tokens     [n_layers x n_experts] host: held-out tokens routed to it
 *   energy     [n_layers] host: the layer's routed output energy (> 0)
 *   fmt_bytes  [3] host: bytes of one expert in TERN160, Q2_0, Q3 (increasing)
 *   cost = err / energy, doubled on the first edge_first and last edge_last
 *   layers; at most floor(max_tern_frac * n_experts) ternary experts per
 *   layer; experts with fewer than min_tokens tokens stay Q2_0 (the pages:
 *   0.5, 8, 2, 3).  Per expert the multiplier picks the least cost + lam *
 *   bytes (equal values: Q2_0, then ternary, then Q3); over the cap, the
 *   ternary experts whose best other value is closest go back (equal: the
 *   higher id first); the greedy fill takes upgrades to a larger, cheaper
 *   format by cost saved per extra byte (equal: lower expert, lower format).
 *   fmt_out    [n_layers x n_experts] host, out: moe_format tags
 *   cost_out, bytes_out: the allocation's total cost and bytes (or NULL)
 * Host only, deterministic.  MOE_EINVAL on a null pointer, a size <= 0, a
 * negative or non-finite error, a non-positive energy or unordered sizes. */
int moe_allocate_formats(int32_t n_layers, int32_t n_experts, const double* err, const int32_t* tokens,
                         const double* energy, const uint64_t* fmt_bytes, double max_tern_frac,
                         int32_t min_tokens, int32_t edge_first, int32_t edge_last, uint8_t* fmt_out,
                         double* cost_out, uint64_t* bytes_out);

/* ------------------------------------------------------------------------ */
/* Device layer.                                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t hidden;     /* H: 5120 for the real layer, 512 for the tiny one       */
  int32_t inter;      /* I: 2304 / 256                                          */
  int32_t n_experts;  /* E routed experts: 384 / 16                             */
  int32_t top_k;      /* k: 6 / 2                                               */
  uint32_t flags;     /* MOE_ACT_* bits; 0 for none                             */
} moe_dims;

/* moe_dims.flags: on the many-row path (rows > MOE_MAX_DECODE_ROWS), MXFP4
 * experts run on the scaled matrix cores with the activations quantised to
 * MXFP8 (as moe_quant_mxfp8).  Without it, and for every other format, the
 * many-row path runs the decode tiles on unquantised activations.  Ignored
 * by the decode path.  Any other bit: MOE_EINVAL. */
#define MOE_ACT_MXFP8 1u

/* One expert: its format and the byte offsets of its three packed matrices
 * inside the `weights` buffer: gate [I x H], up [I x H], down [H x I].  Each
 * offset must be a multiple of 16. */
typedef struct {
  uint32_t fmt;
  uint32_t reserved;  /* must be 0 */
  uint64_t gate, up, down;
} moe_expert_ref;

/* Supported shapes: (hidden, inter) = (5120, 2304) or (512, 256);
 * 1 <= top_k <= MOE_MAX_TOP_K, top_k <= n_experts <= 512; on the decode path
 * rows <= MOE_MAX_DECODE_ROWS and rows * top_k <= 64, on the many-row path
 * rows <= MOE_MAX_PREFILL_ROWS.  Returns 0 for unsupported dims or flags.
 * Every workspace begins with the same area, sized by the dims alone, that
 * holds the fused decode launch's tagged words; every other use of the
 * workspace lies past it, so one workspace may serve calls of any kind and
 * any row count in turn. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t rows);

/* Host check of an expert table (host memory) against the dims and the size
 * of the weights buffer: format tags, reserved fields, alignment, and that
 * every matrix lies inside [0, weights_bytes).  The device entry points read
 * the table from device memory and trust it; validate it once with this call
 * before uploading. */
int moe_check_experts(const moe_dims* dims, const moe_expert_ref* table, int32_t count,
                      size_t weights_bytes);

/* Router GEMV + selection.
 *   x_bf16   [rows x H] bf16, device
 *   w_router [E x H] fp32, device
 *   sel_bias [E] fp32, device, or NULL (no bias).  Changes selection only.
 *   idx      [rows x top_k] int32, device, out: selected ids, key desc / id asc
 *   wts      [rows x top_k] fp32, device, out: mixing weights (unbiased softmax
 *            renormalised over the selection)
 *   ws       device workspace of ws_bytes >= moe_workspace_bytes(dims, rows).
 *            Zero-fill it once before its first use by any entry point;
 *            every call leaves it valid for the next, for any row count.
 *            One workspace must not serve two calls that can overlap.
 * rows == 0 returns MOE_OK and launches nothing. */
int moe_route(const moe_dims* dims, const void* x_bf16, int32_t rows, const float* w_router,
              const float* sel_bias, int32_t* idx, float* wts, void* ws, size_t ws_bytes,
              void* stream);

/* MXFP8 quantisation of activations (the prefill path's first step, exposed
 * on its own): x [rows x k] bf16 (device) -> codes [rows x k] e4m3 and
 * scales [rows x k/32] e8m0 (device).  Per 32 consecutive elements of a row:
 * E = floor(log2 amax) - 8 + 127 clamped to [0, 254] (E = 0 for an all-zero
 * block); element = e4m3 (OCP, finite-only variant) nearest to x / 2^(E-127),
 * ties to the even significand, magnitudes at or above 448 saturating to 448.
 * k must be a positive multiple of 32. */
int moe_quant_mxfp8(const void* x_bf16, int32_t rows, int32_t k, void* codes, void* scales,
                    void* stream);

/* Grouped expert FFN for a given routing.
 *   idx, wts   [rows x top_k], device, as produced by moe_route (any order of
 *              the k entries of a row is accepted; each row's ids must be
 *              distinct and < n_experts)
 *   weights    device buffer holding every packed matrix
 *   experts    [n_experts] moe_expert_ref, device
 *   shared     [1] moe_expert_ref, device, or NULL (no shared expert)
 *   y          [rows x H] fp32, device, out (overwritten)
 * Deterministic: the same inputs give bitwise the same y.
 * An idx entry of -1 is a pair the caller computes elsewhere (an expert the
 * CPU serves, moe_cache_plan): it adds nothing to y and its expert entry is
 * not read.  Any other id outside [0, n_experts) makes its row of y NaN.
 * rows <= MOE_MAX_DECODE_ROWS: the decode path, any formats.
 * MOE_MAX_DECODE_ROWS < rows <= MOE_MAX_PREFILL_ROWS: the many-row path
 * ("[Strata] DeepSeek V4.1 Flash on a single 4090", section 4: prefill runs
 * the experts as matrix products).  Pairs (row, expert) are grouped by
 * expert in ascending (expert, pair) order, then:
 *   - with MOE_ACT_MXFP8 in dims->flags, an MXFP4 expert runs on the scaled
 *     matrix cores in chunks of 64 pairs: x quantised to MXFP8 (as
 *     moe_quant_mxfp8) for gate/up, h = silu(W_gate x) * (W_up x) rounded to
 *     f16 for down (f16 x MXFP4);
 *   - every other expert (any format, MXFP4 too without the flag) and the
 *     shared expert run the decode tiles on unquantised activations, 8 pairs
 *     of one expert per work entry, h in fp32.
 * y[r] = the row's expert outputs, weighted, in ascending expert id, then the
 * shared expert.  The workspace is moe_workspace_bytes(dims, rows) (about
 * rows * top_k * (hidden * 4 + inter * 6) bytes). */
int moe_expert_ffn(const moe_dims* dims, const void* x_bf16, int32_t rows, const int32_t* idx,
                   const float* wts, const void* weights, const moe_expert_ref* experts,
                   const moe_expert_ref* shared, float* y, void* ws, size_t ws_bytes,
                   void* stream);

/* The whole layer, same results as moe_route followed by moe_expert_ffn
 * (rows <= MOE_MAX_DECODE_ROWS), in one launch whose workgroups hand logits,
 * selections, h and partial outputs to each other through words tagged with
 * the call's tag: router, selection, then workers over one list of items
 * (the shared expert's gate/up tiles, the routed gate/up items, then the
 * down items), then a fixed-order combine.  The shared expert streams while
 * the selection is made and down weights stream while h is still being
 * computed.  idx and wts are outputs as in moe_route (NULL: not written).
 * The launch holds at most one residency round of workers (the occupancy the
 * runtime reports for the kernel, times the compute units), since a down item
 * may wait on a gate/up item of any worker.  The launch assumes that its
 * workgroups start in id order and that, once the router and selection
 * workgroups are done, every worker is resident; a kernel on another stream
 * that holds compute units can delay that.  Every wait on another
 * workgroup's words is bounded (moe_set_spin_limit): a wait that gives up
 * poisons what it feeds with NaN (the routing weights, h, the partial
 * outputs, y) and records the call in the workspace's error word, so such a
 * call's y is NaN wherever the failure reached, and moe_workspace_status
 * reports it.  Status MOE_OK means the launch was made, not that every wait
 * succeeded. */
int moe_layer(const moe_dims* dims, const void* x_bf16, int32_t rows, const float* w_router,
              const float* sel_bias, const void* weights, const moe_expert_ref* experts,
              const moe_expert_ref* shared, int32_t* idx, float* wts, float* y, void* ws,
              size_t ws_bytes, void* stream);

/* moe_layer for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace argument: the fused launch's hand-off words live in a fixed
 * device array of the library, 4.5 MiB per GPU (enough for rows <=
 * MOE_MAX_DECODE_ROWS, top_k <= MOE_MAX_TOP_K and up to 512 experts at hidden
 * 5120 / inter 2304), which each GPU the library runs on holds until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); its first call on a device looks up that device's array
 * once.  Arguments, results and errors as moe_layer (idx / wts may be NULL);
 * MOE_EWORKSPACE if the dims would need more than the array holds.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * words: calls queued one after another (one stream) are correct, since each
 * call's words carry its own tag; calls that overlap on one GPU (on
 * different streams or from different threads without ordering) race and
 * give wrong results.  A hand-off wait that gives up shows as NaN in y (the
 * array's error word is not queryable). */
int moe_layer_noalloc(const moe_dims* dims, const void* x_bf16, int32_t rows, const float* w_router,
                      const float* sel_bias, const void* weights, const moe_expert_ref* experts,
                      const moe_expert_ref* shared, int32_t* idx, float* wts, float* y, void* stream);

/* moe_layer with timing: `events` holds n_events >= 2 hipEvent_t handles
 * created by the caller, recorded on the stream before and after the launch. */
int moe_layer_profiled(const moe_dims* dims, const void* x_bf16, int32_t rows,
                       const float* w_router, const float* sel_bias, const void* weights,
                       const moe_expert_ref* experts, const moe_expert_ref* shared,
                       int32_t* idx, float* wts, float* y, void* ws, size_t ws_bytes,
                       void* stream, void* const* events, int32_t n_events);

/* ------------------------------------------------------------------------ */
/* Stack decode.                                                             */
/* ------------------------------------------------------------------------ */

/* The device buffers of one layer, as passed to moe_layer. */
typedef struct {
  const float* w_router;          /* [E x H] fp32                          */
  const float* sel_bias;          /* [E] fp32, or NULL                     */
  const void* weights;            /* packed matrices                       */
  const moe_expert_ref* experts;  /* [E] device                            */
  const moe_expert_ref* shared;   /* [1] device, or NULL                   */
} moe_layer_weights;

/* Decode rows through a stack of layers, each layer's output (plus noise)
 * feeding the next, as in the stacked-layer decode workloads:
 *     y_l     = moe_layer(layer l, x_l)
 *     v       = y_l + noise_l          (one fp32 addition per element)
 *     x_{l+1} = bf16(v / 2^s)          (round to nearest even), per row:
 *               s = floor(log2 max|v|) - 1 when the row's largest |v| is 4
 *               or more (it then lies in [2, 4)), else 0; s = 0 for a row
 *               holding a NaN or an infinity.
 * The power of two bounds each layer's input as a trained stack's
 * normalisation would (synthetic SwiGLU experts have a gain above one and a
 * quadratic response: unbounded, x overflows bf16 within a few layers), and
 * keeps the step exact and independent of summation order.
 *   layers   host array of n_layers layer descriptions (device pointers)
 *   x_all    [(n_layers + 1) x rows x H] bf16, device: the caller fills
 *            x_all[0]; the call writes x_all[1 .. n_layers]
 *   noise    [n_layers x rows x H] fp32, device, or NULL (no noise)
 *   y_all    [n_layers x rows x H] fp32, device, out: every layer's y
 *   idx_all, wts_all  [n_layers x rows x top_k], device, or NULL
 *   ws       as for moe_layer (one workspace serves every layer)
 * One launch per layer on `stream`, no host synchronisation: the layer's
 * combine workgroups exchange their shares of each row's maximum through
 * tagged words and write x_{l+1}.  Every layer has the shape in dims.
 * Returns the first failing layer's status. */
int moe_stack_decode(const moe_dims* dims, int32_t n_layers, const moe_layer_weights* layers,
                     int32_t rows, void* x_all, const float* noise, float* y_all,
                     int32_t* idx_all, float* wts_all, void* ws, size_t ws_bytes, void* stream);

/* Whether a hand-off wait of any fused call (moe_layer, moe_layer_profiled,
 * moe_stack_decode) on this workspace gave up since the workspace was
 * zero-filled or last queried.  Synchronises `stream` (the host blocks until
 * every call queued on it has finished), reads the workspace's error word and
 * clears it.  Returns MOE_OK, MOE_ETIMEOUT (some call's y holds NaN from the
 * failure), MOE_EINVAL (null ws or ws_bytes below 16) or MOE_EDEVICE. */
int moe_workspace_status(void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Test aid: the fused launch's hand-off waits.                              */
/* ------------------------------------------------------------------------ */

/* Every wait of one moe_layer / moe_stack_decode launch on words published
 * by another workgroup of the same launch gives up after `polls` polls
 * (default 65536, tens of ms): the launch then still drains, the failure is
 * recorded in the workspace's error word and poisons the data it feeds with
 * NaN (a worker whose wait for the selection gave up computes with expert 0,
 * weight NaN, instead of reading stale entries).  0 makes every wait give up
 * at once, which lets a test reach that path without a hung producer.
 * Process-wide, read at each launch.  Returns the previous value, or
 * MOE_EINVAL for polls < 0. */
int32_t moe_set_spin_limit(int32_t polls);

/* ------------------------------------------------------------------------ */
/* Measurement aid (not a step of the method).                               */
/* ------------------------------------------------------------------------ */

/* The streaming-read ceiling against which the layer's HBM rate is also
 * reported ("DeepSeek-V4.1-Flash served three ways on 4xL20", section 6: the
 * bandwidth a workload sees falls short of the micro-benchmark figure, so a
 * rate is compared with what the device reaches on a plain stream).  Reads the first floor(bytes / 16) 16-byte chunks of `buf` with
 * one 16-byte load per lane and `unroll` loads in flight per lane per
 * iteration, grid-striding over `grid` workgroups of 256 threads, and
 * writes one xor checksum per thread to `sink` so that no load is dropped.
 *   buf      device, 16-byte aligned, read-only
 *   sink     device, grid * 256 uint32, out (contents are only a checksum)
 *   grid     1 .. 65536 workgroups;  unroll  1, 2, 4 or 8
 * Asynchronous on `stream`; time it with events.  MOE_EINVAL on a null or
 * misaligned pointer or an argument out of range, MOE_EDEVICE if the launch
 * fails. */
int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, int32_t unroll,
                    void* stream);

/* ------------------------------------------------------------------------
 * Stacks larger than HBM.
 * "DeepSeek-V4.1-Flash served three ways on 4xL20", section 3C: one engine
 * keeps every expert in a pinned host store and only a slot cache on the
 * device; a layer's missing experts are either copied to the device or
 * computed on the CPU, the number copied set by the ratio of the two
 * channels' measured bandwidths (section 5: f / (1 - f) = effective PCIe rate
 * / effective CPU rate; "Model task radar 2026-11-03: when the accelerator
 * flips", section 6: q* ~ m * B_P / B_H to first order).  "[Strata] DeepSeek V4.1 Flash on a single 4090",
 * section 5.2: a device LRU of experts in front of a pinned host arena.
 *
 * The calls below are host code; the caller moves the bytes (pinned host ->
 * device slots) and runs the device part with moe_route / moe_expert_ffn
 * (pairs the CPU serves marked -1) and moe_add_chain.
 * ------------------------------------------------------------------------ */
typedef struct moe_slot_cache moe_slot_cache;

/* A cache of n_slots device expert slots for a stack of n_layers x
 * n_experts routed experts, all slots empty.  Host memory only (the slots'
 * device memory is the caller's).  *out is NULL on error (MOE_EINVAL). */
int moe_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, moe_slot_cache** out);
void moe_cache_destroy(moe_slot_cache* cache);

/* One layer step: which of the experts that idx selects are in a slot (hits),
 * which are copied into a slot now, and which the CPU computes.
 *   idx         host [rows x top_k], every id in [0, n_experts)
 *   copy_share  0 .. 1: the share f of the step's m misses to copy;
 *               moe_copy_share gives it from measured bandwidths.  The count
 *               copied is the whole number q next to m f (below or above)
 *               for which max(q (1 - f), (m - q) f) -- the slower of the two
 *               channels, in units of an expert's time -- is smaller, the
 *               larger q on a tie
 * Misses are copied in order of most pairs, then lower id.  A copy takes a
 * free slot (lowest index), else the least recently used slot (lowest index
 * on ties) that this step's experts do not use; when none is left the miss
 * goes to the CPU.  Outputs (host arrays the caller provides):
 *   slot_of     [n_experts]  the slot of each expert of `layer` after the
 *               step (-1: not resident); the slots of this step's device
 *               experts hold them once the copies below are done
 *   copy_expert, copy_slot [rows x top_k]  the copies, *n_copy of them
 *   cpu_expert  [rows x top_k]  the experts the CPU serves, ascending, *n_cpu
 *   idx_gpu     [rows x top_k]  idx with the CPU's experts replaced by -1
 * MOE_EINVAL on a null pointer, an id out of range or a share outside [0, 1]
 * (the cache is then unchanged). */
int moe_cache_plan(moe_slot_cache* cache, int32_t layer, int32_t rows, int32_t top_k, const int32_t* idx,
                   double copy_share, int32_t* slot_of, int32_t* copy_expert, int32_t* copy_slot,
                   int32_t* n_copy, int32_t* cpu_expert, int32_t* n_cpu, int32_t* idx_gpu);

/* The share of misses to copy when copies run at pcie_bytes_per_s and the
 * CPU computes experts at cpu_bytes_per_s (packed bytes per second): the
 * share at which both channels finish together, f = B_P / (B_P + B_C), i.e.
 * f / (1 - f) = B_P / B_C.  0 if both rates are 0 or one is negative. */
double moe_copy_share(double pcie_bytes_per_s, double cpu_bytes_per_s);

/* One expert's FFN on the host CPU for the rows that chose it, accumulated
 * into a host y:  y[row_ids[j]] += row_w[j] * W_down (silu(W_gate x) * (W_up x))
 * with x = x_bf16[row_ids[j]].  gate / up / down are the expert's packed
 * matrices in host memory (format fmt, [inter x hidden] / [hidden x inter]);
 * decoding is exact and every sum is fp64, rounded to fp32 once when added.
 * n_threads host threads (0: all).  MOE_ECODE if a code is invalid,
 * MOE_EFORMAT / MOE_ESHAPE / MOE_EINVAL as moe_unpack. */
int moe_cpu_expert_ffn(const moe_dims* dims, int32_t fmt, const void* gate, const void* up, const void* down,
                       const void* x_bf16, int32_t n_rows, const int32_t* row_ids, const float* row_w, float* y,
                       int32_t n_threads);

/* The end of a layer step computed in parts, on the device, asynchronous on
 * `stream`, one workgroup per row:  y += add (add NULL: nothing added); then,
 * when x_next is not NULL, x_next = the next layer's input from y + noise
 * (noise NULL: 0) exactly as moe_stack_decode chains layers.  y, add, noise:
 * [rows x hidden] fp32; x_next [rows x hidden] bf16; all on the device. */
int moe_add_chain(float* y, const float* add, const float* noise, void* x_next, int32_t rows, int32_t hidden,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BIT_MOE_H */
