// gfx950 kernels of the routed-MoE expert FFN and the C-ABI entry points
// that launch them.
//
// One layer call runs three kernels on the caller's stream:
//   A  router GEMV (fp64 sums) over every expert, one workgroup per expert;
//      the last workgroup to finish selects the top-k per row.  In moe_layer
//      the shared expert's gate/up tiles ride in the same launch, so their
//      weights stream while the router runs.
//   B  grouped gate/up + SwiGLU: one workgroup per (distinct selected expert,
//      tile of intermediate channels); h = silu(W_gate x) * (W_up x) in fp32.
//   C  grouped down projection: one workgroup per (expert, tile of outputs)
//      writes w * (W_down h) for each row it serves; the last workgroup of an
//      output tile sums the partials in ascending expert order (no atomics
//      on data, so results are bitwise reproducible).
//
// The method: "DeepSeek-V4.1-Flash served three ways on 4xL20"
// (lcz.me/topic/2356) section 1 (layer shape, top-6 of 384 plus one shared
// expert) and section 2 (cost = expert bytes streamed); "[Strata] DeepSeek V4.1
// Flash on a single 4090" (lcz.me/post/25274) section 5.3 (selection-only bias,
// mixing weights from the unbiased router) and section 5.1 (per-expert formats).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <type_traits>

#include "../../include/moe.h"
#include "dev_common.h"
#include "formats_dev.h"
#include "host_common.h"

namespace moe {
namespace dev {

constexpr int kThreads = 256;
#ifndef MOE_WAVES_PER_EU
#define MOE_WAVES_PER_EU 2  // occupancy floor: 2 waves per SIMD (<= 256 VGPRs)
#endif
constexpr int kMaxRows = MOE_MAX_DECODE_ROWS;  // rows per call on the decode path
constexpr int kMaxK = MOE_MAX_TOP_K;
constexpr int kNTB = 2;                        // token rows staged in LDS at once
constexpr int kMaxTiles = 1024;                // output-tile counters in the workspace

struct Args {
  const uint16_t* x;      // [R x H] bf16
  const float* w_router;  // [E x H]
  const float* bias;      // [E] or null
  const uint8_t* weights;
  const moe_expert_ref* experts;  // [E]
  const moe_expert_ref* shared;   // [1] or null
  int32_t* idx;                   // [R x k]
  float* wts;                     // [R x k]
  float* y;                       // [R x H]
  double* logits;                 // [R x E]
  uint32_t* counters;             // [0]: router arrivals; [1 + t]: output tile t
  float* h;                       // [(R*k + R) x I]
  float* part;                    // [(R*k + R) x H]
  int R, k, E;
  int shared_in_route;            // 1: kernel A carries the shared gate/up tiles
};

// ---------------------------------------------------------------------------
// shape-dependent constants
// ---------------------------------------------------------------------------
constexpr int lpr_for(int k) { return k >= 4096 ? 16 : (k >= 512 ? 8 : 4); }

template <class F>
constexpr int phase_units() {
  return sizeof(typename F::Raw) > 28 ? 2 : 5;  // bound the registers a phase holds  // bound the registers a phase holds
}

template <int H, int I>
struct Shape {
  static constexpr int kH = H, kI = I;
  static constexpr int LPR_GU = lpr_for(H), LPR_DN = lpr_for(I);
  static constexpr int NPG_GU = 1, NPG_DN = 2;  // channels per lane group
  static constexpr int TN_GU = kThreads / LPR_GU * NPG_GU;
  static constexpr int TN_DN = kThreads / LPR_DN * NPG_DN;
  static constexpr int TILES_GU = (I + TN_GU - 1) / TN_GU;
  static constexpr int TILES_DN = (H + TN_DN - 1) / TN_DN;
  template <class F>
  static constexpr int rec_row_bytes(int k) { return F::units(k) * F::XREC; }
  static constexpr int max_rec_row(int k) {
    int m = rec_row_bytes<FmtQ2>(k);
    m = m > rec_row_bytes<FmtQ8>(k) ? m : rec_row_bytes<FmtQ8>(k);
    m = m > rec_row_bytes<FmtMXFP4>(k) ? m : rec_row_bytes<FmtMXFP4>(k);
    m = m > rec_row_bytes<FmtTern>(k) ? m : rec_row_bytes<FmtTern>(k);
    m = m > rec_row_bytes<FmtQ3>(k) ? m : rec_row_bytes<FmtQ3>(k);
    return m;
  }
  // LDS: token-row records, then the ternary table, then small per-row data
  static constexpr int LDS_REC = kNTB * (max_rec_row(H) > max_rec_row(I) ? max_rec_row(H) : max_rec_row(I));
  static constexpr int LDS_TABLE = 256 * 4;
  static constexpr int LDS_BYTES = LDS_REC + LDS_TABLE;
};

// ---------------------------------------------------------------------------
// slot resolution: which expert a workgroup serves and for which rows
// ---------------------------------------------------------------------------
struct Slot {
  int expert;               // routed id, or -1 for the shared expert
  int nt;                   // rows served
  int n_active;             // distinct routed experts in this call
  int row[kMaxRows];        // token row r
  int pair[kMaxRows];       // h / partial row: r*k + kk (routed) or R*k + r (shared)
  float w[kMaxRows];        // mixing weight (1 for the shared expert)
};

// Routed slot u = the u-th smallest distinct expert id in idx.  Run by one
// full wave; the result goes to `out` in LDS.
__device__ void resolve_slot(const Args& a, int slot, Slot* out) {
  const int lane = threadIdx.x;  // wave 0
  const int n = a.R * a.k;
  const int v = lane < n ? a.idx[lane] : 0x7fffffff;
  bool first = lane < n;
  int rank = 0;
  for (int m = 0; m < n; ++m) {
    const int vm = __shfl(v, m, 64);
    if (m < lane && vm == v) first = false;
  }
  const uint64_t firsts = __ballot(first);
  for (int m = 0; m < n; ++m) {
    const int vm = __shfl(v, m, 64);
    if (((firsts >> m) & 1ull) && vm < v) ++rank;
  }
  const int n_active = __popcll(firsts);
  int expert = -1;
  if (slot < n_active) {
    const uint64_t hit = __ballot(first && rank == slot);
    expert = __shfl(v, static_cast<int>(__ffsll(static_cast<long long>(hit)) - 1), 64);
  }
  const uint64_t mine = __ballot(lane < n && v == expert);
  if (lane == 0) {
    out->expert = slot < n_active ? expert : -2;
    out->n_active = n_active;
    int t = 0;
    uint64_t m = slot < n_active ? mine : 0ull;
    while (m && t < kMaxRows) {  // distinct ids per row bound this by R
      const int l = __ffsll(static_cast<long long>(m)) - 1;
      m &= m - 1;
      out->row[t] = l / a.k;
      out->pair[t] = l;
      out->w[t] = a.wts[l];
      ++t;
    }
    out->nt = t;
  }
}

__device__ void shared_slot(const Args& a, Slot* out, int n_active) {
  if (threadIdx.x == 0) {
    out->expert = -1;
    out->nt = a.R;
    out->n_active = n_active;
    for (int r = 0; r < a.R; ++r) {
      out->row[r] = r;
      out->pair[r] = a.R * a.k + r;
      out->w[r] = 1.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// activation staging: x' records of up to kNTB token rows in LDS
// ---------------------------------------------------------------------------
// SUBV values starting at element e0 (a multiple of 4), zero at and beyond KR
template <int SUBV, int KR, bool BF16>
__device__ __forceinline__ void load_vals(const void* src, int e0, float (&v)[SUBV]) {
#pragma unroll
  for (int c = 0; c < SUBV / 4; ++c) {
    const int e = e0 + 4 * c;
    if (e < KR) {
      if constexpr (BF16) {
        const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + e);
        v[4 * c + 0] = bf16_bits_to_f32(q.x & 0xFFFFu);
        v[4 * c + 1] = bf16_bits_to_f32(q.x >> 16);
        v[4 * c + 2] = bf16_bits_to_f32(q.y & 0xFFFFu);
        v[4 * c + 3] = bf16_bits_to_f32(q.y >> 16);
      } else {
        const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + e);
        v[4 * c + 0] = q.x;
        v[4 * c + 1] = q.y;
        v[4 * c + 2] = q.z;
        v[4 * c + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * c + i] = 0.0f;
    }
  }
}

// Builds records for `nb` rows; rows[t] points at the source row.  sigma is
// a power of two chosen from the row's largest |value| so every record value
// stays inside the f16 range; 1/sigma goes to inv_sigma[t].
template <class F, int KR, bool BF16>
__device__ void stage_rows(const void* const* rows, int nb, uint8_t* rec, float* inv_sigma,
                           float* red) {
  constexpr int KP = F::units(KR) * F::UNIT;  // padded length
  constexpr int NBU = F::units(KR);
  constexpr int RSTRIDE = NBU * F::XREC;
  constexpr int PER = BF16 ? 8 : 4;
  (void)KP;
  // 1) largest magnitude per row (as fp32 bit patterns, monotone for |v|)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < kNTB; ++t) {
    if (t < nb) {
      uint32_t m = 0;
      for (int c = threadIdx.x; c < KR / PER; c += blockDim.x) {
        const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(rows[t]) +
                                                        static_cast<size_t>(c) * 16);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (BF16) {
            const uint32_t a = (w[i] & 0x7FFFu) << 16, b = (w[i] >> 16 & 0x7FFFu) << 16;
            m = m > a ? m : a;
            m = m > b ? m : b;
          } else {
            const uint32_t a = w[i] & 0x7FFFFFFFu;
            m = m > a ? m : a;
          }
        }
      }
      m = wave_max_u32(m);
      if (lane == 0) reinterpret_cast<uint32_t*>(red)[wave * kNTB + t] = m;
    }
  }
  __syncthreads();
  if (threadIdx.x < nb) {
    uint32_t m = 0;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) {
      const uint32_t v = reinterpret_cast<uint32_t*>(red)[w * kNTB + threadIdx.x];
      m = m > v ? m : v;
    }
    // exponent of the largest magnitude; 2^(14 - PSHIFT - e) keeps |x'| < 2^15
    const int e = m ? static_cast<int>(m >> 23) - 127 : 0;
    const int s = 14 - F::PSHIFT - e;
    red[64 + threadIdx.x] = __builtin_ldexpf(1.0f, s);
    inv_sigma[threadIdx.x] = __builtin_ldexpf(1.0f, -s);
  }
  __syncthreads();
  // 2) one record sub-unit per (row, unit, sub) work item
  constexpr int PER_ROW = NBU * F::SUBS;
  for (int item = threadIdx.x; item < nb * PER_ROW; item += blockDim.x) {
    const int t = item / PER_ROW, rem = item - t * PER_ROW;
    const int u = rem / F::SUBS, sub = rem - u * F::SUBS;
    float v[F::SUBV];
    load_vals<F::SUBV, KR, BF16>(rows[t], u * F::UNIT + sub * F::SUBV, v);
    const float sg = red[64 + t];
#pragma unroll
    for (int i = 0; i < F::SUBV; ++i) v[i] *= sg;
    F::prep_sub(v, sub, rec + t * RSTRIDE + u * F::XREC);
  }
}

// ---------------------------------------------------------------------------
// one tile of one matrix pair (gate/up) or matrix (down)
// ---------------------------------------------------------------------------
template <class F, int K, int LPR, int RT, int NT>
__device__ __forceinline__ void dot_units(const typename F::Raw (&raw)[RT], const uint8_t* rec,
                                          int nt, float (&acc)[RT][NT], const uint32_t* table,
                                          int b) {
  constexpr int RSTRIDE = F::units(K) * F::XREC;
  if constexpr (std::is_same_v<F, FmtTern>)
    FmtTern::template dot<RT, NT>(raw, rec + b * F::XREC, RSTRIDE, nt, acc, table);
  else
    F::template dot<RT, NT>(raw, rec + b * F::XREC, RSTRIDE, nt, acc);
}

// Streams the lane's units of RT matrix rows and accumulates against the
// staged records.  mats[r] / rows[r] give matrix base and row for each of
// the RT rows; valid == false skips the loads (tail tiles).
template <class F, int K, int LPR, int RT>
__device__ __forceinline__ void stream_rows(const uint8_t* const (&mats)[RT], const int (&rows)[RT],
                                            int nrows, bool valid, const uint8_t* rec, int nt,
                                            float (&acc)[RT][kNTB], const uint32_t* table) {
  constexpr int NBU = F::units(K);
  constexpr int UPL = (NBU + LPR - 1) / LPR;
  constexpr int G = phase_units<F>() < UPL ? phase_units<F>() : UPL;
  const int c = threadIdx.x % LPR;

#pragma unroll
  for (int j0 = 0; j0 < UPL; j0 += G) {
    typename F::Raw raw[G][RT];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int b = c + (j0 + g) * LPR;
      if (valid && j0 + g < UPL && (NBU % LPR == 0 || b < NBU))
#pragma unroll
        for (int r = 0; r < RT; ++r) F::load(raw[g][r], mats[r], nrows, NBU, rows[r], b);
    }
    // every load of the phase is in flight before the first decode; each
    // unit's LDS reads and dot products stay between two scheduling fences
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int b = c + (j0 + g) * LPR;
      if (valid && j0 + g < UPL && (NBU % LPR == 0 || b < NBU))
        dot_units<F, K, LPR, RT, kNTB>(raw[g], rec, nt, acc, table, b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// gate/up tile: channels [tile*TN, tile*TN + TN) of the expert's I
template <class S, class F>
__device__ void gateup_tile(const Args& a, const moe_expert_ref& ref, const Slot& sl, int tile,
                            uint8_t* lds) {
  constexpr int H = S::kH, I = S::kI, LPR = S::LPR_GU;
  uint8_t* rec = lds;
  uint32_t* table = reinterpret_cast<uint32_t*>(lds + S::LDS_REC);
  __shared__ float inv_sigma[kNTB];
  __shared__ float red[128];
  __shared__ const void* srcs[kNTB];
  if constexpr (std::is_same_v<F, FmtTern>)
    for (int i = threadIdx.x; i < 256; i += blockDim.x) table[i] = FmtTern::table_entry(i);
  const int rg = threadIdx.x / LPR, c = threadIdx.x % LPR;
  const int n = tile * S::TN_GU + rg;
  const bool valid = n < I;
  const uint8_t* const mats[2] = {a.weights + ref.gate, a.weights + ref.up};
  const int rows[2] = {n, n};
  for (int t0 = 0; t0 < sl.nt; t0 += kNTB) {
    const int nb = sl.nt - t0 < kNTB ? sl.nt - t0 : kNTB;
    __syncthreads();
    if (threadIdx.x < nb) srcs[threadIdx.x] = a.x + static_cast<size_t>(sl.row[t0 + threadIdx.x]) * H;
    __syncthreads();
    stage_rows<F, H, true>(srcs, nb, rec, inv_sigma, red);
    __syncthreads();
    float acc[2][kNTB] = {};
    stream_rows<F, H, LPR, 2>(mats, rows, I, valid, rec, nb, acc, table);
#pragma unroll
    for (int t = 0; t < kNTB; ++t) {
      acc[0][t] = group_sum<LPR>(acc[0][t]);
      acc[1][t] = group_sum<LPR>(acc[1][t]);
    }
    if (valid && c == 0) {
#pragma unroll
      for (int t = 0; t < kNTB; ++t) {
        if (t < nb) {
          const float g = acc[0][t] * inv_sigma[t], v = acc[1][t] * inv_sigma[t];
          a.h[static_cast<size_t>(sl.pair[t0 + t]) * I + n] = g / (1.0f + expf(-g)) * v;
        }
      }
    }
  }
}

// down tile: outputs [tile*TN, tile*TN + TN) of H for every row of the slot
template <class S, class F>
__device__ void down_tile(const Args& a, const moe_expert_ref& ref, const Slot& sl, int tile,
                          uint8_t* lds) {
  constexpr int H = S::kH, I = S::kI, LPR = S::LPR_DN, NPG = S::NPG_DN;
  uint8_t* rec = lds;
  uint32_t* table = reinterpret_cast<uint32_t*>(lds + S::LDS_REC);
  __shared__ float inv_sigma[kNTB];
  __shared__ float red[128];
  __shared__ const void* srcs[kNTB];
  if constexpr (std::is_same_v<F, FmtTern>)
    for (int i = threadIdx.x; i < 256; i += blockDim.x) table[i] = FmtTern::table_entry(i);
  const int rg = threadIdx.x / LPR, c = threadIdx.x % LPR;
  const int n0 = tile * S::TN_DN + rg * NPG;
  const uint8_t* const md = a.weights + ref.down;
  const uint8_t* const mats[NPG] = {md, md};
  const int rows[NPG] = {n0, n0 + 1};
  const bool valid = n0 + NPG <= H;
  for (int t0 = 0; t0 < sl.nt; t0 += kNTB) {
    const int nb = sl.nt - t0 < kNTB ? sl.nt - t0 : kNTB;
    __syncthreads();
    if (threadIdx.x < nb) srcs[threadIdx.x] = a.h + static_cast<size_t>(sl.pair[t0 + threadIdx.x]) * I;
    __syncthreads();
    stage_rows<F, I, false>(srcs, nb, rec, inv_sigma, red);
    __syncthreads();
    float acc[NPG][kNTB] = {};
    stream_rows<F, I, LPR, NPG>(mats, rows, H, valid, rec, nb, acc, table);
#pragma unroll
    for (int q = 0; q < NPG; ++q)
#pragma unroll
      for (int t = 0; t < kNTB; ++t) acc[q][t] = group_sum<LPR>(acc[q][t]);
    if (valid && c == 0) {
#pragma unroll
      for (int t = 0; t < kNTB; ++t) {
        if (t < nb) {
          const float sc = inv_sigma[t] * sl.w[t0 + t];
#pragma unroll
          for (int q = 0; q < NPG; ++q)
            a.part[static_cast<size_t>(sl.pair[t0 + t]) * H + n0 + q] = acc[q][t] * sc;
        }
      }
    }
  }
}

template <class S, bool GATEUP>
__device__ void run_slot(const Args& a, const moe_expert_ref& ref, const Slot& sl, int tile,
                         uint8_t* lds) {
  switch (ref.fmt) {
    case MOE_FMT_Q2_0:
      if constexpr (GATEUP) gateup_tile<S, FmtQ2>(a, ref, sl, tile, lds); else down_tile<S, FmtQ2>(a, ref, sl, tile, lds);
      break;
    case MOE_FMT_Q8:
      if constexpr (GATEUP) gateup_tile<S, FmtQ8>(a, ref, sl, tile, lds); else down_tile<S, FmtQ8>(a, ref, sl, tile, lds);
      break;
    case MOE_FMT_MXFP4:
      if constexpr (GATEUP) gateup_tile<S, FmtMXFP4>(a, ref, sl, tile, lds); else down_tile<S, FmtMXFP4>(a, ref, sl, tile, lds);
      break;
    case MOE_FMT_TERN160:
      if constexpr (GATEUP) gateup_tile<S, FmtTern>(a, ref, sl, tile, lds); else down_tile<S, FmtTern>(a, ref, sl, tile, lds);
      break;
    case MOE_FMT_Q3:
      if constexpr (GATEUP) gateup_tile<S, FmtQ3>(a, ref, sl, tile, lds); else down_tile<S, FmtQ3>(a, ref, sl, tile, lds);
      break;
    default:
      break;  // tables are checked on the host (moe_check_experts)
  }
}

// ---------------------------------------------------------------------------
// router GEMV + top-k
// ---------------------------------------------------------------------------
template <int H>
__device__ void router_wg(const Args& a, int e, double* red) {
  double acc[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.0;
  const float4* wr = reinterpret_cast<const float4*>(a.w_router + static_cast<size_t>(e) * H);
  for (int j = threadIdx.x; j < H / 4; j += blockDim.x) {
    const float4 w = wr[j];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      if (r < a.R) {
        const uint2 xb = *reinterpret_cast<const uint2*>(a.x + static_cast<size_t>(r) * H + 4 * j);
        double s = acc[r];
        s = fma(static_cast<double>(w.x), static_cast<double>(bf16_bits_to_f32(xb.x & 0xFFFFu)), s);
        s = fma(static_cast<double>(w.y), static_cast<double>(bf16_bits_to_f32(xb.x >> 16)), s);
        s = fma(static_cast<double>(w.z), static_cast<double>(bf16_bits_to_f32(xb.y & 0xFFFFu)), s);
        s = fma(static_cast<double>(w.w), static_cast<double>(bf16_bits_to_f32(xb.y >> 16)), s);
        acc[r] = s;
      }
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    if (r < a.R) {
      const double s = wave_sum_f64(acc[r]);
      if (lane == 0) red[r * 16 + wave] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x < a.R) {
    double s = 0.0;
    for (int w = 0; w < nw; ++w) s += red[threadIdx.x * 16 + w];
    a.logits[static_cast<size_t>(threadIdx.x) * a.E + e] = s;
  }
}

// Top-k of one row by key = logit + bias, ties to the lower id; weights are
// the softmax of the unbiased logits over the selection.  One wave per row.
__device__ void select_row(const Args& a, int r) {
  const int lane = threadIdx.x & 63;
  int sel[kMaxK];
  double keyv[kMaxK];
  for (int j = 0; j < a.k; ++j) {
    double best = -INFINITY;
    int bid = 0x7fffffff;
    for (int e = lane; e < a.E; e += 64) {
      bool taken = false;
      for (int q = 0; q < j; ++q) taken |= (sel[q] == e);
      if (taken) continue;
      double key = coherent_load_f64(a.logits + static_cast<size_t>(r) * a.E + e);
      if (a.bias) key += static_cast<double>(a.bias[e]);
      if (key > best || (key == best && e < bid)) {
        best = key;
        bid = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bid, o, 64);
      if (ob > best || (ob == best && oi < bid)) {
        best = ob;
        bid = oi;
      }
    }
    sel[j] = bid;
    keyv[j] = best;
  }
  (void)keyv;
  if (lane == 0) {
    double l[kMaxK], m = -INFINITY;
    for (int j = 0; j < a.k; ++j) {
      l[j] = coherent_load_f64(a.logits + static_cast<size_t>(r) * a.E + sel[j]);
      m = l[j] > m ? l[j] : m;
    }
    double s = 0.0;
    for (int j = 0; j < a.k; ++j) {
      l[j] = exp(l[j] - m);
      s += l[j];
    }
    for (int j = 0; j < a.k; ++j) {
      a.idx[r * a.k + j] = sel[j];
      a.wts[r * a.k + j] = static_cast<float>(l[j] / s);
    }
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_route(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ double red[kMaxRows * 16];
  __shared__ Slot sl;
  __shared__ int last;
  const int bid = blockIdx.x;
  if (bid >= a.E) {  // shared expert gate/up tiles streaming beside the router
    shared_slot(a, &sl, 0);
    __syncthreads();
    run_slot<S, true>(a, *a.shared, sl, bid - a.E, lds);
    return;
  }
  router_wg<S::kH>(a, bid, red);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = (atomicAdd(&a.counters[0], 1u) == static_cast<uint32_t>(a.E - 1));
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int r = threadIdx.x >> 6; r < a.R; r += blockDim.x >> 6) select_row(a, r);
  if (threadIdx.x == 0) __hip_atomic_store(&a.counters[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_gateup(Args a, int n_slots) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ Slot sl;
  const int slot = blockIdx.x % n_slots, tile = blockIdx.x / n_slots;
  const bool is_shared = a.shared && !a.shared_in_route && slot == n_slots - 1;
  if (is_shared) {
    shared_slot(a, &sl, 0);
  } else if (threadIdx.x < 64) {
    resolve_slot(a, slot, &sl);
  }
  __syncthreads();
  if (sl.expert == -2) return;
  const moe_expert_ref ref = is_shared ? *a.shared : a.experts[sl.expert];
  run_slot<S, true>(a, ref, sl, tile, lds);
}

template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_down(Args a, int n_slots) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ Slot sl;
  __shared__ int last;
  __shared__ int order[kMaxRows][kMaxK];
  const int slot = blockIdx.x % n_slots, tile = blockIdx.x / n_slots;
  const bool is_shared = a.shared && slot == n_slots - 1;
  // every workgroup needs the number of distinct experts: the arrival target
  if (threadIdx.x < 64) resolve_slot(a, is_shared ? 0 : slot, &sl);
  __syncthreads();
  if (is_shared) {
    const int n_active = sl.n_active;
    __syncthreads();
    shared_slot(a, &sl, n_active);
  }
  __syncthreads();
  if (sl.expert == -2) return;
  const moe_expert_ref ref = is_shared ? *a.shared : a.experts[sl.expert];
  run_slot<S, false>(a, ref, sl, tile, lds);

  // arrival: the last workgroup of this output tile combines the partials
  __threadfence();
  __syncthreads();
  const uint32_t target = static_cast<uint32_t>(sl.n_active + (a.shared ? 1 : 0));
  if (threadIdx.x == 0) last = (atomicAdd(&a.counters[1 + tile], 1u) == target - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  if (threadIdx.x < a.R) {  // row r's entries in ascending expert id
    const int r = threadIdx.x;
    int ids[kMaxK], ord[kMaxK];
    for (int j = 0; j < a.k; ++j) {
      ids[j] = a.idx[r * a.k + j];
      ord[j] = j;
    }
    for (int i = 1; i < a.k; ++i)
      for (int j = i; j > 0 && ids[ord[j]] < ids[ord[j - 1]]; --j) {
        const int tmp = ord[j];
        ord[j] = ord[j - 1];
        ord[j - 1] = tmp;
      }
    for (int j = 0; j < a.k; ++j) order[r][j] = ord[j];
  }
  __syncthreads();
  const int n_lo = tile * S::TN_DN;
  for (int i = threadIdx.x; i < a.R * S::TN_DN; i += blockDim.x) {
    const int r = i / S::TN_DN, n = n_lo + i % S::TN_DN;
    if (n >= S::kH) continue;
    float s = 0.0f;
    for (int j = 0; j < a.k; ++j)
      s += coherent_load_f32(a.part + static_cast<size_t>(r * a.k + order[r][j]) * S::kH + n);
    if (a.shared) s += coherent_load_f32(a.part + static_cast<size_t>(a.R * a.k + r) * S::kH + n);
    a.y[static_cast<size_t>(r) * S::kH + n] = s;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[1 + tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dev

// ===========================================================================
// host side
// ===========================================================================
namespace {

struct WsLayout {
  size_t logits, counters, idx, wts, h, part, total;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

WsLayout ws_layout(const moe_dims& d, int rows) {
  WsLayout l{};
  size_t o = 0;
  const size_t pairs = static_cast<size_t>(rows) * d.top_k + rows;
  l.counters = o; o = align_up(o + 4 * (1 + dev::kMaxTiles), 256);
  l.logits = o;   o = align_up(o + 8 * static_cast<size_t>(rows) * d.n_experts, 256);
  l.idx = o;      o = align_up(o + 4 * static_cast<size_t>(rows) * d.top_k, 256);
  l.wts = o;      o = align_up(o + 4 * static_cast<size_t>(rows) * d.top_k, 256);
  l.h = o;        o = align_up(o + 4 * pairs * d.inter, 256);
  l.part = o;     o = align_up(o + 4 * pairs * d.hidden, 256);
  l.total = o;
  return l;
}

int shape_class(const moe_dims* d) {
  if (d->hidden == 5120 && d->inter == 2304) return 1;
  if (d->hidden == 512 && d->inter == 256) return 2;
  return 0;
}

int check_dims(const moe_dims* d, int rows) {
  if (!d) return MOE_EINVAL;
  if (rows < 0) return MOE_EINVAL;
  if (!shape_class(d)) return MOE_ESHAPE;
  if (d->top_k < 1 || d->top_k > MOE_MAX_TOP_K || d->n_experts < d->top_k || d->n_experts > 4096)
    return MOE_ESHAPE;
  if (rows > MOE_MAX_DECODE_ROWS || rows * d->top_k > 64) return MOE_ESHAPE;
  return MOE_OK;
}

template <class S>
int launch_layer(const moe_dims* d, int rows, dev::Args a, bool route, bool ffn, hipStream_t s,
                 void* const* events, int n_events) {
  const size_t lds = S::LDS_BYTES;
  const int n_routed = rows * d->top_k;
  auto rec = [&](int i) {
    if (events && i < n_events) hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
  };
  rec(0);
  if (route) {
    const int extra = (a.shared && a.shared_in_route) ? S::TILES_GU : 0;
    hipLaunchKernelGGL(dev::k_route<S>, dim3(d->n_experts + extra), dim3(dev::kThreads), lds, s, a);
    if (hipGetLastError() != hipSuccess) return MOE_EDEVICE;
  }
  rec(1);
  if (ffn) {
    const int slots_gu = n_routed + ((a.shared && !a.shared_in_route) ? 1 : 0);
    hipLaunchKernelGGL(dev::k_gateup<S>, dim3(slots_gu * S::TILES_GU), dim3(dev::kThreads), lds, s,
                       a, slots_gu);
    if (hipGetLastError() != hipSuccess) return MOE_EDEVICE;
    rec(2);
    const int slots_dn = n_routed + (a.shared ? 1 : 0);
    hipLaunchKernelGGL(dev::k_down<S>, dim3(slots_dn * S::TILES_DN), dim3(dev::kThreads), lds, s,
                       a, slots_dn);
    if (hipGetLastError() != hipSuccess) return MOE_EDEVICE;
    rec(3);
  }
  return MOE_OK;
}

int run(const moe_dims* d, const void* x, int rows, const float* w_router, const float* bias,
        const void* weights, const moe_expert_ref* experts, const moe_expert_ref* shared,
        int32_t* idx, float* wts, float* y, void* ws, size_t ws_bytes, void* stream,
        bool route, bool ffn, void* const* events, int n_events) {
  int st = check_dims(d, rows);
  if (st) return st;
  if (rows == 0) return MOE_OK;
  if (!x || !ws) return MOE_EINVAL;
  if (route && !w_router) return MOE_EINVAL;
  if (ffn && (!weights || !experts || !y)) return MOE_EINVAL;
  if (!route && (!idx || !wts)) return MOE_EINVAL;
  const WsLayout l = ws_layout(*d, rows);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  dev::Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w_router = w_router;
  a.bias = bias;
  a.weights = static_cast<const uint8_t*>(weights);
  a.experts = experts;
  a.shared = shared;
  a.idx = idx ? idx : reinterpret_cast<int32_t*>(w8 + l.idx);
  a.wts = wts ? wts : reinterpret_cast<float*>(w8 + l.wts);
  a.y = y;
  a.logits = reinterpret_cast<double*>(w8 + l.logits);
  a.counters = reinterpret_cast<uint32_t*>(w8 + l.counters);
  a.h = reinterpret_cast<float*>(w8 + l.h);
  a.part = reinterpret_cast<float*>(w8 + l.part);
  a.R = rows;
  a.k = d->top_k;
  a.E = d->n_experts;
  a.shared_in_route = (route && ffn && shared) ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (shape_class(d)) {
    case 1: return launch_layer<dev::Shape<5120, 2304>>(d, rows, a, route, ffn, s, events, n_events);
    case 2: return launch_layer<dev::Shape<512, 256>>(d, rows, a, route, ffn, s, events, n_events);
    default: return MOE_ESHAPE;
  }
}

}  // namespace
}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_EFORMAT: return "unknown weight format";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EDEVICE: return "HIP launch or runtime error";
    case MOE_ECODE: return "invalid packed code";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_dims* dims, int32_t rows) {
  if (moe::check_dims(dims, rows < 1 ? 1 : rows)) return 0;
  return moe::ws_layout(*dims, rows < 1 ? 1 : rows).total;
}

int moe_check_experts(const moe_dims* dims, const moe_expert_ref* table, int32_t count,
                      size_t weights_bytes) {
  if (!dims || !table || count < 0) return MOE_EINVAL;
  if (!moe::shape_class(dims)) return MOE_ESHAPE;
  for (int i = 0; i < count; ++i) {
    const moe_expert_ref& r = table[i];
    if (moe::format_info(static_cast<int>(r.fmt)).block == 0) return MOE_EFORMAT;
    if (r.reserved != 0) return MOE_EINVAL;
    const size_t gu = moe::packed_bytes(static_cast<int>(r.fmt), dims->inter, dims->hidden);
    const size_t dn = moe::packed_bytes(static_cast<int>(r.fmt), dims->hidden, dims->inter);
    if (!gu || !dn) return MOE_ESHAPE;
    const uint64_t offs[3] = {r.gate, r.up, r.down};
    const size_t sizes[3] = {gu, gu, dn};
    for (int m = 0; m < 3; ++m) {
      if (offs[m] % 16) return MOE_EINVAL;
      if (offs[m] > weights_bytes || sizes[m] > weights_bytes - offs[m]) return MOE_EINVAL;
    }
  }
  return MOE_OK;
}

int moe_route(const moe_dims* dims, const void* x_bf16, int32_t rows, const float* w_router,
              const float* sel_bias, int32_t* idx, float* wts, void* ws, size_t ws_bytes,
              void* stream) {
  if (rows > 0 && (!idx || !wts)) return MOE_EINVAL;
  return moe::run(dims, x_bf16, rows, w_router, sel_bias, nullptr, nullptr, nullptr, idx, wts,
                  nullptr, ws, ws_bytes, stream, true, false, nullptr, 0);
}

int moe_expert_ffn(const moe_dims* dims, const void* x_bf16, int32_t rows, const int32_t* idx,
                   const float* wts, const void* weights, const moe_expert_ref* experts,
                   const moe_expert_ref* shared, float* y, void* ws, size_t ws_bytes,
                   void* stream) {
  return moe::run(dims, x_bf16, rows, nullptr, nullptr, weights, experts, shared,
                  const_cast<int32_t*>(idx), const_cast<float*>(wts), y, ws, ws_bytes, stream,
                  false, true, nullptr, 0);
}

int moe_layer(const moe_dims* dims, const void* x_bf16, int32_t rows, const float* w_router,
              const float* sel_bias, const void* weights, const moe_expert_ref* experts,
              const moe_expert_ref* shared, int32_t* idx, float* wts, float* y, void* ws,
              size_t ws_bytes, void* stream) {
  return moe::run(dims, x_bf16, rows, w_router, sel_bias, weights, experts, shared, idx, wts, y,
                  ws, ws_bytes, stream, true, true, nullptr, 0);
}

int moe_layer_profiled(const moe_dims* dims, const void* x_bf16, int32_t rows,
                       const float* w_router, const float* sel_bias, const void* weights,
                       const moe_expert_ref* experts, const moe_expert_ref* shared,
                       int32_t* idx, float* wts, float* y, void* ws, size_t ws_bytes,
                       void* stream, void* const* events, int32_t n_events) {
  if (!events || n_events < 4) return MOE_EINVAL;
  return moe::run(dims, x_bf16, rows, w_router, sel_bias, weights, experts, shared, idx, wts, y,
                  ws, ws_bytes, stream, true, true, events, n_events);
}

}  // extern "C"
