// gfx950 kernels of the routed-MoE expert FFN and the C-ABI entry points
// that launch them.
//
// One layer call runs five kernels on the caller's stream.  No kernel waits
// on another workgroup of its own launch: on MI355X a device-scope release
// (or a contended atomic) from hundreds of workgroups serialises across the
// eight XCDs, so every cross-workgroup hand-off is a kernel boundary.
//   route    router GEMV (fp64 sums), one workgroup per expert; beside it,
//            workgroups that build the activation records of every weight
//            format, and the shared expert's gate/up tiles (its weights
//            stream while the router runs)
//   select   one workgroup: top-k per row by logit + bias, ties to the lower
//            id; softmax of the unbiased logits over the selection; the slot
//            table of distinct experts and the rows each serves
//   gateup   one workgroup per (distinct expert, tile of channels):
//            h = silu(W_gate x) * (W_up x) in fp32
//   down     one workgroup per (expert, tile of outputs): w * (W_down h)
//   combine  y = the row's expert outputs in ascending id, then the shared
//            expert -- a fixed order, so y is bitwise reproducible
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
constexpr int kMaxSlots = 64;                  // distinct routed experts per call (rows * top_k)
constexpr int kNumFmt = 5;                     // format tags 1..5
constexpr int kPrepWGs = 16;                   // workgroups building activation records
constexpr int kSelQ = 8;                       // experts per lane in the selection (E <= 512)

// One entry of the slot table: a distinct selected expert (or the shared one)
// and the rows it serves.
struct SlotEntry {
  moe_expert_ref ref;       // format and matrix offsets, copied from the expert table
  int expert;               // routed id, -1 for the shared expert
  int nt;                   // rows served
  int row[kMaxRows];        // token row r
  int pair[kMaxRows];       // h / partial row: r*k + kk (routed) or R*k + r (shared)
  float w[kMaxRows];        // mixing weight (1 for the shared expert)
};

struct SlotTable {
  int n_active;             // distinct routed experts in this call
  int pad[3];
  SlotEntry e[kMaxSlots];
};

struct Args {
  const uint16_t* x;              // [R x H] bf16
  const float* w_router;          // [E x H]
  const float* bias;              // [E] or null
  const uint8_t* weights;
  const moe_expert_ref* experts;  // [E]
  const moe_expert_ref* shared;   // [1] or null
  int32_t* idx;                   // [R x k]
  float* wts;                     // [R x k]
  float* y;                       // [R x H]
  double* logits;                 // [R x E]
  SlotTable* slots;
  int32_t* order;                 // [R x k]: each row's k slots in ascending expert id
  uint8_t* xrec;                  // [kNumFmt][R][xrow]: activation records per format and row
  float* xinv;                    // [kNumFmt][R]: 1/sigma of those records
  float* h;                       // [(R*k + R) x I]
  float* part;                    // [(R*k + R) x H]
  int xrow;                       // bytes of one (format, row) record block
  int R, k, E;
  int shared_early;               // 1: the shared expert's gate/up rides with the selection
                                  // and its down with the routed gate/up (moe_layer)
};

// ---------------------------------------------------------------------------
// shape-dependent constants
// ---------------------------------------------------------------------------
constexpr int lpr_for(int k) { return k >= 4096 ? 16 : (k >= 512 ? 8 : 4); }

template <class F>
constexpr int phase_units() {
  return sizeof(typename F::Raw) > 28 ? 2 : 5;  // units per load phase: bounds the registers
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
  static constexpr int XROW = max_rec_row(H);   // one (format, row) block of x records
  // LDS: token-row records, then the ternary decode table
  static constexpr int LDS_REC = kNTB * (max_rec_row(H) > max_rec_row(I) ? max_rec_row(H) : max_rec_row(I));
  static constexpr int LDS_TABLE = 256 * 4;
  static constexpr int LDS_BYTES = LDS_REC + LDS_TABLE;
};

// ---------------------------------------------------------------------------
// activation records
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

// sigma = 2^(14 - PSHIFT - e) for the row's largest magnitude 2^e <= m < 2^(e+1):
// every record value stays below 2^15 in magnitude.
template <class F>
__device__ __forceinline__ int sigma_exp(uint32_t max_bits) {
  const int e = max_bits ? static_cast<int>(max_bits >> 23) - 127 : 0;
  return 14 - F::PSHIFT - e;
}

// Largest |value| of a row, as monotone fp32 bits; called by every thread of
// the workgroup, result valid in all threads.
template <int KR, bool BF16>
__device__ uint32_t row_max_bits(const void* src, uint32_t* red) {
  constexpr int PER = BF16 ? 8 : 4;
  constexpr int CH = (KR / PER + kThreads - 1) / kThreads;
  uint4 qs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = threadIdx.x + i * kThreads;
    qs[i] = c < KR / PER ? *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(src) +
                                                           static_cast<size_t>(c) * 16)
                         : uint4{0, 0, 0, 0};
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint4 q = qs[i];
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
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) r = r > red[w] ? r : red[w];
  return r;
}

// Records of `nb` rows into LDS, with sigma given per row (sig_exp[t]).
template <class F, int KR, bool BF16>
__device__ __forceinline__ void build_records(const void* const* rows, int nb, const int* sig_exp,
                                              uint8_t* rec, int item0, int stride) {
  constexpr int NBU = F::units(KR);
  constexpr int RSTRIDE = NBU * F::XREC;
  constexpr int PER_ROW = NBU * F::SUBS;
  for (int item = item0; item < nb * PER_ROW; item += stride) {
    const int t = item / PER_ROW, rem = item - t * PER_ROW;
    const int u = rem / F::SUBS, sub = rem - u * F::SUBS;
    float v[F::SUBV];
    load_vals<F::SUBV, KR, BF16>(rows[t], u * F::UNIT + sub * F::SUBV, v);
    const float sg = __builtin_ldexpf(1.0f, sig_exp[t]);
#pragma unroll
    for (int i = 0; i < F::SUBV; ++i) v[i] *= sg;
    F::prep_sub(v, sub, rec + t * RSTRIDE + u * F::XREC);
  }
}

// ---------------------------------------------------------------------------
// weight streaming: a double-buffered pipeline of load phases
// ---------------------------------------------------------------------------
template <class F, int K, int LPR, int RT, int NT>
__device__ __forceinline__ void dot_unit(const typename F::Raw (&raw)[RT], const uint8_t* rec,
                                         int nt, float (&acc)[RT][NT], const uint32_t* table,
                                         int b) {
  constexpr int RSTRIDE = F::units(K) * F::XREC;
  if constexpr (std::is_same_v<F, FmtTern>)
    FmtTern::template dot<RT, NT>(raw, rec + b * F::XREC, RSTRIDE, nt, acc, table);
  else
    F::template dot<RT, NT>(raw, rec + b * F::XREC, RSTRIDE, nt, acc);
}

// Streams the lane's units of RT matrix rows (mats[r], row rows[r]) and
// accumulates them against the staged records.  Phase 0 is loaded by
// load_first() so the caller can overlap it with record staging.
template <class F, int K, int LPR, int RT>
struct Stream {
  static constexpr int NBU = F::units(K);
  static constexpr int UPL = (NBU + LPR - 1) / LPR;
  static constexpr int G = phase_units<F>() < UPL ? phase_units<F>() : UPL;
  static constexpr int P = (UPL + G - 1) / G;
  typename F::Raw raw[2][G][RT];

  __device__ __forceinline__ bool live(int j, int c) const {
    return j < UPL && (NBU % LPR == 0 || c + j * LPR < NBU);
  }
  __device__ __forceinline__ void load(int p, const Buf (&mats)[RT],
                                       const int (&rows)[RT], int nrows, bool valid) {
    const int c = threadIdx.x % LPR;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = p * G + g;
      if (valid && live(j, c))
#pragma unroll
        for (int r = 0; r < RT; ++r) F::load(raw[p & 1][g][r], mats[r], nrows, NBU, rows[r], c + j * LPR);
    }
  }
  template <int NT>
  __device__ __forceinline__ void run(const Buf (&mats)[RT], const int (&rows)[RT],
                                      int nrows, bool valid, const uint8_t* rec, int nt,
                                      float (&acc)[RT][NT], const uint32_t* table) {
    const int c = threadIdx.x % LPR;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (p + 1 < P) load(p + 1, mats, rows, nrows, valid);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int j = p * G + g;
        if (valid && live(j, c)) dot_unit<F, K, LPR, RT, NT>(raw[p & 1][g], rec, nt, acc, table, c + j * LPR);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

template <class F>
__device__ __forceinline__ void build_tern_table(uint32_t* table) {
  if constexpr (std::is_same_v<F, FmtTern>)
    for (int i = threadIdx.x; i < 256; i += blockDim.x) table[i] = FmtTern::table_entry(i);
}

// ---------------------------------------------------------------------------
// gate/up tile: channels [tile*TN, tile*TN + TN) of one expert for its rows.
// STAGE_LOCAL: records are built here from x (shared expert riding in the
// router launch); otherwise they are copied from the per-layer record buffer.
// ---------------------------------------------------------------------------
template <class S, class F, bool STAGE_LOCAL>
__device__ void gateup_tile(const Args& a, const SlotEntry& sl, int tile, uint8_t* lds) {
  constexpr int H = S::kH, I = S::kI, LPR = S::LPR_GU;
  constexpr int RSTRIDE = F::units(H) * F::XREC;
  uint8_t* rec = lds;
  uint32_t* table = reinterpret_cast<uint32_t*>(lds + S::LDS_REC);
  __shared__ float inv_sigma[kNTB];
  __shared__ int sig_exp[kNTB];
  __shared__ uint32_t red[16];
  __shared__ const void* srcs[kNTB];
  build_tern_table<F>(table);
  const int rg = threadIdx.x / LPR, c = threadIdx.x % LPR;
  const int n = tile * S::TN_GU + rg;
  const bool valid = n < I;
  const Buf mats[2] = {make_buf(a.weights + sl.ref.gate, F::bytes(I, H)),
                       make_buf(a.weights + sl.ref.up, F::bytes(I, H))};
  const int rows[2] = {n, n};
  Stream<F, H, LPR, 2> st;
  const int fi = uniform(static_cast<int>(sl.ref.fmt) - 1);
  const int nt_all = uniform(sl.nt);
  for (int t0 = 0; t0 < nt_all; t0 += kNTB) {
    const int nb = nt_all - t0 < kNTB ? nt_all - t0 : kNTB;
    st.load(0, mats, rows, I, valid);            // weights in flight while records are staged
    __syncthreads();
    if constexpr (STAGE_LOCAL) {
      if (threadIdx.x < nb) srcs[threadIdx.x] = a.x + static_cast<size_t>(sl.row[t0 + threadIdx.x]) * H;
      __syncthreads();
      for (int t = 0; t < nb; ++t) {
        const uint32_t m = row_max_bits<H, true>(srcs[t], red);
        if (threadIdx.x == 0) {
          sig_exp[t] = sigma_exp<F>(m);
          inv_sigma[t] = __builtin_ldexpf(1.0f, -sig_exp[t]);
        }
      }
      __syncthreads();
      build_records<F, H, true>(srcs, nb, sig_exp, rec, threadIdx.x, blockDim.x);
    } else {
      // copy this format's records of the rows from the per-layer buffer
      // straight into LDS (global_load_lds_dwordx4): each wave moves 1 KB per
      // instruction, no registers involved
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      constexpr int CHUNKS = RSTRIDE / 1024 + (RSTRIDE % 1024 ? 1 : 0);
      for (int t = 0; t < nb; ++t) {
        const uint8_t* src = a.xrec + (static_cast<size_t>(fi) * a.R + sl.row[t0 + t]) * a.xrow;
        for (int ch = wave; ch < CHUNKS; ch += kThreads / 64) {
          const int off = ch * 1024 + lane * 16;
          if (off < RSTRIDE)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src + off),
                (__attribute__((address_space(3))) void*)(rec + t * RSTRIDE + ch * 1024),
                16, 0, 0);
        }
        if (threadIdx.x == 0) inv_sigma[t] = a.xinv[fi * a.R + sl.row[t0 + t]];
      }
    }
    __syncthreads();
    float acc[2][kNTB] = {};
    st.template run<kNTB>(mats, rows, I, valid, rec, nb, acc, table);
#pragma unroll
    for (int t = 0; t < kNTB; ++t) {
      acc[0][t] = group_sum<LPR>(acc[0][t]);
      acc[1][t] = group_sum<LPR>(acc[1][t]);
    }
#pragma unroll
    for (int t = 0; t < kNTB; ++t) {
      if (t < nb) {
        const float g = acc[0][t] * inv_sigma[t], v = acc[1][t] * inv_sigma[t];
        const float hv = g / (1.0f + expf(-g)) * v;
        if (valid && c == 0) a.h[static_cast<size_t>(sl.pair[t0 + t]) * I + n] = hv;
      }
    }
  }
}

// down tile: outputs [tile*TN, tile*TN + TN) of H for every row of the slot
template <class S, class F>
__device__ void down_tile(const Args& a, const SlotEntry& sl, int tile, uint8_t* lds) {
  constexpr int H = S::kH, I = S::kI, LPR = S::LPR_DN, NPG = S::NPG_DN;
  uint8_t* rec = lds;
  uint32_t* table = reinterpret_cast<uint32_t*>(lds + S::LDS_REC);
  __shared__ float inv_sigma[kNTB];
  __shared__ int sig_exp[kNTB];
  __shared__ uint32_t red[16];
  __shared__ const void* srcs[kNTB];
  build_tern_table<F>(table);
  const int rg = threadIdx.x / LPR, c = threadIdx.x % LPR;
  const int n0 = tile * S::TN_DN + rg * NPG;
  const Buf md = make_buf(a.weights + sl.ref.down, F::bytes(H, I));
  const Buf mats[NPG] = {md, md};
  const int rows[NPG] = {n0, n0 + 1};
  const bool valid = n0 + NPG <= H;
  Stream<F, I, LPR, NPG> st;
  const int nt_all = uniform(sl.nt);
  for (int t0 = 0; t0 < nt_all; t0 += kNTB) {
    const int nb = nt_all - t0 < kNTB ? nt_all - t0 : kNTB;
    st.load(0, mats, rows, H, valid);
    __syncthreads();
    if (threadIdx.x < nb) srcs[threadIdx.x] = a.h + static_cast<size_t>(sl.pair[t0 + threadIdx.x]) * I;
    __syncthreads();
    for (int t = 0; t < nb; ++t) {
      const uint32_t m = row_max_bits<I, false>(srcs[t], red);
      if (threadIdx.x == 0) {
        sig_exp[t] = sigma_exp<F>(m);
        inv_sigma[t] = __builtin_ldexpf(1.0f, -sig_exp[t]);
      }
    }
    __syncthreads();
    build_records<F, I, false>(srcs, nb, sig_exp, rec, threadIdx.x, blockDim.x);
    __syncthreads();
    float acc[NPG][kNTB] = {};
    st.template run<kNTB>(mats, rows, H, valid, rec, nb, acc, table);
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

template <class S, int STAGE>  // STAGE: 0 down, 1 gate/up from records, 2 gate/up staged locally
__device__ void run_slot(const Args& a, const SlotEntry& sl, int tile, uint8_t* lds) {
#define MOE_RUN_FMT(TAG, FT)                                                    \
  case TAG:                                                                    \
    if constexpr (STAGE == 0) down_tile<S, FT>(a, sl, tile, lds);              \
    else gateup_tile<S, FT, STAGE == 2>(a, sl, tile, lds);                     \
    break;
  switch (sl.ref.fmt) {
    MOE_RUN_FMT(MOE_FMT_Q2_0, FmtQ2)
    MOE_RUN_FMT(MOE_FMT_Q8, FmtQ8)
    MOE_RUN_FMT(MOE_FMT_MXFP4, FmtMXFP4)
    MOE_RUN_FMT(MOE_FMT_TERN160, FmtTern)
    MOE_RUN_FMT(MOE_FMT_Q3, FmtQ3)
    default:
      break;  // tables are checked on the host (moe_check_experts)
  }
#undef MOE_RUN_FMT
}

// ---------------------------------------------------------------------------
// per-layer preparation: slot table and activation records
// ---------------------------------------------------------------------------
// Distinct experts of the routing in ascending id, each with the rows that
// chose it, and every row's k entries in ascending id.  Run by wave 0; ids
// and weights come from LDS (ids[R*k], wv[R*k]).
__device__ void build_slot_table(const Args& a, const int* ids, const float* wv) {
  const int lane = threadIdx.x;
  const int n = a.R * a.k;
  const int v = lane < n ? ids[lane] : 0x7fffffff;
  bool first = lane < n;
  int rank = 0;
  for (int m = 0; m < n; ++m) {
    const int vm = ids[m];
    if (m < lane && vm == v) first = false;
  }
  const uint64_t firsts = __ballot(first);
  for (int m = 0; m < n; ++m)
    if (((firsts >> m) & 1ull) && ids[m] < v) ++rank;
  if (first) {
    SlotEntry& e = a.slots->e[rank];
    e.ref = a.experts[v];
    e.expert = v;
    int t = 0;
    for (int m = 0; m < n && t < kMaxRows; ++m) {  // distinct ids per row bound t by R
      if (ids[m] == v) {
        e.row[t] = m / a.k;
        e.pair[t] = m;
        e.w[t] = wv[m];
        ++t;
      }
    }
    e.nt = t;
  }
  if (lane < a.R) {
    const int* row = ids + lane * a.k;
    for (int j = 0; j < a.k; ++j) {   // position of entry j = number of smaller ids in the row
      int pos = 0;
      for (int q = 0; q < a.k; ++q) pos += row[q] < row[j] || (row[q] == row[j] && q < j);
      a.order[lane * a.k + pos] = j;
    }
  }
  if (lane == 0) a.slots->n_active = __popcll(firsts);
}

// Activation records of every format for every row, built by kPrepWGs
// workgroups (p = 0 .. kPrepWGs-1).
template <class S, class F>
__device__ void prep_format(const Args& a, int p, const int* sig_base) {
  constexpr int H = S::kH;
  const int fi = F::TAG - 1;
  __shared__ int sig_exp[kMaxRows];
  __shared__ const void* srcs[kMaxRows];
  if (threadIdx.x < a.R) {
    sig_exp[threadIdx.x] = sig_base[threadIdx.x] - F::PSHIFT;
    srcs[threadIdx.x] = a.x + static_cast<size_t>(threadIdx.x) * H;
    if (p == 0) a.xinv[fi * a.R + threadIdx.x] = __builtin_ldexpf(1.0f, -sig_exp[threadIdx.x]);
  }
  __syncthreads();
  // rows of this format are a.xrow apart; build_records strides rows by the
  // format's own record row, so build one row at a time
  for (int r = 0; r < a.R; ++r)
    build_records<F, H, true>(srcs + r, 1, sig_exp + r, a.xrec + (static_cast<size_t>(fi) * a.R + r) * a.xrow,
                              p * blockDim.x + threadIdx.x, kPrepWGs * blockDim.x);
}

template <class S>
__device__ void prep_wg(const Args& a, int p) {
  __shared__ uint32_t red[16];
  __shared__ int base[kMaxRows];
  for (int r = 0; r < a.R; ++r) {
    const uint32_t m = row_max_bits<S::kH, true>(a.x + static_cast<size_t>(r) * S::kH, red);
    if (threadIdx.x == 0) base[r] = m ? 14 - (static_cast<int>(m >> 23) - 127) : 14;
  }
  __syncthreads();
  prep_format<S, FmtQ2>(a, p, base);
  prep_format<S, FmtQ8>(a, p, base);
  prep_format<S, FmtMXFP4>(a, p, base);
  prep_format<S, FmtTern>(a, p, base);
  prep_format<S, FmtQ3>(a, p, base);
}

// ---------------------------------------------------------------------------
// router GEMV + top-k
// ---------------------------------------------------------------------------
template <int H>
__device__ void router_wg(const Args& a, int e, double* red) {
  constexpr int CH = (H / 4 + kThreads - 1) / kThreads;   // float4 chunks per thread
  double acc[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.0;
  const float4* wr = reinterpret_cast<const float4*>(a.w_router + static_cast<size_t>(e) * H);
  float4 w[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = threadIdx.x + i * kThreads;
    w[i] = j < H / 4 ? wr[j] : float4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    if (r < a.R) {
      uint2 xb[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int j = threadIdx.x + i * kThreads;
        xb[i] = j < H / 4 ? *reinterpret_cast<const uint2*>(a.x + static_cast<size_t>(r) * H + 4 * j)
                          : uint2{0u, 0u};
      }
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        s = fma(static_cast<double>(w[i].x), static_cast<double>(bf16_bits_to_f32(xb[i].x & 0xFFFFu)), s);
        s = fma(static_cast<double>(w[i].y), static_cast<double>(bf16_bits_to_f32(xb[i].x >> 16)), s);
        s = fma(static_cast<double>(w[i].z), static_cast<double>(bf16_bits_to_f32(xb[i].y & 0xFFFFu)), s);
        s = fma(static_cast<double>(w[i].w), static_cast<double>(bf16_bits_to_f32(xb[i].y >> 16)), s);
      }
      acc[r] = s;
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
// the softmax of the unbiased logits over the selection.  One wave per row;
// the logits come from the previous kernel, so plain loads see them.
__device__ void select_row(const Args& a, int r, int* sel, float* wsel) {
  const int lane = threadIdx.x & 63;
  const double* lg = a.logits + static_cast<size_t>(r) * a.E;
  // every logit and key of the lane in registers before the k rounds
  double lv[kSelQ];
  uint64_t kv[kSelQ];
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    const int e = lane + 64 * q;
    lv[q] = e < a.E ? lg[e] : 0.0;
  }
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    const int e = lane + 64 * q;
    const double key = ((e < a.E && a.bias) ? lv[q] + static_cast<double>(a.bias[e]) : lv[q]) + 0.0;  // -0 -> +0
    kv[q] = e < a.E ? f64_order_key(key) : 0ull;   // 0 is below every real key
  }
  double my_l = 0.0;     // lane j keeps the unbiased logit of the j-th selection
  int my_id = 0;
  double lmax = -INFINITY;
  for (int j = 0; j < a.k; ++j) {
    uint64_t bk = 0;
    int bid = 0x7fffffff;
    double bl = 0.0;
#pragma unroll
    for (int q = 0; q < kSelQ; ++q) {
      const int e = lane + 64 * q;
      if (e < a.E && key_better(kv[q], e, bk, bid)) {
        bk = kv[q];
        bid = e;
        bl = lv[q];
      }
    }
    int wid = bid;
    uint64_t wk = bk;
    wave_argmax(wk, wid);
    // the winner's unbiased logit, from the lane that holds it
    const int owner = wid & 63;
    const uint32_t l_lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(__builtin_bit_cast(uint64_t, bl)), owner);
    const uint32_t l_hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(__builtin_bit_cast(uint64_t, bl) >> 32), owner);
    const double wlog = __builtin_bit_cast(double, (static_cast<uint64_t>(l_hi) << 32) | l_lo);
#pragma unroll
    for (int q = 0; q < kSelQ; ++q)
      if (lane + 64 * q == wid) kv[q] = 0ull;   // taken
    if (lane == j) {
      my_l = wlog;
      my_id = wid;
    }
    lmax = wlog > lmax ? wlog : lmax;
  }
  // softmax of the unbiased logits over the selection: one exp per lane
  const double e = lane < a.k ? exp(my_l - lmax) : 0.0;
  double s = e;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o, 64);
  if (lane < a.k) {
    const float w = static_cast<float>(e / s);
    sel[lane] = my_id;
    wsel[lane] = w;
    a.idx[r * a.k + lane] = my_id;
    a.wts[r * a.k + lane] = w;
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// route: router workgroups [0, E) write logits; record builders
// [E, E + kPrepWGs) build the activation records of every format.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_route(Args a) {
  __shared__ double red[kMaxRows * 16];
  const int bid = blockIdx.x;
  if (bid >= a.E) {
    prep_wg<S>(a, bid - a.E);
    return;
  }
  router_wg<S::kH>(a, bid, red);
}

__device__ void shared_entry_init(const Args& a, SlotEntry* e) {
  if (threadIdx.x == 0) {
    e->ref = *a.shared;
    e->expert = -1;
    e->nt = a.R;
    for (int r = 0; r < a.R; ++r) {
      e->row[r] = r;
      e->pair[r] = a.R * a.k + r;
      e->w[r] = 1.0f;
    }
  }
  __syncthreads();
}

// select: workgroup 0 picks the top-k per row and builds the slot table;
// workgroups 1.. stream the shared expert's gate/up tiles meanwhile (they
// depend only on x), so the selection's latency is hidden behind them.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_select(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ SlotEntry se;
  if (blockIdx.x > 0) {
    shared_entry_init(a, &se);
    run_slot<S, 1>(a, se, blockIdx.x - 1, lds);
    return;
  }
  __shared__ int sel[kMaxRows * kMaxK];
  __shared__ float wsel[kMaxRows * kMaxK];
  for (int r = threadIdx.x >> 6; r < a.R; r += blockDim.x >> 6)
    select_row(a, r, sel + r * a.k, wsel + r * a.k);
  __syncthreads();
  if (a.experts && threadIdx.x < 64) build_slot_table(a, sel, wsel);
}

// Preparation for a caller-given routing: slot table (workgroup 0) and
// activation records (workgroups 1 .. kPrepWGs).
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_prep(Args a) {
  if (blockIdx.x == 0) {
    __shared__ int ids[kMaxRows * kMaxK];
    __shared__ float wv[kMaxRows * kMaxK];
    for (int i = threadIdx.x; i < a.R * a.k; i += blockDim.x) {
      ids[i] = a.idx[i];
      wv[i] = a.wts[i];
    }
    __syncthreads();
    if (threadIdx.x < 64) build_slot_table(a, ids, wv);
    return;
  }
  prep_wg<S>(a, blockIdx.x - 1);
}

__device__ __forceinline__ void load_slot(const Args& a, int si, SlotEntry* sl) {
  if (threadIdx.x < static_cast<int>(sizeof(SlotEntry) / 4))
    reinterpret_cast<uint32_t*>(sl)[threadIdx.x] = reinterpret_cast<const uint32_t*>(&a.slots->e[si])[threadIdx.x];
  __syncthreads();
}

// gateup: routed (slot, tile) workgroups [0, n_slots * TILES_GU); then the
// shared expert's gate/up tiles (caller-given routing) or, in moe_layer, its
// down tiles, which only need the shared h of the previous kernel.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_gateup(Args a, int n_slots) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ SlotEntry sl;
  const int routed = n_slots * S::TILES_GU;
  if (static_cast<int>(blockIdx.x) >= routed) {
    shared_entry_init(a, &sl);
    if (a.shared_early) run_slot<S, 0>(a, sl, blockIdx.x - routed, lds);
    else run_slot<S, 1>(a, sl, blockIdx.x - routed, lds);
    return;
  }
  const int slot = blockIdx.x % n_slots, tile = blockIdx.x / n_slots;
  if (slot >= a.slots->n_active) return;
  load_slot(a, slot, &sl);
  run_slot<S, 1>(a, sl, tile, lds);
}

// down: routed (slot, output tile) workgroups write w * (W_down h) into the
// partials; then the shared expert's down tiles when not done earlier.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_down(Args a, int n_slots) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ SlotEntry sl;
  const int routed = n_slots * S::TILES_DN;
  if (static_cast<int>(blockIdx.x) >= routed) {
    shared_entry_init(a, &sl);
    run_slot<S, 0>(a, sl, blockIdx.x - routed, lds);
    return;
  }
  const int slot = blockIdx.x % n_slots, tile = blockIdx.x / n_slots;
  if (slot >= a.slots->n_active) return;
  load_slot(a, slot, &sl);
  run_slot<S, 0>(a, sl, tile, lds);
}

// Combine: y[r] = sum over the row's experts in ascending id, then the shared
// expert -- a fixed order, so y is bitwise reproducible.
template <class S>
__global__ __launch_bounds__(kThreads) void k_combine(Args a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.R * S::kH) return;
  const int r = i / S::kH, n = i - r * S::kH;
  float s = 0.0f;
  for (int j = 0; j < a.k; ++j)
    s += a.part[static_cast<size_t>(r * a.k + a.order[r * a.k + j]) * S::kH + n];
  if (a.shared) s += a.part[static_cast<size_t>(a.R * a.k + r) * S::kH + n];
  a.y[i] = s;
}

}  // namespace dev

// ===========================================================================
// host side
// ===========================================================================
namespace {

struct WsLayout {
  size_t logits, idx, wts, slots, order, xinv, xrec, h, part, total;
  int xrow;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int xrow_for(const moe_dims& d) {
  if (d.hidden == 5120) return dev::Shape<5120, 2304>::XROW;
  return dev::Shape<512, 256>::XROW;
}

WsLayout ws_layout(const moe_dims& d, int rows) {
  WsLayout l{};
  size_t o = 0;
  const size_t pairs = static_cast<size_t>(rows) * d.top_k + rows;
  l.xrow = xrow_for(d);
  l.logits = o;   o = align_up(o + 8 * static_cast<size_t>(rows) * d.n_experts, 256);
  l.idx = o;      o = align_up(o + 4 * static_cast<size_t>(rows) * d.top_k, 256);
  l.wts = o;      o = align_up(o + 4 * static_cast<size_t>(rows) * d.top_k, 256);
  l.slots = o;    o = align_up(o + sizeof(dev::SlotTable), 256);
  l.order = o;    o = align_up(o + 4 * static_cast<size_t>(rows) * d.top_k, 256);
  l.xinv = o;     o = align_up(o + 4 * static_cast<size_t>(dev::kNumFmt) * rows, 256);
  l.xrec = o;     o = align_up(o + static_cast<size_t>(dev::kNumFmt) * rows * l.xrow, 256);
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
  if (d->top_k < 1 || d->top_k > MOE_MAX_TOP_K || d->n_experts < d->top_k ||
      d->n_experts > 64 * dev::kSelQ)
    return MOE_ESHAPE;
  if (rows > MOE_MAX_DECODE_ROWS || rows * d->top_k > 64) return MOE_ESHAPE;
  return MOE_OK;
}

template <class S>
int launch_layer(const moe_dims* d, int rows, dev::Args a, bool route, bool ffn, hipStream_t s,
                 void* const* events, int n_events) {
  const size_t lds = S::LDS_BYTES;
  const int n_routed = rows * d->top_k;
  const bool sh = a.shared != nullptr;
  int ev = 0;
  auto rec = [&]() {
    if (events && ev < n_events) (void)hipEventRecord(static_cast<hipEvent_t>(events[ev]), s);
    ++ev;
  };
  auto launched = [&]() {
    rec();
    return hipGetLastError() == hipSuccess;
  };
  rec();
  if (route) {
    hipLaunchKernelGGL(dev::k_route<S>, dim3(d->n_experts + dev::kPrepWGs), dim3(dev::kThreads), 0,
                       s, a);
    if (!launched()) return MOE_EDEVICE;
    const int shared_gu = (sh && a.shared_early) ? S::TILES_GU : 0;
    hipLaunchKernelGGL(dev::k_select<S>, dim3(1 + shared_gu), dim3(dev::kThreads), lds, s, a);
    if (!launched()) return MOE_EDEVICE;
  } else {
    hipLaunchKernelGGL(dev::k_prep<S>, dim3(1 + dev::kPrepWGs), dim3(dev::kThreads), 0, s, a);
    if (!launched()) return MOE_EDEVICE;
  }
  if (ffn) {
    const int shared_b = sh ? (a.shared_early ? S::TILES_DN : S::TILES_GU) : 0;
    hipLaunchKernelGGL(dev::k_gateup<S>, dim3(n_routed * S::TILES_GU + shared_b), dim3(dev::kThreads),
                       lds, s, a, n_routed);
    if (!launched()) return MOE_EDEVICE;
    const int shared_c = (sh && !a.shared_early) ? S::TILES_DN : 0;
    hipLaunchKernelGGL(dev::k_down<S>, dim3(n_routed * S::TILES_DN + shared_c), dim3(dev::kThreads),
                       lds, s, a, n_routed);
    if (!launched()) return MOE_EDEVICE;
    hipLaunchKernelGGL(dev::k_combine<S>, dim3((rows * S::kH + dev::kThreads - 1) / dev::kThreads),
                       dim3(dev::kThreads), 0, s, a);
    if (!launched()) return MOE_EDEVICE;
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
  a.slots = reinterpret_cast<dev::SlotTable*>(w8 + l.slots);
  a.order = reinterpret_cast<int32_t*>(w8 + l.order);
  a.xinv = reinterpret_cast<float*>(w8 + l.xinv);
  a.xrec = w8 + l.xrec;
  a.xrow = l.xrow;
  a.h = reinterpret_cast<float*>(w8 + l.h);
  a.part = reinterpret_cast<float*>(w8 + l.part);
  a.R = rows;
  a.k = d->top_k;
  a.E = d->n_experts;
  a.shared_early = (route && ffn && shared) ? 1 : 0;
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
  if (!events || n_events < 6) return MOE_EINVAL;
  return moe::run(dims, x_bf16, rows, w_router, sel_bias, weights, experts, shared, idx, wts, y,
                  ws, ws_bytes, stream, true, true, events, n_events);
}

}  // extern "C"
