// gfx950 kernels of the routed-MoE expert FFN and the C-ABI entry points
// that launch them.
//
// moe_layer is one launch (k_layer) whose workgroups hand work to each other
// through tagged words in the workspace (a 64-bit word: call tag << 32 |
// payload, written and polled with relaxed device-scope accesses; a word
// counts only once it carries this call's tag, so no fences and no counters):
//   router     one workgroup per expert: logits with fp64 sums
//   selection  one wave per row: top-k by logit + bias, ties to the lower id,
//              softmax of the unbiased logits over the selection; published
//              with each expert's matrix offsets in 16 copies
//   workers    one residency round of workgroups over one list of items: the
//              shared expert's gate/up tiles (before the selection), the
//              routed gate/up items h = silu(W_gate x) * (W_up x), then the
//              down items w * (W_down h) (routed and shared)
//   combine    y = the row's expert outputs in ascending id, then the shared
//              expert -- a fixed order, so y is bitwise reproducible
// moe_route and moe_expert_ffn run the same tiles as separate kernels (route,
// select, prep, gate/up, down, combine) with kernel boundaries as the only
// synchronisation.
//
// The method: "DeepSeek-V4.1-Flash served three ways on 4xL20"
// (lcz.me/topic/2356) section 1 (layer shape, top-6 of 384 plus one shared
// expert) and section 2 (cost = expert bytes streamed); "[Strata] DeepSeek V4.1
// Flash on a single 4090" (lcz.me/post/25274) section 5.3 (selection-only bias,
// mixing weights from the unbiased router) and section 5.1 (per-expert formats).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "../../include/moe.h"
#include "dev_common.h"
#include "formats_dev.h"
#include "host_api.h"
#include "host_common.h"
#include "layout.h"
#include "prefill.h"

namespace moe {
namespace dev {

constexpr int kThreads = lay::kThreads;
#ifndef MOE_WAVES_PER_EU
#define MOE_WAVES_PER_EU 4  // occupancy floor: 4 waves per SIMD (<= 128 VGPRs)
#endif
constexpr int kMaxRows = lay::kMaxRows;        // rows per call on the decode path
constexpr int kMaxK = lay::kMaxK;
constexpr int kNTB = 1;                        // token rows staged in LDS at once
constexpr int kMaxSlots = lay::kMaxSlots;      // distinct routed experts per call (rows * top_k)
constexpr int kNumFmt = lay::kNumFmt;          // format tags 1..5
constexpr int kPrepWGs = 16;                   // workgroups building activation records
constexpr int kSelQ = lay::kMaxExperts / 64;   // experts per lane in the selection
// The published selection of the fused launch (layout.h): kSelWords tagged
// words per entry in kSelRep copies, kSelRepWords apart.  The workers poll
// copy blockIdx % kSelRep, so a thousand polling workgroups spread over many
// memory channels instead of queueing on the same few lines.  Copy 0 is the
// one the combine reads.  Word kSelEntryWords of each copy: "the logits are
// all out" (payload 1), published by the selection of row 0 as soon as its
// wait ends.
constexpr int kSelWords = lay::kSelWords;
constexpr int kSelRep = lay::kSelRep;
constexpr int kSelEntryWords = lay::kSelEntryWords;
constexpr int kSelRepWords = lay::kSelRepWords;

using lay::SlotEntry;
using lay::SlotTable;

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
  // fused layer (one launch for route, select, gate/up and down): tagged
  // hand-off words and the layout of the workgroup roles
  uint32_t tag;                   // this call's tag: unique in the process (never 0)
  uint32_t* err;                  // [1] the tag of a call in which a wait gave up
  int spin_limit;                 // polls before a hand-off wait gives up
  uint64_t* part_t;               // [(R*k + R) x H] partial outputs as tagged fp32
  uint64_t* rmax_t;               // [R x H / kThreads] per combine workgroup: max |y + noise| (stack decode)
  const float* noise;             // stack decode: [R x H] fp32 added to y, or null
  uint16_t* x_next;               // stack decode: [R x H] the next layer's bf16 input, or null
  uint64_t* lgt;                  // [R x E x 2] logits as tagged halves (low, high)
  uint64_t* selt;                 // kSelRep copies of [R x k x kSelWords] selection entries
  uint64_t* ht;                   // [(R*k + R) x I] h as tagged fp32
  int base_b, nb;                 // fused launch: first worker workgroup, number of workers
  int nsw;                        // fused launch: workers that take the shared gate/up tiles
  // stack decode: the fused combine also writes the next layer's input
  int shared_early;               // 1: the shared expert's gate/up runs beside the router
                                  // (moe_layer), so the gate/up launch skips it
  int base_y;                     // fused launch: first combine workgroup
  // many-row generic path: entries of at most kGenRows pairs of one expert
  // run through the decode tiles (idx / wts are the given routing there)
  lay::GenEntry* gen;             // [max_gen]
  int32_t* gen_n;                 // [3]: entries, gate/up items, down items
  int32_t* map_gu;                // gate/up item -> entry
  int32_t* map_dn;                // down item -> entry
  const int32_t* list;            // [R k]: pair ids grouped by expert, ascending
  const int32_t* cnt;             // [E]: pairs per expert
  int mfma;                       // 1: MXFP4 experts are left to the matrix cores
};

// ---------------------------------------------------------------------------
// tile shapes
// ---------------------------------------------------------------------------
// How one workgroup covers a matrix of format F with reduction length K: LPR
// lanes share a group of NPG channels (rows of the matrix); a workgroup owns
// TN consecutive channels.  LPR is the smallest power of two that lets every
// lane issue all of its loads at once within kLaneBudget bytes of registers,
// so a tile costs one round trip to HBM however heavy its format is; a
// format with few bytes per channel gives each lane group two channels
// instead of fewer than 8 lanes, which keeps 128-byte runs per load.
constexpr int kLaneBudget = 216;

template <class F, int K, bool GU>
struct TileCfg {
  static constexpr int NBU = F::units(K);
  static constexpr int RAW = static_cast<int>(sizeof(typename F::Raw));
  static constexpr int RTC = GU ? 2 : 1;  // matrices per channel (gate and up)
  static constexpr int lpr0() {
    int l = 1;
    while (l < 64 && ((NBU + l - 1) / l) * RTC * RAW > kLaneBudget) l *= 2;
    return l;
  }
  static constexpr int pow2_floor(int v) {
    int p = 1;
    while (p * 2 <= v) p *= 2;
    return p;
  }
  static constexpr int LPR_MIN = NBU >= 8 ? 8 : pow2_floor(NBU);
  static constexpr int LPR = lpr0() > LPR_MIN ? lpr0() : LPR_MIN;
  static constexpr int NPG = (!GU && lpr0() * 2 <= LPR) ? 2 : 1;
  static constexpr int RT = RTC * NPG;     // matrix rows per lane
  static constexpr int TN = kThreads / LPR * NPG;
  static constexpr int UPL = (NBU + LPR - 1) / LPR;
  static constexpr int g0() {
    int g = UPL;
    while (g > 1 && g * RT * RAW > kLaneBudget) --g;
    return g;
  }
  static constexpr int G = g0();           // units per load phase
  static_assert(kThreads % LPR == 0 && LPR <= 64, "lane groups must tile a wave");
};

template <int H, int I>
struct Shape {
  static constexpr int kH = H, kI = I;
  template <class F>
  static constexpr int tiles_gu() { return (I + TileCfg<F, H, true>::TN - 1) / TileCfg<F, H, true>::TN; }
  template <class F>
  static constexpr int tiles_dn() { return (H + TileCfg<F, I, false>::TN - 1) / TileCfg<F, I, false>::TN; }
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int MAX_TILES_GU =
      cmax(cmax(cmax(tiles_gu<FmtQ2>(), tiles_gu<FmtQ8>()), cmax(tiles_gu<FmtMXFP4>(), tiles_gu<FmtTern>())),
           tiles_gu<FmtQ3>());
  static constexpr int MAX_TILES_DN =
      cmax(cmax(cmax(tiles_dn<FmtQ2>(), tiles_dn<FmtQ8>()), cmax(tiles_dn<FmtMXFP4>(), tiles_dn<FmtTern>())),
           tiles_dn<FmtQ3>());
  template <class F>
  static constexpr int rec_row_bytes(int k) { return F::units(k) * F::XREC; }
  static constexpr int max_rec_row(int k) {
    return cmax(cmax(cmax(rec_row_bytes<FmtQ2>(k), rec_row_bytes<FmtQ8>(k)),
                     cmax(rec_row_bytes<FmtMXFP4>(k), rec_row_bytes<FmtTern>(k))),
                rec_row_bytes<FmtQ3>(k));
  }
  static constexpr int XROW = max_rec_row(H);   // one (format, row) block of x records
  // LDS: token-row records, then the ternary decode table
  static constexpr int LDS_REC = kNTB * cmax(max_rec_row(H), max_rec_row(I));
  static constexpr int LDS_TABLE = 256 * 4;
  static constexpr int LDS_BYTES = LDS_REC + LDS_TABLE;
  // staging of raw activations: x rows (bf16) for locally built gate/up
  // records, or h rows (fp32) handed over inside the fused launch
  static constexpr int LDS_STAGE = cmax(kNTB * I * 4, kNTB * H * 2);
  static constexpr int LDS_WITH_STAGE = LDS_BYTES + LDS_STAGE;
  // fused launch: the workers' selection words, expert refs, ids and weights
  // sit in the record area until the slot table is built (past the staging
  // area when the record area is too small): the staging area keeps x
  static constexpr int LDS_SEL_WORDS = kMaxRows * kMaxK * kSelWords * 4;
  static constexpr int LDS_SEL = LDS_SEL_WORDS + kMaxRows * kMaxK * (static_cast<int>(sizeof(moe_expert_ref)) + 8);
  static constexpr int LDS_SEL_OFF = LDS_REC >= LDS_SEL ? 0 : LDS_WITH_STAGE;
  // the ternary table [LDS_REC, LDS_BYTES) is built once per fused worker:
  // the selection's staging never overlaps it
  static_assert(LDS_SEL_OFF + LDS_SEL <= LDS_REC || LDS_SEL_OFF >= LDS_BYTES, "table kept intact");
  // the selection workgroup keeps the whole expert table (up to 64 * kSelQ
  // entries) there
  static constexpr int LDS_REFS = 64 * kSelQ * static_cast<int>(sizeof(moe_expert_ref));
  static constexpr int LDS_LAYER = cmax(cmax(LDS_WITH_STAGE, LDS_SEL_OFF + LDS_SEL), LDS_REFS);
};

// tiles of a format tag (device side: the tag comes from the expert table)
template <class S, bool GU>
__device__ __forceinline__ int tiles_of(uint32_t fmt) {
  switch (fmt) {
    case MOE_FMT_Q2_0: return GU ? S::template tiles_gu<FmtQ2>() : S::template tiles_dn<FmtQ2>();
    case MOE_FMT_Q8: return GU ? S::template tiles_gu<FmtQ8>() : S::template tiles_dn<FmtQ8>();
    case MOE_FMT_MXFP4: return GU ? S::template tiles_gu<FmtMXFP4>() : S::template tiles_dn<FmtMXFP4>();
    case MOE_FMT_TERN160: return GU ? S::template tiles_gu<FmtTern>() : S::template tiles_dn<FmtTern>();
    case MOE_FMT_Q3: return GU ? S::template tiles_gu<FmtQ3>() : S::template tiles_dn<FmtQ3>();
    default: return 0;
  }
}

// the host sizes record rows and generic work maps with layout.h's copies of
// these numbers
static_assert(Shape<5120, 2304>::XROW == lay::max_rec_row(5120) && Shape<512, 256>::XROW == lay::max_rec_row(512),
              "record row size");
static_assert(Shape<5120, 2304>::MAX_TILES_GU == 576 && Shape<5120, 2304>::MAX_TILES_DN == 320 &&
                  Shape<512, 256>::MAX_TILES_GU == 8 && Shape<512, 256>::MAX_TILES_DN == 8,
              "generic-path tile counts in layout.h");

// ---------------------------------------------------------------------------
// activation records
// ---------------------------------------------------------------------------
// A bf16 source row in LDS is read through an LDS pointer: a generic (flat)
// access also counts as a memory load, and waiting for it would wait for
// every weight load in flight as well.  (fp32 rows are still read through
// generic pointers.)
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <bool LDS>
__device__ __forceinline__ v2u ld8(const void* src, int i) {
  if constexpr (LDS)
    return reinterpret_cast<const __attribute__((address_space(3))) v2u*>(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(src)))[i];
  else return static_cast<const v2u*>(src)[i];
}
template <bool LDS>
__device__ __forceinline__ v4u ld16(const void* src, int i) {
  if constexpr (LDS)
    return reinterpret_cast<const __attribute__((address_space(3))) v4u*>(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(src)))[i];
  else return static_cast<const v4u*>(src)[i];
}

// SUBV values starting at element e0 (a multiple of 4), zero at and beyond KR
template <int SUBV, int KR, bool BF16, bool LDS = false>
__device__ __forceinline__ void load_vals(const void* src, int e0, float (&v)[SUBV]) {
#pragma unroll
  for (int c = 0; c < SUBV / 4; ++c) {
    const int e = e0 + 4 * c;
    if (e < KR) {
      if constexpr (BF16) {
        const v2u q = ld8<LDS>(src, e / 4);
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
template <int KR, bool BF16, bool LDS = false>
__device__ __forceinline__ uint32_t row_max_bits(const void* src, uint32_t* red) {
  constexpr int PER = BF16 ? 8 : 4;
  constexpr int CH = (KR / PER + kThreads - 1) / kThreads;
  v4u qs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid() + i * kThreads;
    qs[i] = c < KR / PER ? ld16<LDS>(src, c) : v4u{0, 0, 0, 0};
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const v4u q = qs[i];
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
  if ((tid() & 63) == 0) red[tid() >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
  return r;
}

// Records of `nb` rows into LDS, with sigma given per row (sig_exp[t]).
template <class F, int KR, bool BF16, bool LDS = false>
__device__ __forceinline__ void build_records(const void* const* rows, int nb, const int* sig_exp,
                                              uint8_t* rec, int item0, int stride) {
  constexpr int NBU = F::units(KR);
  constexpr int RSTRIDE = NBU * F::XREC;
  constexpr int PER_ROW = NBU * F::SUBS;
  for (int item = item0; item < nb * PER_ROW; item += stride) {
    const int t = item / PER_ROW, rem = item - t * PER_ROW;
    const int u = rem / F::SUBS, sub = rem - u * F::SUBS;
    float v[F::SUBV];
    load_vals<F::SUBV, KR, BF16, LDS>(rows[t], u * F::UNIT + sub * F::SUBV, v);
    F::prep_sub(v, __builtin_ldexpf(1.0f, sig_exp[t]), sub, rec + t * RSTRIDE + u * F::XREC);
  }
}

// Records of one row (src) into LDS with sigma 2^se; every thread calls it
// with the same se.
template <class F, int KR, bool BF16, bool LDS = false>
__device__ __forceinline__ void build_row_records(const void* src, int se, uint8_t* rec) {
  constexpr int PER_ROW = F::units(KR) * F::SUBS;
  const float g = __builtin_ldexpf(1.0f, se);
  for (int item = tid(); item < PER_ROW; item += kThreads) {
    const int u = item / F::SUBS, sub = item - u * F::SUBS;
    float v[F::SUBV];
    load_vals<F::SUBV, KR, BF16, LDS>(src, u * F::UNIT + sub * F::SUBV, v);
    F::prep_sub(v, g, sub, rec + u * F::XREC);
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
template <class F, int K, int LPR, int RT, int G>
struct Stream {
  static constexpr int NBU = F::units(K);
  static constexpr int UPL = (NBU + LPR - 1) / LPR;
  static constexpr int P = (UPL + G - 1) / G;
  typename F::Raw raw[2][G][RT];

  __device__ __forceinline__ bool live(int j, int c) const {
    return j < UPL && (NBU % LPR == 0 || c + j * LPR < NBU);
  }
  __device__ __forceinline__ void load(int p, const Buf (&mats)[RT],
                                       const int (&rows)[RT], int nrows, bool valid) {
    const int c = tid() % LPR;
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
    const int c = tid() % LPR;
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

// The ternary decode table (byte -> five trits) in LDS.  The split kernels
// build it per ternary tile; the fused launch's workers build it once, at
// their start (no other use of the fused launch's LDS overlaps it), so an
// item's weight loads are not held back by it.
template <class F, bool TAG>
__device__ __forceinline__ void build_tern_table(uint32_t* table) {
  if constexpr (std::is_same_v<F, FmtTern> && !TAG)
    for (int i = tid(); i < 256; i += kThreads) table[i] = FmtTern::table_entry(i);
}

// ---------------------------------------------------------------------------
// gate/up tile: channels [tile*TN, tile*TN + TN) of one expert for its rows.
// STAGE_LOCAL: records are built here from x (shared expert riding in the
// router launch); otherwise they are copied from the per-layer record buffer.
// ---------------------------------------------------------------------------
// Fused launch: the staging area keeps x row g_xrow (bf16) between gate/up
// items, with the largest |x| as fp32 bits in g_xmax, so that an item of that
// row loads nothing but its weights.  The workers stage row 0 at their start,
// before they wait for anything; -1: nothing staged.
__shared__ int g_xrow;
__shared__ uint32_t g_xmax;

// Stages x row r into the staging area and records it as g_xrow / g_xmax.
template <class S>
__device__ __forceinline__ void stage_x_row(const Args& a, int r, uint8_t* lds) {
  constexpr int H = S::kH, XCH = (H / 8 + kThreads - 1) / kThreads;
  __shared__ uint32_t red[kThreads / 64];
  const Buf xb = make_buf(reinterpret_cast<const uint8_t*>(a.x), static_cast<uint32_t>(a.R * H * 2));
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + S::LDS_BYTES);
  u32x4 xq[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int ch = tid() + i * kThreads;
    xq[i] = bload128(xb, ch < H / 8 ? static_cast<uint32_t>((r * H + 8 * ch) * 2) : 0x7FFFFFF0u);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int ch = tid() + i * kThreads;
    if (ch < H / 8) {
      *reinterpret_cast<u32x4*>(xs + 8 * ch) = xq[i];
      const uint32_t w[4] = {xq[i].x, xq[i].y, xq[i].z, xq[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (w[q] & 0x7FFFu) << 16, hi = (w[q] >> 16 & 0x7FFFu) << 16;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
      }
    }
  }
  m = wave_max_u32(m);
  if ((tid() & 63) == 0) red[tid() >> 6] = m;
  __syncthreads();
  if (tid() == 0) {
    uint32_t mm = 0;
    for (int w = 0; w < kThreads / 64; ++w) mm = mm > red[w] ? mm : red[w];
    g_xmax = mm;
    g_xrow = r;
  }
  __syncthreads();
}

template <class S, class F, bool STAGE_LOCAL, bool TAG>
__device__ __forceinline__ void gateup_tile(const Args& a, const SlotEntry& sl, int tile, uint8_t* lds, uint32_t tag) {
  using C = TileCfg<F, S::kH, true>;
  constexpr int H = S::kH, I = S::kI, LPR = C::LPR;
  constexpr int RSTRIDE = F::units(H) * F::XREC;
  uint8_t* rec = lds;
  uint32_t* table = reinterpret_cast<uint32_t*>(lds + S::LDS_REC);
  __shared__ float inv_sigma[kNTB];
  __shared__ int sig_exp[kNTB];
  __shared__ uint32_t red[16];
  __shared__ const void* srcs[kNTB];
  build_tern_table<F, TAG>(table);
  const int rg = tid() / LPR, c = tid() % LPR;
  const int n = tile * C::TN + rg;
  const bool valid = n < I;
  const Buf mats[2] = {make_buf(a.weights + sl.ref.gate, F::bytes(I, H)),
                       make_buf(a.weights + sl.ref.up, F::bytes(I, H))};
  const int rows[2] = {n, n};
  Stream<F, H, LPR, 2, C::G> st;
  const int fi = uniform(static_cast<int>(sl.ref.fmt) - 1);
  const int nt_all = uniform(sl.nt);
  for (int t0 = 0; t0 < nt_all; t0 += kNTB) {
    const int nb = nt_all - t0 < kNTB ? nt_all - t0 : kNTB;
    // local records: the x rows are loaded before the weights, so the
    // records are built while the weights are still in flight and one round
    // trip to memory covers both
    constexpr int XCH = (H / 8 + kThreads - 1) / kThreads;   // 16-byte chunks per thread and row
    u32x4 xq[kNTB][XCH];
    const bool cached = TAG && kNTB == 1 && uniform(g_xrow) == uniform(sl.row[t0]);
    if (STAGE_LOCAL && !cached) {
      // buffer loads: chunks past the row or rows past the batch read an
      // offset beyond the buffer and come back as zeros, without branches
      const Buf xb = make_buf(reinterpret_cast<const uint8_t*>(a.x), static_cast<uint32_t>(a.R * H * 2));
      constexpr uint32_t kNone = 0x7FFFFFF0u;
#pragma unroll
      for (int t = 0; t < kNTB; ++t) {
        const int row = t < nb ? uniform(sl.row[t0 + t]) : 0;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
          const int ch = tid() + i * kThreads;
          const uint32_t off = (t < nb && ch < H / 8) ? static_cast<uint32_t>((row * H + 8 * ch) * 2) : kNone;
          xq[t][i] = bload128(xb, off);
        }
      }
    }
    // weights in flight while records are staged; with one load phase they
    // stay in registers, so the next rows of the slot reuse them
    if (Stream<F, H, LPR, 2, C::G>::P > 1 || t0 == 0) st.load(0, mats, rows, I, valid);
    // a later row overwrites the records and staging the previous row's
    // products read; in the fused launch an item's first row follows the
    // barrier that ended the previous item
    if (!TAG || t0 > 0) __syncthreads();
    if (STAGE_LOCAL && cached) {
      // sigma from the staged row's maximum, which every thread reads (it was
      // written before an earlier barrier)
      const int se = sigma_exp<F>(g_xmax);
      if (tid() == 0) inv_sigma[0] = __builtin_ldexpf(1.0f, -se);
      build_row_records<F, H, true, true>(lds + S::LDS_BYTES, se, rec);
    } else if constexpr (STAGE_LOCAL && TAG) {
      // the row goes to the staging area and becomes the staged row; every
      // thread takes sigma from the four waves' maxima
      uint16_t* xs = reinterpret_cast<uint16_t*>(lds + S::LDS_BYTES);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < XCH; ++i) {
        const int ch = tid() + i * kThreads;
        if (ch < H / 8) {
          *reinterpret_cast<u32x4*>(xs + 8 * ch) = xq[0][i];
          const uint32_t w[4] = {xq[0][i].x, xq[0][i].y, xq[0][i].z, xq[0][i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (w[q] & 0x7FFFu) << 16, hi = (w[q] >> 16 & 0x7FFFu) << 16;
            m = m > lo ? m : lo;
            m = m > hi ? m : hi;
          }
        }
      }
      m = wave_max_u32(m);
      if ((tid() & 63) == 0) red[tid() >> 6] = m;
      __syncthreads();
      for (int w = 0; w < kThreads / 64; ++w) m = m > red[w] ? m : red[w];
      const int se = sigma_exp<F>(m);
      if (tid() == 0) {
        inv_sigma[0] = __builtin_ldexpf(1.0f, -se);
        g_xrow = sl.row[t0];
        g_xmax = m;
      }
      build_row_records<F, H, true, true>(xs, se, rec);
    } else if constexpr (STAGE_LOCAL) {
      uint16_t* xs = reinterpret_cast<uint16_t*>(lds + S::LDS_BYTES);
#pragma unroll
      for (int t = 0; t < kNTB; ++t) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
          const int ch = tid() + i * kThreads;
          if (t < nb && ch < H / 8) {
            *reinterpret_cast<u32x4*>(xs + t * H + 8 * ch) = xq[t][i];
            const uint32_t w[4] = {xq[t][i].x, xq[t][i].y, xq[t][i].z, xq[t][i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t lo = (w[q] & 0x7FFFu) << 16, hi = (w[q] >> 16 & 0x7FFFu) << 16;
              m = m > lo ? m : lo;
              m = m > hi ? m : hi;
            }
          }
        }
        m = wave_max_u32(m);
        if ((tid() & 63) == 0) red[t * 4 + (tid() >> 6)] = m;
      }
      __syncthreads();
      if (tid() < nb) {
        const int t = tid();
        uint32_t m = 0;
        for (int w = 0; w < kThreads / 64; ++w) m = m > red[t * 4 + w] ? m : red[t * 4 + w];
        sig_exp[t] = sigma_exp<F>(m);
        inv_sigma[t] = __builtin_ldexpf(1.0f, -sig_exp[t]);
        srcs[t] = xs + t * H;
        if (TAG && kNTB == 1) {
          g_xrow = sl.row[t0];
          g_xmax = m;
        }
      }
      __syncthreads();
      build_records<F, H, true, true>(srcs, nb, sig_exp, rec, tid(), kThreads);
    } else {
      // copy this format's records of the rows from the per-layer buffer
      // straight into LDS (global_load_lds_dwordx4): each wave moves 1 KB per
      // instruction, no registers involved
      const int wave = tid() >> 6, lane = tid() & 63;
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
        if (tid() == 0) inv_sigma[t] = a.xinv[fi * a.R + sl.row[t0 + t]];
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
        if (valid && c == 0) {
          const size_t o = static_cast<size_t>(sl.pair[t0 + t]) * I + n;
          if constexpr (TAG) tstore(a.ht + o, tag, __builtin_bit_cast(uint32_t, hv));
          else a.h[o] = hv;
        }
      }
    }
  }
}

// down tile: outputs [tile*TN, tile*TN + TN) of H for every row of the slot
template <class S, class F, bool TAG>
__device__ __forceinline__ void down_tile(const Args& a, const SlotEntry& sl, int tile, uint8_t* lds, uint32_t tag) {
  using C = TileCfg<F, S::kI, false>;
  constexpr int H = S::kH, I = S::kI, LPR = C::LPR, NPG = C::NPG;
  uint8_t* rec = lds;
  uint32_t* table = reinterpret_cast<uint32_t*>(lds + S::LDS_REC);
  __shared__ float inv_sigma[kNTB];
  __shared__ int sig_exp[kNTB];
  __shared__ uint32_t red[16];
  __shared__ float wrow;                 // fused launch: the row's mixing weight
  __shared__ const void* srcs[kNTB];
  build_tern_table<F, TAG>(table);
  const int rg = tid() / LPR, c = tid() % LPR;
  const int n0 = tile * C::TN + rg * NPG;
  const Buf md = make_buf(a.weights + sl.ref.down, F::bytes(H, I));
  Buf mats[NPG];
  int rows[NPG];
#pragma unroll
  for (int q = 0; q < NPG; ++q) {
    mats[q] = md;
    rows[q] = n0 + q;
  }
  const bool valid = n0 + NPG <= H;   // H is a multiple of NPG
  Stream<F, I, LPR, NPG, C::G> st;
  const int nt_all = uniform(sl.nt);
  for (int t0 = 0; t0 < nt_all; t0 += kNTB) {
    const int nb = nt_all - t0 < kNTB ? nt_all - t0 : kNTB;
    if (Stream<F, I, LPR, NPG, C::G>::P > 1 || t0 == 0) st.load(0, mats, rows, H, valid);   // kept for later rows
    if (!TAG || t0 > 0) __syncthreads();   // as in gateup_tile
    bool lost = false;   // a wait for h gave up: this tile's partials are NaN
    if constexpr (TAG) {
      // h comes from gate/up workgroups of the same launch: wait for its
      // tagged words, stage the values in LDS and take the row's largest
      // |h| from the same registers; every thread then derives sigma from
      // the four waves' maxima
      static_assert(kNTB == 1, "one h row at a time");
      float* hs = reinterpret_cast<float*>(lds + S::LDS_BYTES);
      // h overwrites the staged x row: a later gate/up item stages x again
      if (tid() == 0) g_xrow = -1;
      constexpr int PER = (I + kThreads - 1) / kThreads;
      const uint64_t* src = a.ht + static_cast<size_t>(sl.pair[t0]) * I;
      // a routed pair's mixing weight is published by the selection after
      // its ids: thread 0 polls it beside its share of h
      const uint64_t* wsrc = sl.expert >= 0 ? a.selt + (blockIdx.x % kSelRep) * kSelRepWords +
                                                  static_cast<size_t>(sl.pair[t0]) * kSelWords + 1
                                            : nullptr;
      uint32_t v[PER + 1];
      const bool got = await_batch<PER + 1>(
          [src, wsrc](int j) -> const uint64_t* {
            if (j == PER) return tid() == 0 ? wsrc : nullptr;
            const int i = tid() + j * kThreads;
            return i < I ? src + i : nullptr;
          },
          tag, a.err, v, a.spin_limit);
      // a routed entry's own weight is 0 (its word is not read with the
      // selection) or NaN (the worker's wait for the selection gave up):
      // adding it keeps the polled weight exact or poisons it
      if (tid() == 0) wrow = wsrc ? __builtin_bit_cast(float, v[PER]) + sl.w[t0] : sl.w[t0];
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = tid() + j * kThreads;
        if (i < I) {
          hs[i] = __builtin_bit_cast(float, v[j]);
          const uint32_t mag = v[j] & 0x7FFFFFFFu;
          m = m > mag ? m : mag;
        }
      }
      m = wave_max_u32(m);
      if ((tid() & 63) == 0) red[tid() >> 6] = m;
      lost = __syncthreads_or(!got);
      for (int w = 0; w < kThreads / 64; ++w) m = m > red[w] ? m : red[w];
      const int se = sigma_exp<F>(m);
      if (tid() == 0) inv_sigma[0] = __builtin_ldexpf(1.0f, -se);
      build_row_records<F, I, false, true>(hs, se, rec);
    } else {
      if (tid() < nb) srcs[tid()] = a.h + static_cast<size_t>(sl.pair[t0 + tid()]) * I;
      __syncthreads();
      for (int t = 0; t < nb; ++t) {
        const uint32_t m = row_max_bits<I, false, false>(srcs[t], red);
        if (tid() == 0) {
          sig_exp[t] = sigma_exp<F>(m);
          inv_sigma[t] = __builtin_ldexpf(1.0f, -sig_exp[t]);
        }
      }
      __syncthreads();
      build_records<F, I, false, false>(srcs, nb, sig_exp, rec, tid(), kThreads);
    }
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
          const float sc = lost ? __builtin_nanf("") : inv_sigma[t] * (TAG ? wrow : sl.w[t0 + t]);
#pragma unroll
          for (int q = 0; q < NPG; ++q) {
            const size_t o = static_cast<size_t>(sl.pair[t0 + t]) * H + n0 + q;
            if constexpr (TAG) tstore(a.part_t + o, tag, __builtin_bit_cast(uint32_t, acc[q][t] * sc));
            else a.part[o] = acc[q][t] * sc;
          }
        }
      }
    }
  }
}

// STAGE: 0 down, 1 gate/up from records, 2 gate/up staged locally.
// TAG: h is handed over as tagged words (fused launch).
template <class S, int STAGE, bool TAG = false>
__device__ __forceinline__ void run_slot(const Args& a, const SlotEntry& sl, int tile, uint8_t* lds, uint32_t tag = 0) {
#define MOE_RUN_FMT(FTAG, FT)                                                  \
  case FTAG:                                                                   \
    if constexpr (STAGE == 0) down_tile<S, FT, TAG>(a, sl, tile, lds, tag);    \
    else gateup_tile<S, FT, STAGE == 2, TAG>(a, sl, tile, lds, tag);           \
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
// chose it, every row's k entries in ascending id, then the shared expert's
// slot and the work-item offsets of both launches.  Run by wave 0; ids and
// weights come from LDS (ids[R*k], wv[R*k]).
template <class S>
__device__ __forceinline__ void build_slot_table(const Args& a, const int* ids, const float* wv, SlotTable* tab,
                                 bool write_order, const moe_expert_ref* eref = nullptr,
                                 const moe_expert_ref* shref = nullptr) {
  __shared__ int tg[kMaxSlots + 1], td[kMaxSlots + 1];
  const int lane = tid();
  const int n = a.R * a.k;
  // an id outside [0, E) names no expert: -1 is a pair the caller computes
  // elsewhere, anything else is invalid (the combine makes that row NaN);
  // neither reads the expert table
  const bool live = lane < n && ids[lane] >= 0 && ids[lane] < a.E;
  const int v = live ? ids[lane] : 0x7fffffff;
  bool first = live;
  int rank = 0;
  for (int m = 0; m < n; ++m) {
    const int vm = ids[m];
    if (m < lane && vm == v) first = false;
  }
  const uint64_t firsts = __ballot(first);
  for (int m = 0; m < n; ++m)
    if (((firsts >> m) & 1ull) && ids[m] < v) ++rank;
  const int n_active = __popcll(firsts);
  if (first) {
    SlotEntry& e = tab->e[rank];
    const moe_expert_ref ref = eref ? eref[lane] : a.experts[v];
    e.ref = ref;
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
    tg[rank] = tiles_of<S, true>(ref.fmt);
    td[rank] = tiles_of<S, false>(ref.fmt);
  }
  if (a.shared && lane < a.R) {
    SlotEntry& e = tab->e[n_active];
    if (lane == 0) {
      const moe_expert_ref ref = shref ? *shref : *a.shared;
      e.ref = ref;
      e.expert = -1;
      e.nt = a.R;
      tg[n_active] = a.shared_early ? 0 : tiles_of<S, true>(ref.fmt);
      td[n_active] = tiles_of<S, false>(ref.fmt);
    }
    e.row[lane] = lane;
    e.pair[lane] = n + lane;
    e.w[lane] = 1.0f;
  }
  if (write_order && lane < a.R) {
    const int* row = ids + lane * a.k;
    for (int j = 0; j < a.k; ++j) {   // position of entry j = number of smaller ids in the row
      int pos = 0;
      for (int q = 0; q < a.k; ++q) pos += row[q] < row[j] || (row[q] == row[j] && q < j);
      a.order[lane * a.k + pos] = j;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");  // LDS tile counts visible to lane 0
  if (lane == 0) {
    const int ns = n_active + (a.shared ? 1 : 0);
    int og = 0, od = 0;
    for (int q = 0; q < ns; ++q) {
      tab->gu_off[q] = og;
      tab->dn_off[q] = od;
      og += tg[q];
      od += td[q];
    }
    tab->gu_off[ns] = og;
    tab->dn_off[ns] = od;
    tab->n_active = n_active;
    tab->n_slots = ns;
    tab->n_gu = og;
    tab->n_dn = od;
  }
}

// The same table, built by wave 0 of a fused-launch worker straight from the
// published selection words (entry m: kSelWords words at ew + kSelWords * m,
// as the selection writes them).  Lane m holds pair m; which pairs repeat an
// expert, the rank of each distinct expert and the tile offsets before it
// come from cross-lane reads of registers, so the only LDS traffic is one
// read of the lane's entry and the table's stores: this runs between the
// selection and the first weight load of every worker.
template <class S>
__device__ __forceinline__ void slot_table_from_words(const Args& a, const uint32_t* ew, const moe_expert_ref& shref,
                                                      SlotTable* tab) {
  const int lane = tid();
  const int n = a.R * a.k;
  const bool act = lane < n;
  // the entry's words: id | fmt << 16, weight bits, then the 32-bit halves
  // of its gate, up and down offsets
  uint32_t q[kSelWords];
#pragma unroll
  for (int f = 0; f < kSelWords; ++f) q[f] = act ? ew[kSelWords * lane + f] : 0u;
  const int id = static_cast<int>(q[0] & 0xFFFFu);
  const uint32_t fmt = q[0] >> 16;
  // pairs of the same expert before this one (its position in the slot's
  // rows) and in all (the slot's row count); the loop is uniform over lanes
  int before = 0, same = 0;
  for (int j = 0; j < n; ++j) {
    const bool eq = __builtin_amdgcn_readlane(id, j) == id;
    same += eq ? 1 : 0;
    before += (eq && j < lane) ? 1 : 0;
  }
  const bool first = act && before == 0;
  const uint64_t firsts = __ballot(first);
  const int tg = first ? tiles_of<S, true>(fmt) : 0;
  const int td = first ? tiles_of<S, false>(fmt) : 0;
  // slot = number of distinct experts of lower id; its first items follow
  // the tiles of those experts
  int rank = 0, og = 0, od = 0, tot_g = 0, tot_d = 0;
  for (uint64_t m = firsts; m != 0; m &= m - 1) {
    const int j = __builtin_ctzll(m);
    const int gj = __builtin_amdgcn_readlane(tg, j), dj = __builtin_amdgcn_readlane(td, j);
    const bool lt = __builtin_amdgcn_readlane(id, j) < id;
    rank += lt ? 1 : 0;
    og += lt ? gj : 0;
    od += lt ? dj : 0;
    tot_g += gj;
    tot_d += dj;
  }
  const int n_active = __popcll(firsts);
  if (act && before < kMaxRows) {   // a lost selection names one expert n times: keep the first kMaxRows
    SlotEntry& e = tab->e[rank];
    e.row[before] = lane / a.k;
    e.pair[before] = lane;
    e.w[before] = __builtin_bit_cast(float, q[1]);
    if (first) {
      e.ref.fmt = fmt;
      e.ref.reserved = 0;
      e.ref.gate = (static_cast<uint64_t>(q[3]) << 32) | q[2];
      e.ref.up = (static_cast<uint64_t>(q[5]) << 32) | q[4];
      e.ref.down = (static_cast<uint64_t>(q[7]) << 32) | q[6];
      e.expert = id;
      e.nt = same < kMaxRows ? same : kMaxRows;
      tab->gu_off[rank] = og;
      tab->dn_off[rank] = od;
    }
  }
  if (a.shared && lane < a.R) {
    SlotEntry& e = tab->e[n_active];
    e.row[lane] = lane;
    e.pair[lane] = n + lane;
    e.w[lane] = 1.0f;
  }
  if (lane == 0) {
    int ng = tot_g, nd = tot_d;
    if (a.shared) {
      SlotEntry& e = tab->e[n_active];
      e.ref = shref;
      e.expert = -1;
      e.nt = a.R;
      tab->gu_off[n_active] = ng;
      tab->dn_off[n_active] = nd;
      ng += a.shared_early ? 0 : tiles_of<S, true>(shref.fmt);
      nd += tiles_of<S, false>(shref.fmt);
    }
    const int ns = n_active + (a.shared ? 1 : 0);
    tab->gu_off[ns] = ng;
    tab->dn_off[ns] = nd;
    tab->n_active = n_active;
    tab->n_slots = ns;
    tab->n_gu = ng;
    tab->n_dn = nd;
  }
}

// Activation records of every format for every row, built by kPrepWGs
// workgroups (p = 0 .. kPrepWGs-1).
template <class S, class F>
__device__ __forceinline__ void prep_format(const Args& a, int p, const int* sig_base) {
  constexpr int H = S::kH;
  const int fi = F::TAG - 1;
  __shared__ int sig_exp[kMaxRows];
  __shared__ const void* srcs[kMaxRows];
  if (tid() < a.R) {
    sig_exp[tid()] = sig_base[tid()] - F::PSHIFT;
    srcs[tid()] = a.x + static_cast<size_t>(tid()) * H;
    if (p == 0) a.xinv[fi * a.R + tid()] = __builtin_ldexpf(1.0f, -sig_exp[tid()]);
  }
  __syncthreads();
  // rows of this format are a.xrow apart; build_records strides rows by the
  // format's own record row, so build one row at a time
  for (int r = 0; r < a.R; ++r)
    build_records<F, H, true>(srcs + r, 1, sig_exp + r, a.xrec + (static_cast<size_t>(fi) * a.R + r) * a.xrow,
                              p * kThreads + tid(), kPrepWGs * kThreads);
}

template <class S>
__device__ __forceinline__ void prep_wg(const Args& a, int p) {
  __shared__ uint32_t red[16];
  __shared__ int base[kMaxRows];
  for (int r = 0; r < a.R; ++r) {
    const uint32_t m = row_max_bits<S::kH, true>(a.x + static_cast<size_t>(r) * S::kH, red);
    if (tid() == 0) base[r] = m ? 14 - (static_cast<int>(m >> 23) - 127) : 14;
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
__device__ __forceinline__ void router_wg(const Args& a, int e, double* red, uint32_t tag = 0) {
  constexpr int CH = (H / 4 + kThreads - 1) / kThreads;   // float4 chunks per thread
  double acc[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.0;
  const float4* wr = reinterpret_cast<const float4*>(a.w_router + static_cast<size_t>(e) * H);
  float4 w[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = tid() + i * kThreads;
    w[i] = j < H / 4 ? wr[j] : float4{0.f, 0.f, 0.f, 0.f};
  }
  // the x rows of a group are all requested before any is used: one round
  // trip per group of kXG rows, not one per row
  constexpr int kXG = 4;
#pragma unroll
  for (int r0 = 0; r0 < kMaxRows; r0 += kXG) {
    if (r0 < a.R) {
      uint2 xb[kXG][CH];
#pragma unroll
      for (int g = 0; g < kXG; ++g)
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int j = tid() + i * kThreads;
          xb[g][i] = (r0 + g < a.R && j < H / 4)
                         ? *reinterpret_cast<const uint2*>(a.x + static_cast<size_t>(r0 + g) * H + 4 * j)
                         : uint2{0u, 0u};
        }
#pragma unroll
      for (int g = 0; g < kXG; ++g) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          s = fma(static_cast<double>(w[i].x), static_cast<double>(bf16_bits_to_f32(xb[g][i].x & 0xFFFFu)), s);
          s = fma(static_cast<double>(w[i].y), static_cast<double>(bf16_bits_to_f32(xb[g][i].x >> 16)), s);
          s = fma(static_cast<double>(w[i].z), static_cast<double>(bf16_bits_to_f32(xb[g][i].y & 0xFFFFu)), s);
          s = fma(static_cast<double>(w[i].w), static_cast<double>(bf16_bits_to_f32(xb[g][i].y >> 16)), s);
        }
        acc[r0 + g] = s;
      }
    }
  }
  const int wave = tid() >> 6, lane = tid() & 63, nw = kThreads / 64;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    if (r < a.R) {
      const double s = wave_sum_f64(acc[r]);
      if (lane == 0) red[r * 16 + wave] = s;
    }
  }
  __syncthreads();
  if (tid() < a.R) {
    double s = 0.0;
    for (int w = 0; w < nw; ++w) s += red[tid() * 16 + w];
    const size_t o = static_cast<size_t>(tid()) * a.E + e;
    if (a.lgt) {   // fused launch: publish as two tagged halves
      const uint64_t b = __builtin_bit_cast(uint64_t, s);
      tstore(a.lgt + 2 * o, tag, static_cast<uint32_t>(b));
      tstore(a.lgt + 2 * o + 1, tag, static_cast<uint32_t>(b >> 32));
    } else {
      a.logits[o] = s;
    }
  }
}

// Top-k of one row by key = logit + bias, ties to the lower id; weights are
// the softmax of the unbiased logits over the selection.  One wave per row,
// given the lane's logits (lv) and biases of experts lane + 64 q.  Each of
// the k rounds takes the wave's largest key (f64 max over DPP), then the
// lowest id holding it (ballots), and retires that entry.
__device__ __forceinline__ void select_core(const Args& a, int r, const double (&lv)[kSelQ],
                                           const float (&bias)[kSelQ], int* sel, float* wsel, uint32_t tag,
                                           const moe_expert_ref* refs, bool lost = false);

// The lane's share of the selection-only bias (0 where there is none).
__device__ __forceinline__ void load_bias(const Args& a, float (&bias)[kSelQ]) {
  const int lane = tid() & 63;
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    const int e = lane + 64 * q;
    bias[q] = (a.bias && e < a.E) ? a.bias[e] : 0.0f;
  }
}

__device__ __forceinline__ void select_row(const Args& a, int r, int* sel, float* wsel) {
  const int lane = tid() & 63;
  float bias[kSelQ];
  load_bias(a, bias);
  const double* lg = a.logits + static_cast<size_t>(r) * a.E;
  double lv[kSelQ];
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    const int e = lane + 64 * q;
    lv[q] = e < a.E ? lg[e] : 0.0;
  }
  select_core(a, r, lv, bias, sel, wsel, 0, nullptr);
}

// The fused launch: the row's logits arrive as tagged halves from the router
// workgroups of the same launch.
__device__ __forceinline__ void select_row_tagged(const Args& a, int r, int* sel, float* wsel, uint32_t tag,
                                  const moe_expert_ref* refs) {
  const int lane = tid() & 63;
  const uint64_t* lg = a.lgt + static_cast<size_t>(r) * a.E * 2;
  float bias[kSelQ];   // loaded before the wait, off the critical path
  load_bias(a, bias);
  uint32_t half[2 * kSelQ];
  const bool got = await_batch<2 * kSelQ>(
      [lg, lane, E = a.E](int j) -> const uint64_t* {
        const int e = lane + 64 * (j >> 1);
        return e < E ? lg + 2 * e + (j & 1) : nullptr;
      },
      tag, a.err, half, a.spin_limit);
  if (r == 0 && a.selt && lane < kSelRep) tstore(a.selt + lane * kSelRepWords + kSelEntryWords, tag, 1u);
  double lv[kSelQ];
#pragma unroll
  for (int q = 0; q < kSelQ; ++q)
    lv[q] = __builtin_bit_cast(double, (static_cast<uint64_t>(half[2 * q + 1]) << 32) | half[2 * q]);
  // a wait that gave up leaves stale halves: the ids still name real experts,
  // but their weights are NaN, so nothing downstream looks valid
  select_core(a, r, lv, bias, sel, wsel, tag, refs, __ballot(!got) != 0);
}

__device__ __forceinline__ void select_core(const Args& a, int r, const double (&lv)[kSelQ],
                                           const float (&bias)[kSelQ], int* sel, float* wsel, uint32_t tag,
                                           const moe_expert_ref* refs, bool lost) {
  const int lane = tid() & 63;
  // selection keys: the double key mapped to an unsigned 64-bit integer of
  // the same order (a NaN key of a real expert counts as -inf, -0 as +0),
  // held as 32-bit halves.  Every real key has a nonzero upper half, so 0
  // marks an entry past E or already taken.
  uint32_t kh[kSelQ], kl[kSelQ];
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    const int e = lane + 64 * q;
    double key = (lv[q] + static_cast<double>(bias[q])) + 0.0;   // -0 -> +0
    key = key == key ? key : -INFINITY;
    uint64_t b = __builtin_bit_cast(uint64_t, key);
    b = (b >> 63) ? ~b : (b | (1ull << 63));
    kh[q] = e < a.E ? static_cast<uint32_t>(b >> 32) : 0u;
    kl[q] = e < a.E ? static_cast<uint32_t>(b) : 0u;
  }
  int my_id = 0;         // lane j ends with the j-th selection
  for (int j = 0; j < a.k; ++j) {
    // the largest upper half; only when several entries share it do the
    // lower halves of those entries decide
    uint32_t mh = kh[0];
#pragma unroll
    for (int q = 1; q < kSelQ; ++q) mh = mh > kh[q] ? mh : kh[q];
    mh = wave_max_u32(mh);
    uint64_t bq[kSelQ];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kSelQ; ++q) {
      bq[q] = __ballot(kh[q] == mh);
      cnt += __popcll(bq[q]);
    }
    if (cnt > 1) {
      uint32_t ml = 0;
#pragma unroll
      for (int q = 0; q < kSelQ; ++q) {
        const uint32_t v = kh[q] == mh ? kl[q] : 0u;
        ml = ml > v ? ml : v;
      }
      ml = wave_max_u32(ml);
#pragma unroll
      for (int q = 0; q < kSelQ; ++q) bq[q] = __ballot(kh[q] == mh && kl[q] == ml);
    }
    // the lowest id holding the maximum: the lowest q with a match, then the
    // lowest lane of it (ids are lane + 64 q)
    uint64_t bm = 0;
    int wq = 0;
#pragma unroll
    for (int q = kSelQ - 1; q >= 0; --q) {
      wq = bq[q] ? q : wq;
      bm = bq[q] ? bq[q] : bm;
    }
    const int owner = static_cast<int>(__builtin_ctzll(bm));
#pragma unroll
    for (int q = 0; q < kSelQ; ++q) kh[q] = (q == wq && lane == owner) ? 0u : kh[q];   // taken
    my_id = lane == j ? owner + 64 * wq : my_id;
  }
  // fused launch: entry j of the row is 8 words (id | fmt << 16, weight
  // bits, then the 32-bit halves of its gate, up and down offsets); lane L
  // writes word L & 7 of entry L >> 3 into every copy.  Everything but the
  // weight goes out now: the gate/up items need only ids and offsets, and
  // the weight (below, after the softmax) is read by the down items.
  const int nw_sel = a.k * kSelWords, ent = lane >> 3, fld = lane & 7;
  const int id_e = __shfl(my_id, ent, 64);
  uint64_t* sel_o = a.selt ? a.selt + static_cast<size_t>(r) * nw_sel + lane : nullptr;
  if (a.selt && lane < nw_sel && fld != 1) {
    const uint32_t* f = reinterpret_cast<const uint32_t*>(refs + id_e);   // fmt, reserved, gate, up, down
    const uint32_t v = fld == 0 ? (static_cast<uint32_t>(id_e) | (f[0] << 16)) : f[fld];
#pragma unroll
    for (int c = 0; c < kSelRep; ++c) tstore(sel_o + c * kSelRepWords, tag, v);
  }
  // the unbiased logit of each lane's selection, fetched from the lane that
  // holds it, then the softmax over the selection: one exp per lane, the max
  // and the sum gathered from the k lanes
  double my_l = 0.0;
  {
    const int oq = my_id >> 6, ol = my_id & 63;
#pragma unroll
    for (int q = 0; q < kSelQ; ++q) {
      const double v = __shfl(lv[q], ol, 64);
      my_l = oq == q ? v : my_l;
    }
  }
  double lmax = -INFINITY;
  for (int j = 0; j < a.k; ++j) {
    const uint64_t lb = __builtin_bit_cast(uint64_t, my_l);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(lb), j);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(lb >> 32), j);
    const double v = __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
    lmax = v > lmax ? v : lmax;
  }
  const double e = lane < a.k ? exp(my_l - lmax) : 0.0;
  double s = 0.0;
  for (int j = 0; j < a.k; ++j) {
    const uint64_t eb = __builtin_bit_cast(uint64_t, e);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(eb), j);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(eb >> 32), j);
    s += __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
  }
  const float w = lost ? __builtin_nanf("") : static_cast<float>(e / s);
  if (lane < a.k) {
    sel[lane] = my_id;
    wsel[lane] = w;
    a.idx[r * a.k + lane] = my_id;
    a.wts[r * a.k + lane] = w;
  }
  if (a.selt) {
    const uint32_t w_e = __shfl(__builtin_bit_cast(uint32_t, w), ent, 64);
    if (lane < nw_sel && fld == 1) {
#pragma unroll
      for (int c = 0; c < kSelRep; ++c) tstore(sel_o + c * kSelRepWords, tag, w_e);
    }
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// route: router workgroups [0, E) write logits; record builders
// [E, E + kPrepWGs) build the activation records of every format; in
// moe_layer, the shared expert's gate/up tiles follow (they need only x, so
// their weights stream while the router runs; records are built locally).
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_route(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int bid = blockIdx.x;
  if (bid < a.E) {
    __shared__ double red[kMaxRows * 16];
    router_wg<S::kH>(a, bid, red);
    return;
  }
  if (bid < a.E + kPrepWGs) {
    prep_wg<S>(a, bid - a.E);
    return;
  }
  __shared__ SlotEntry se;
  const int tile = bid - a.E - kPrepWGs;
  if (tid() == 0) {
    se.ref = *a.shared;
    se.expert = -1;
    se.nt = a.R;
    for (int r = 0; r < a.R; ++r) {
      se.row[r] = r;
      se.pair[r] = a.R * a.k + r;
      se.w[r] = 1.0f;
    }
  }
  __syncthreads();
  if (tile < tiles_of<S, true>(se.ref.fmt)) run_slot<S, 2>(a, se, tile, lds);
}

// select: one workgroup picks the top-k of every row and builds the slot
// table and the work lists.
template <class S>
__global__ __launch_bounds__(kThreads) void k_select(Args a) {
  __shared__ int sel[kMaxRows * kMaxK];
  __shared__ float wsel[kMaxRows * kMaxK];
  for (int r = tid() >> 6; r < a.R; r += kThreads / 64)
    select_row(a, r, sel + r * a.k, wsel + r * a.k);
  __syncthreads();
  if (a.experts && tid() < 64) build_slot_table<S>(a, sel, wsel, a.slots, true);
}

// Preparation for a caller-given routing: slot table (workgroup 0) and
// activation records (workgroups 1 .. kPrepWGs).
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_prep(Args a) {
  if (blockIdx.x == 0) {
    __shared__ int ids[kMaxRows * kMaxK];
    __shared__ float wv[kMaxRows * kMaxK];
    for (int i = tid(); i < a.R * a.k; i += kThreads) {
      ids[i] = a.idx[i];
      wv[i] = a.wts[i];
    }
    __syncthreads();
    if (tid() < 64) build_slot_table<S>(a, ids, wv, a.slots, true);
    return;
  }
  prep_wg<S>(a, blockIdx.x - 1);
}

// One work item: the slot whose range [offs[slot], offs[slot + 1]) holds it
// (offs in LDS; binary search over at most 65 slots), its entry copied to
// LDS, then that slot's tile.  Ends with a barrier: LDS and the slot entry
// are reused by the next item.
template <class S, int STAGE, bool TAG>
__device__ __forceinline__ void run_item(const Args& a, const SlotTable* tab, const int* offs, int ns, int item,
                                         SlotEntry& sl, uint8_t* lds, uint32_t tag) {
  int lo = 0, hi = ns - 1;             // largest slot with offs[slot] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  const int slot = lo, tile = item - offs[lo];
  if (tid() < static_cast<int>(sizeof(SlotEntry) / 4))
    reinterpret_cast<uint32_t*>(&sl)[tid()] = reinterpret_cast<const uint32_t*>(&tab->e[slot])[tid()];
  __syncthreads();
  run_slot<S, STAGE, TAG>(a, sl, tile, lds, tag);
  __syncthreads();
}

// One work item of the fused launch: the table is in this workgroup's LDS
// for the whole call, so the slot's entry is used in place.  The slot is the
// number of slot starts at or below the item, counted with ballots over one
// LDS read per lane (at most kMaxSlots + 1 slots).
template <class S, int STAGE>
__device__ __forceinline__ void run_item_fused(const Args& a, const SlotTable& tab, const int* offs, int ns, int item,
                                               uint8_t* lds, uint32_t tag) {
  static_assert(kMaxSlots + 1 <= 128, "two offsets a lane");
  const int lane = tid() & 63;
  const int o0 = lane < ns ? offs[lane] : 0x7fffffff;
  const int o1 = lane + 64 < ns ? offs[lane + 64] : 0x7fffffff;
  const int slot = __popcll(__ballot(o0 <= item)) + __popcll(__ballot(o1 <= item)) - 1;
  const int start = slot < 64 ? __builtin_amdgcn_readlane(o0, slot) : __builtin_amdgcn_readlane(o1, slot - 64);
  run_slot<S, STAGE, true>(a, tab.e[slot], item - start, lds, tag);
  __syncthreads();
}

// Work items of one list, strided over `nw` workers (this is worker w).
// STAGE as in run_slot; the list is the down list for STAGE 0, else the
// gate/up list.
template <class S, int STAGE, bool TAG>
__device__ __forceinline__ void run_items(const Args& a, const SlotTable* tab, int w, int nw, uint8_t* lds,
                          uint32_t tag = 0) {
  __shared__ SlotEntry sl;
  __shared__ int offs[kMaxSlots + 2];
  const int ns = uniform(tab->n_slots);
  const int* off_g = STAGE == 0 ? tab->dn_off : tab->gu_off;
  const int n_items = uniform(off_g[ns]);
  if (w >= n_items) return;
  for (int i = tid(); i <= ns; i += kThreads) offs[i] = off_g[i];
  __syncthreads();
  for (int item = w; item < n_items; item += nw) run_item<S, STAGE, TAG>(a, tab, offs, ns, item, sl, lds, tag);
}

// gateup: h = silu(W_gate x) * (W_up x) for every (slot, tile) item.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_gateup(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  run_items<S, 1, false>(a, a.slots, blockIdx.x, gridDim.x, lds);
}

// down: w * (W_down h) into the partials for every (slot, tile) item.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_down(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  run_items<S, 0, false>(a, a.slots, blockIdx.x, gridDim.x, lds);
}

// The bf16 (round to nearest even) bits of v.
__device__ __forceinline__ uint16_t bf16_rne(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = (u & 0x7FFFFFFFu) > 0x7F800000u ? (u | 0x00400000u) : u + 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// The power of two 2^s that bounds a row of the next layer's input (s = 0 if
// the row's largest |v| is below 4 or the row holds a NaN or an infinity).
__device__ __forceinline__ int chain_shift(float m, bool odd) {
  return (!odd && m >= 4.0f) ? ilogbf(m) - 1 : 0;
}

// Output element i = (r, n) of the fused launch: the row's k partials in
// ascending expert id (ids from the published selection), then the shared
// expert; every input is a tagged word of this call.  A call in which a
// hand-off wait gave up yields NaN (as far as this element can tell).
// Called by every thread of a combine workgroup (kThreads consecutive
// elements of one row, since H is a multiple of kThreads).  In a stack decode
// it also writes the next layer's input, x = bf16(v / 2^s), v = y + noise,
// with s from the row's largest |v|: each workgroup publishes its share of
// that maximum as a tagged word and reads its row's others.
template <class S>
__device__ __forceinline__ void combine_out(const Args& a, int i, uint32_t tag) {
  static_assert(S::kH % kThreads == 0, "a combine workgroup lies in one row");
  if (i >= a.R * S::kH) return;   // whole workgroups: the grid covers R * H exactly
  const int r = i / S::kH, n = i - r * S::kH;
  const int k = a.k;
  // the pairs' ids (published long before), then the partials and the shared
  // expert's partial with two polls in flight; partial words a call does not
  // use read the first id word and are not waited for
  uint32_t wid[kMaxK], wp[kMaxK + 1];
  const bool got_id = await_batch<kMaxK>(
      [sel = a.selt, r, k](int j) -> const uint64_t* { return j < k ? sel + kSelWords * (r * k + j) : nullptr; },
      tag, a.err, wid, a.spin_limit);
  const bool has_sh = a.shared != nullptr;
  uint32_t need = has_sh ? 1u << kMaxK : 0u;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) need |= j < k ? 1u << j : 0u;
  const bool got_p = await_batch2<kMaxK + 1>(
      [sel = a.selt, part = a.part_t, r, n, k, sh = has_sh, R = a.R](int q) -> const uint64_t* {
        if (q < k) return part + static_cast<size_t>(r * k + q) * S::kH + n;
        return (q == kMaxK && sh) ? part + static_cast<size_t>(R * k + r) * S::kH + n : sel;
      },
      need, tag, a.err, wp, a.spin_limit);
  const bool got = got_id && got_p;
  int id[kMaxK], rank[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) id[j] = j < k ? static_cast<int>(wid[j] & 0xFFFFu) : 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rank[j] = 0;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q) rank[j] += id[q] < id[j];
  }
  float s = 0.0f;
#pragma unroll
  for (int pos = 0; pos < kMaxK; ++pos) {
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) t = rank[j] == pos ? __builtin_bit_cast(float, wp[j]) : t;
    if (pos < k) s += t;
  }
  if (a.shared) s += __builtin_bit_cast(float, wp[kMaxK]);
  if (!got || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) s = __builtin_nanf("");
  a.y[i] = s;
  if (!a.x_next) return;
  constexpr int NC = S::kH / kThreads;   // combine workgroups per row
  const float v = a.noise ? s + a.noise[i] : s;
  const float av = __builtin_fabsf(v);
  bool odd = !(av <= 3.4028234663852886e38f);
  float m = odd ? 0.0f : av;
  for (int o = 32; o > 0; o >>= 1) {
    const float t = __shfl_xor(m, o, 64);
    m = t > m ? t : m;
  }
  odd = __ballot(odd) != 0;
  __shared__ float wm[kThreads / 64];
  __shared__ int wodd[kThreads / 64];
  __shared__ int shift;
  if ((tid() & 63) == 0) {
    wm[tid() >> 6] = m;
    wodd[tid() >> 6] = odd ? 1 : 0;
  }
  __syncthreads();
  if (tid() < 64) {
    float mm = 0.0f;
    int bad = 0;
    for (int q = 0; q < kThreads / 64; ++q) {
      mm = wm[q] > mm ? wm[q] : mm;
      bad |= wodd[q];
    }
    // this workgroup's share: the maximum's bits, or a NaN pattern for a row
    // holding a NaN or an infinity
    uint64_t* row = a.rmax_t + static_cast<size_t>(r) * NC;
    if (tid() == 0) tstore(row + n / kThreads, tag, bad ? 0x7FC00000u : __builtin_bit_cast(uint32_t, mm));
    uint32_t pv[1];
    const int lane = tid();
    const bool got_all = __ballot(!await_batch<1>([row, lane](int) -> const uint64_t* {
                                                    return lane < NC ? row + lane : nullptr;
                                                  },
                                                  tag, a.err, pv, a.spin_limit)) == 0;
    const float pm = __builtin_bit_cast(float, pv[0]);
    const bool podd = lane < NC && !(pm <= 3.4028234663852886e38f);
    float rm = lane < NC && !podd ? pm : 0.0f;
    for (int o = 32; o > 0; o >>= 1) {
      const float t = __shfl_xor(rm, o, 64);
      rm = t > rm ? t : rm;
    }
    // a wait that gave up leaves the row's bound unknown: its x is NaN
    if (tid() == 0) shift = got_all ? chain_shift(rm, __ballot(podd) != 0) : 0x7fffffff;
  }
  __syncthreads();
  const int sh = shift;
  a.x_next[i] = sh == 0x7fffffff ? static_cast<uint16_t>(0x7FC0u) : bf16_rne(__builtin_ldexpf(v, -sh));
}

// ---------------------------------------------------------------------------
// fused layer: one launch, workgroup roles in dependency order
// ---------------------------------------------------------------------------
// [0, E)              router GEMV, logits published as tagged words
// [E, E + R)          selection of row blockIdx - E (one wave), published tagged
// [base_b, base_y)    workers over one list of items: the shared expert's
//                     gate/up tiles (they need only x and stream while the
//                     selection is made), the routed gate/up (slot, tile)
//                     items, then the down items, routed and shared
// [base_y, ...)       combine: one output element per thread
// Every role waits only on roles with lower workgroup ids, which the
// dispatcher has started before it, so the waits always end; the workers
// build the slot table themselves from the published selection.  Down
// workers issue their weight loads before they wait for h.
template <class S>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_layer(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int bid = blockIdx.x;
  const uint32_t tag = a.tag;
  if (bid < a.E) {
    __shared__ double red[kMaxRows * 16];
    router_wg<S::kH>(a, bid, red, tag);
    return;
  }
  if (bid < a.E + a.R) {
    __shared__ int sel[kMaxK];
    __shared__ float wsel[kMaxK];
    // the expert table goes to LDS while the router still runs, so the
    // published entries carry their matrices without another round trip
    // the selection is on every routed expert's critical path: its wave goes
    // first among the waves sharing the SIMD
    __builtin_amdgcn_s_setprio(3);
    moe_expert_ref* refs = reinterpret_cast<moe_expert_ref*>(lds);
    for (int i = tid(); i < a.E * 4; i += kThreads)
      reinterpret_cast<uint64_t*>(refs)[i] = reinterpret_cast<const uint64_t*>(a.experts)[i];
    __syncthreads();
    if (tid() < 64) select_row_tagged(a, bid - a.E, sel, wsel, tag, refs);
    return;
  }
  if (bid >= a.base_y) {
    combine_out<S>(a, (bid - a.base_y) * kThreads + tid(), tag);
    return;
  }
  // workers.  Worker w takes items w, w + nw, ... of one list: the shared
  // expert's gate/up tiles, then the routed gate/up items, then the down
  // items (routed and shared).  A down item waits only for gate/up items,
  // which come earlier in the list, so the worker holding them has done them
  // or runs them (every worker is started: the roles before the workers never
  // wait on them); its weights are in flight while it waits for h.
  // The shared expert's table entry is read once, at the start, and kept in
  // LDS: nothing after the selection waits on a global load that could sit
  // behind the weight traffic.
  const int w = bid - a.base_b, nw = a.nb;
  __shared__ SlotTable tab;
  __shared__ moe_expert_ref shref;
  __shared__ SlotEntry sl;
  if (tid() == 0 && a.shared) shref = *a.shared;
  for (int i = tid(); i < 256; i += kThreads)
    reinterpret_cast<uint32_t*>(lds + S::LDS_REC)[i] = FmtTern::table_entry(i);
  stage_x_row<S>(a, 0, lds);   // before any wait: every gate/up item of row 0 finds x here

  const int nsh = a.shared ? uniform(tiles_of<S, true>(shref.fmt)) : 0;
  // workers taking the shared gate/up tiles: one tile each, but at one row a
  // tile is cheap and two each leave more workers free for the routed items
  // when the selection comes out (a.nsw caps it)
  const int nsw_want = a.R == 1 ? (nsh + 1) / 2 : nsh;
  const int nsw = a.nsw < nsw_want ? a.nsw : nsw_want;
  if (w < nsw) {
    // shared gate/up tiles need only x: they stream while the selection is
    // made.  At one row they wait until the selection has every logit, so
    // neither the router's loads nor the selection's poll queue behind this
    // traffic; with more rows the tiles are long enough that starting at
    // once is worth more.
    if (tid() == 0) {
      sl.ref = shref;
      sl.expert = -1;
      sl.nt = a.R;
      for (int r = 0; r < a.R; ++r) {
        sl.row[r] = r;
        sl.pair[r] = a.R * a.k + r;
        sl.w[r] = 1.0f;
      }
      if (a.R == 1) (void)await_word(a.selt + (w % kSelRep) * kSelRepWords + kSelEntryWords, tag, a.err, a.spin_limit);
    }
    __syncthreads();
    for (int t = w; t < nsh; t += nsw) {
      run_slot<S, 2, true>(a, sl, t, lds, tag);
      __syncthreads();   // LDS is reused next
    }
  }
  // the selection of every row, then the slot table in LDS; the selection's
  // staging shares the dynamic region with the tiles' records
  uint32_t* ew = reinterpret_cast<uint32_t*>(lds + S::LDS_SEL_OFF);
  const int n = a.R * a.k;
  // One wave polls the whole selection, a few words a lane: a thousand
  // workgroups polling with every lane would hammer the same lines, and a
  // single-word poll followed by a full read would cost a second round trip
  // once the selection is there
  if (tid() < 64) {
    constexpr int PER = kSelEntryWords / 64;
    const int lane = tid();
    uint32_t v[PER];
    const uint64_t* selt = a.selt + (bid % kSelRep) * kSelRepWords;
    const int lim = n * kSelWords;
    bool got;   // two polls in flight: this wave has nothing else out
    if (lim <= 64) {
      // one word a lane (a row's whole selection)
      static_assert(kSelEntryWords >= 64, "every lane's word lies in the entry area");
      uint32_t v1[1];
      got = await_batch2<1>([selt, lane](int) { return selt + lane; },
                            lane < lim && (lane & (kSelWords - 1)) != 1 ? 1u : 0u,   // weights come later
                            tag, a.err, v1, a.spin_limit);
      v[0] = v1[0];
#pragma unroll
      for (int j = 1; j < PER; ++j) v[j] = 0;
    } else {
      uint32_t need = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = lane + j * 64;
        need |= i < lim && (i & (kSelWords - 1)) != 1 ? 1u << j : 0u;
      }
      got = await_batch2<PER>([selt, lane](int j) { return selt + lane + j * 64; }, need, tag, a.err, v,
                              a.spin_limit);
    }
    // a wait that gave up leaves stale words, whose offsets could lie outside
    // this call's weights: every entry then names expert 0 with weight NaN,
    // so nothing below reads through them and every partial it makes is NaN
    if (__ballot(!got) == 0) {
#pragma unroll
      for (int j = 0; j < PER; ++j) ew[lane + j * 64] = v[j];
    } else {
      const uint32_t* e0 = reinterpret_cast<const uint32_t*>(a.experts);   // fmt, reserved, gate, up, down
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = lane + j * 64, f = i % kSelWords;
        ew[i] = f == 0 ? e0[0] << 16 : f == 1 ? 0x7FC00000u : e0[f];
      }
    }
    // the words just stored are read back by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // every wave of this workgroup waits for the table, and the waves it
    // shares its SIMD with are decoding: it goes first meanwhile
    __builtin_amdgcn_s_setprio(3);
    slot_table_from_words<S>(a, ew, shref, &tab);
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  const int ns = uniform(tab.n_slots);
  const int n_gu = uniform(tab.n_gu), n_dn = uniform(tab.n_dn);
  // At one row the down list is taken from the shared expert's tiles on
  // (they are the list's last, from n_dn - sh_dn): its h is ready long
  // before the routed ones, so its weights stream while the routed gate/up
  // items are still finishing; the routed slots follow in list order.
  const int sh_dn = a.shared ? uniform(tab.dn_off[ns] - tab.dn_off[ns - 1]) : 0;
  // The routed list starts at worker nsw: the workers holding shared tiles
  // get its later positions, so the routed gate/up items start on free
  // workers as soon as the selection is out.
  //
  // With several rows the shared expert's down tiles go to the shared
  // workers first (its h comes from their own gate/up tiles, done by then):
  // worker w < nsw takes shared down tiles w, w + nsw, ... before its list
  // positions, and the list holds only the routed down items.
  const int pre = (a.R > 1 && w < nsw && w < sh_dn) ? (sh_dn - 1 - w) / nsw + 1 : 0;
  const int n_list = a.R > 1 ? n_gu + n_dn - sh_dn : n_gu + n_dn;
  const int dn_first = a.R > 1 ? 0 : n_dn - sh_dn;
  const int j0 = (w - nsw + nw) % nw;
  for (int q = 0;; ++q) {
    const int j = q < pre ? -1 : j0 + (q - pre) * nw;
    if (j >= n_list) break;
    const bool gu = j >= 0 && j < n_gu;
    const int item = gu ? j : j < 0 ? n_dn - sh_dn + w + q * nsw : (j - n_gu + dn_first) % n_dn;
    if (gu) run_item_fused<S, 2>(a, tab, tab.gu_off, ns, item, lds, tag);
    else run_item_fused<S, 0>(a, tab, tab.dn_off, ns, item, lds, tag);
  }
}

// Combine: y[r] = sum over the row's experts in ascending id, then the shared
// expert -- a fixed order, so y is bitwise reproducible.
template <class S>
__global__ __launch_bounds__(kThreads) void k_combine(Args a) {
  const int i = blockIdx.x * kThreads + tid();
  if (i >= a.R * S::kH) return;
  const int r = i / S::kH, n = i - r * S::kH;
  float s = 0.0f;
  bool bad = false;
  for (int j = 0; j < a.k; ++j) {
    const int q = a.order[r * a.k + j];
    const int e = a.idx[r * a.k + q];
    if (e == -1) continue;   // computed by the caller elsewhere: contributes nothing here
    bad = bad || e < -1 || e >= a.E;
    if (e >= 0 && e < a.E) s += a.part[static_cast<size_t>(r * a.k + q) * S::kH + n];
  }
  if (a.shared) s += a.part[static_cast<size_t>(a.R * a.k + r) * S::kH + n];
  a.y[i] = bad ? __builtin_nanf("") : s;
}

// The end of a layer step, one workgroup per row of H: y += add (when
// given); then, when x_next is given, the next layer's input: v = y + noise
// (one fp32 addition), divided by 2^s when the row's largest |v| is 4 or more
// (s = floor(log2 max|v|) - 1 brings it into [2, 4); s = 0 if the row holds a
// NaN or an infinity), rounded to bf16 (nearest even).  A power of two keeps
// the step exact and its decision free of summation order.
__global__ __launch_bounds__(kThreads) void k_chain_rows(float* y, const float* add, const float* noise,
                                                         uint16_t* x_next, int H) {
  const size_t base = static_cast<size_t>(blockIdx.x) * H;
  float* yr = y + base;
  float m = 0.0f;
  bool odd = false;   // a NaN or an infinity in the row
  for (int i = tid(); i < H; i += kThreads) {
    float v = yr[i];
    if (add) {
      v += add[base + i];
      yr[i] = v;
    }
    if (x_next) {
      if (noise) v += noise[base + i];
      const float av = __builtin_fabsf(v);
      odd = odd || !(av <= 3.4028234663852886e38f);
      m = av > m ? av : m;
    }
  }
  if (!x_next) return;
  __shared__ float wm[kThreads / 64];
  __shared__ int wodd[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) {
    const float t = __shfl_xor(m, o, 64);
    m = t > m ? t : m;
  }
  const bool any_odd = __ballot(odd) != 0;
  if ((tid() & 63) == 0) {
    wm[tid() >> 6] = m;
    wodd[tid() >> 6] = any_odd ? 1 : 0;
  }
  __syncthreads();
  float mm = 0.0f;
  int bad = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    mm = wm[w] > mm ? wm[w] : mm;
    bad |= wodd[w];
  }
  const int sh = chain_shift(mm, bad != 0);
  for (int i = tid(); i < H; i += kThreads) {
    float v = yr[i];
    if (noise) v += noise[base + i];
    x_next[base + i] = bf16_rne(__builtin_ldexpf(v, -sh));
  }
}

// ---------------------------------------------------------------------------
// many-row generic path: the decode tiles over entries of at most kGenRows
// pairs of one expert (any format, and the shared expert), h in fp32
// ---------------------------------------------------------------------------
// Exclusive prefix sum of v over the workgroup's threads in thread order;
// *total gets the sum of all.  tmp: kThreads ints of LDS.
__device__ __forceinline__ int wg_scan(int v, int* tmp, int* total) {
  const int t = tid();
  tmp[t] = v;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int add = t >= o ? tmp[t - o] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int incl = tmp[t];
  *total = tmp[kThreads - 1];
  __syncthreads();
  return incl - v;
}

// Plan (one workgroup): the generic entries of every routed expert in
// ascending id (those the matrix cores do not take), each with the offsets of
// its first gate/up and down items, then the shared expert's entries; counts
// in gen_n.  Thread t handles experts 2t and 2t + 1 (E <= 2 * kThreads).
template <class S>
__global__ __launch_bounds__(kThreads) void k_gen_plan(Args a) {
  static_assert(lay::kMaxExperts <= 2 * kThreads, "two experts per thread");
  __shared__ int tmp[kThreads];
  constexpr int G = lay::kGenRows;
  const int t = tid();
  int c[2], n[2], tg[2], td[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = 2 * t + j;
    c[j] = e < a.E ? a.cnt[e] : 0;
    const uint32_t fmt = e < a.E ? a.experts[e].fmt : 0u;
    const bool gen = c[j] > 0 && !(a.mfma && fmt == MOE_FMT_MXFP4);
    n[j] = gen ? (c[j] + G - 1) / G : 0;
    tg[j] = tiles_of<S, true>(fmt);
    td[j] = tiles_of<S, false>(fmt);
  }
  int tot_c, tot_n, tot_g, tot_d;
  const int off_c = wg_scan(c[0] + c[1], tmp, &tot_c);
  const int off_n = wg_scan(n[0] + n[1], tmp, &tot_n);
  const int off_g = wg_scan(n[0] * tg[0] + n[1] * tg[1], tmp, &tot_g);
  const int off_d = wg_scan(n[0] * td[0] + n[1] * td[1], tmp, &tot_d);
  int oc = off_c, on = off_n, og = off_g, od = off_d;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    for (int q = 0; q < n[j]; ++q) {
      const int m = c[j] - G * q < G ? c[j] - G * q : G;
      a.gen[on + q] = lay::GenEntry{2 * t + j, oc + G * q, m, og + q * tg[j], od + q * td[j]};
    }
    oc += c[j];
    on += n[j];
    og += n[j] * tg[j];
    od += n[j] * td[j];
  }
  // the shared expert: every row, in entries of G rows
  const int nsh = a.shared ? (a.R + G - 1) / G : 0;
  const uint32_t sfmt = a.shared ? a.shared->fmt : 0u;
  const int sg = tiles_of<S, true>(sfmt), sd = tiles_of<S, false>(sfmt);
  for (int q = t; q < nsh; q += kThreads) {
    const int m = a.R - G * q < G ? a.R - G * q : G;
    a.gen[tot_n + q] = lay::GenEntry{-1, G * q, m, tot_g + q * sg, tot_d + q * sd};
  }
  if (t == 0) {
    a.gen_n[0] = tot_n + nsh;
    a.gen_n[1] = tot_g + nsh * sg;
    a.gen_n[2] = tot_d + nsh * sd;
  }
}

// Item maps: workgroup i writes entry i's gate/up and down items.
template <class S>
__global__ __launch_bounds__(kThreads) void k_gen_fill(Args a) {
  const int i = blockIdx.x;
  if (i >= a.gen_n[0]) return;
  const lay::GenEntry ge = a.gen[i];
  const uint32_t fmt = ge.expert >= 0 ? a.experts[ge.expert].fmt : a.shared->fmt;
  const int tg = tiles_of<S, true>(fmt), td = tiles_of<S, false>(fmt);
  for (int q = tid(); q < tg; q += kThreads) a.map_gu[ge.gu_off + q] = i;
  for (int q = tid(); q < td; q += kThreads) a.map_dn[ge.dn_off + q] = i;
}

// Gate/up (GU) or down items of the generic entries, grid-striding.  A routed
// entry's pairs come from the expert-sorted list (row = pair / k, weight =
// the routing weight); the shared expert's pairs are R*k + r with weight 1.
template <class S, bool GU>
__global__ __launch_bounds__(kThreads, MOE_WAVES_PER_EU) void k_gen_ffn(Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ SlotEntry sl;
  __shared__ int tile_s;
  const int n_items = uniform(a.gen_n[GU ? 1 : 2]);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    if (tid() < lay::kGenRows) {
      const int i = (GU ? a.map_gu : a.map_dn)[item];
      const lay::GenEntry ge = a.gen[i];
      const int t = tid();
      if (t == 0) {
        sl.ref = ge.expert >= 0 ? a.experts[ge.expert] : *a.shared;
        sl.expert = ge.expert;
        sl.nt = ge.m;
        tile_s = item - (GU ? ge.gu_off : ge.dn_off);
      }
      if (t < ge.m) {
        if (ge.expert >= 0) {
          const int pair = a.list[ge.s0 + t];
          sl.row[t] = pair / a.k;
          sl.pair[t] = pair;
          sl.w[t] = a.wts[pair];
        } else {
          sl.row[t] = ge.s0 + t;
          sl.pair[t] = a.R * a.k + ge.s0 + t;
          sl.w[t] = 1.0f;
        }
      }
    }
    __syncthreads();
    run_slot<S, GU ? 2 : 0, false>(a, sl, uniform(tile_s), lds);
    __syncthreads();
  }
}

// Streaming-read ceiling: every lane reads U 16-byte chunks per iteration,
// grid-striding, and folds them into an xor checksum.
template <int U>
__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  const size_t nth = static_cast<size_t>(gridDim.x) * kThreads;
  const size_t t = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  const size_t rounds = n16 / (U * nth);   // whole rounds; the rest is the tail
  for (size_t m = 0, i = t; m < rounds; ++m, i += U * nth) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * nth);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (size_t i = t + rounds * U * nth; i < n16; i += nth) {   // the tail
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[t] = acc;
}

}  // namespace dev

// ===========================================================================
// host side
// ===========================================================================
namespace {

int shape_class(const moe_dims* d) { return lay::shape_class(*d); }

// Grid of a work-list launch: enough workgroups for every item of the
// heaviest format mix, capped (items beyond the grid are strided over).
// one residency round: MOE_WAVES_PER_EU workgroups of 4 waves per CU, 256 CUs
constexpr int kMaxGrid = MOE_WAVES_PER_EU * 256;
int item_grid(int upper, int cap = kMaxGrid) { return upper < cap ? upper : cap; }
// Fused launch: at most one residency round of workers, so that all of them
// can be resident at once once the router and selection workgroups are done
// (a down item may wait on a gate/up item of any worker).
// at most this many workers take the shared expert's gate/up tiles (before
// the selection); the others are free for routed gate/up items at once
constexpr int kSharedWorkers = 576;

// Workgroups of k_layer<S> the device holds at once: the occupancy the
// runtime reports for its registers and LDS, times the compute units.  Kept
// per device (a lookup once per device and shape; racing first calls compute
// the same value).  0 on failure.
template <class S>
int fused_workers() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dev::k_layer<S>, dev::kThreads, S::LDS_LAYER) !=
          hipSuccess || per_cu <= 0)
    return 0;
  const int n = per_cu * cus;
  if (dev >= 0 && dev < kMaxDev) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Tags of fused calls: unique in the process, so no word a workspace holds
// from an earlier call can carry the tag of a later one.
std::atomic<uint32_t> g_call_tag{0};
std::atomic<int> g_spin_limit{dev::kSpinLimit};

uint32_t next_tag() {
  uint32_t t;
  do t = g_call_tag.fetch_add(1, std::memory_order_relaxed) + 1; while (t == 0);
  return t;
}

// moe_layer: one fused launch.
template <class S>
int launch_fused(const moe_dims* d, int rows, dev::Args a, uint8_t* w8, const lay::TaggedLayout& l,
                 hipStream_t s, void* const* events, int n_events) {
  const int n_routed = rows * d->top_k;
  const bool sh = a.shared != nullptr;
  const int workers = fused_workers<S>();
  if (workers <= 0) return MOE_EDEVICE;
  a.tag = next_tag();
  a.err = reinterpret_cast<uint32_t*>(w8 + l.err);
  a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  a.part_t = reinterpret_cast<uint64_t*>(w8 + l.part_t);
  a.lgt = reinterpret_cast<uint64_t*>(w8 + l.lgt);
  a.selt = reinterpret_cast<uint64_t*>(w8 + l.selt);
  a.ht = reinterpret_cast<uint64_t*>(w8 + l.ht);
  a.rmax_t = reinterpret_cast<uint64_t*>(w8 + l.rmax);
  a.shared_early = 1;     // the shared gate/up tiles are taken by the workers before the selection
  a.base_b = d->n_experts + rows;
  a.nb = item_grid((sh ? S::MAX_TILES_GU : 0) + n_routed * S::MAX_TILES_GU + (n_routed + (sh ? 1 : 0)) * S::MAX_TILES_DN,
                   workers);
  a.base_y = a.base_b + a.nb;
  a.nsw = item_grid(kSharedWorkers, a.nb);
  const int ny = (rows * S::kH + dev::kThreads - 1) / dev::kThreads;
  const size_t lds = S::LDS_LAYER;
  int ev = 0;
  auto rec = [&]() {
    if (events && ev < n_events) (void)hipEventRecord(static_cast<hipEvent_t>(events[ev]), s);
    ++ev;
  };
  rec();
  hipLaunchKernelGGL(dev::k_layer<S>, dim3(a.base_y + ny), dim3(dev::kThreads), lds, s, a);
  rec();
  if (hipGetLastError() != hipSuccess) return MOE_EDEVICE;
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
    const int shared_gu = (sh && a.shared_early) ? S::MAX_TILES_GU : 0;
    hipLaunchKernelGGL(dev::k_route<S>, dim3(d->n_experts + dev::kPrepWGs + shared_gu),
                       dim3(dev::kThreads), S::LDS_WITH_STAGE, s, a);
    if (!launched()) return MOE_EDEVICE;
    hipLaunchKernelGGL(dev::k_select<S>, dim3(1), dim3(dev::kThreads), 0, s, a);
    if (!launched()) return MOE_EDEVICE;
  } else {
    hipLaunchKernelGGL(dev::k_prep<S>, dim3(1 + dev::kPrepWGs), dim3(dev::kThreads), 0, s, a);
    if (!launched()) return MOE_EDEVICE;
  }
  if (ffn) {
    const int slots_gu = n_routed + ((sh && !a.shared_early) ? 1 : 0);
    const int slots_dn = n_routed + (sh ? 1 : 0);
    hipLaunchKernelGGL(dev::k_gateup<S>, dim3(item_grid(slots_gu * S::MAX_TILES_GU)),
                       dim3(dev::kThreads), lds, s, a);
    if (!launched()) return MOE_EDEVICE;
    hipLaunchKernelGGL(dev::k_down<S>, dim3(item_grid(slots_dn * S::MAX_TILES_DN)),
                       dim3(dev::kThreads), lds, s, a);
    if (!launched()) return MOE_EDEVICE;
    hipLaunchKernelGGL(dev::k_combine<S>, dim3((rows * S::kH + dev::kThreads - 1) / dev::kThreads),
                       dim3(dev::kThreads), 0, s, a);
    if (!launched()) return MOE_EDEVICE;
  }
  return MOE_OK;
}

// fused_only: the workspace holds only the fused launch's area (the fixed
// workspace of moe_layer_noalloc, lay::fused_layout), not a full decode layout.
int run(const moe_dims* d, const void* x, int rows, const float* w_router, const float* bias,
        const void* weights, const moe_expert_ref* experts, const moe_expert_ref* shared,
        int32_t* idx, float* wts, float* y, void* ws, size_t ws_bytes, void* stream,
        bool route, bool ffn, void* const* events, int n_events, bool fused_only = false,
        const float* noise = nullptr, uint16_t* x_next = nullptr) {
  int st = check_dims(d, rows);
  if (st) return st;
  if (rows == 0) return MOE_OK;
  if (!x || !ws) return MOE_EINVAL;
  if (route && !w_router) return MOE_EINVAL;
  if (ffn && (!weights || !experts || !y)) return MOE_EINVAL;
  if (!route && (!idx || !wts)) return MOE_EINVAL;
  lay::DecodeLayout l = lay::decode_layout(*d, rows);
  if (fused_only) {
    if (!(route && ffn)) return MOE_EINVAL;
    const lay::FusedLayout f = lay::fused_layout(*d);
    if (ws_bytes < f.total) return MOE_EWORKSPACE;
    l = lay::DecodeLayout{};            // the split path's regions do not exist here
    l.idx = f.idx;
    l.wts = f.wts;
  } else if (ws_bytes < l.total) {
    return MOE_EWORKSPACE;
  }
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
  if (!fused_only) {
    a.logits = reinterpret_cast<double*>(w8 + l.logits);
    a.slots = reinterpret_cast<dev::SlotTable*>(w8 + l.slots);
    a.order = reinterpret_cast<int32_t*>(w8 + l.order);
    a.xinv = reinterpret_cast<float*>(w8 + l.xinv);
    a.xrec = w8 + l.xrec;
    a.xrow = l.xrow;
    a.h = reinterpret_cast<float*>(w8 + l.h);
    a.part = reinterpret_cast<float*>(w8 + l.part);
  }
  a.R = rows;
  a.k = d->top_k;
  a.E = d->n_experts;
  a.shared_early = (route && ffn && shared) ? 1 : 0;
  a.noise = noise;
  a.x_next = x_next;     // only the fused launch writes it
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (route && ffn) {
    switch (shape_class(d)) {
      case 1: return launch_fused<dev::Shape<5120, 2304>>(d, rows, a, w8, lay::tagged_layout(*d), s, events, n_events);
      case 2: return launch_fused<dev::Shape<512, 256>>(d, rows, a, w8, lay::tagged_layout(*d), s, events, n_events);
      default: return MOE_ESHAPE;
    }
  }
  switch (shape_class(d)) {
    case 1: return launch_layer<dev::Shape<5120, 2304>>(d, rows, a, route, ffn, s, events, n_events);
    case 2: return launch_layer<dev::Shape<512, 256>>(d, rows, a, route, ffn, s, events, n_events);
    default: return MOE_ESHAPE;
  }
}

// ---------------------------------------------------------------------------
// The fixed workspace of moe_layer_noalloc: one array per GPU, held until the
// process ends, for callers that cannot allocate.  Host code never names the
// array itself (that is a host-side stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and is kept per device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t{4608} << 10;   // 4.5 MiB
static_assert(lay::fused_layout(moe_dims{5120, 2304, lay::kMaxExperts, lay::kMaxK, 0}).total <= kScratchBytes,
              "the fixed workspace holds the fused area of the largest supported layer");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The device address of this device's scratch, looked up on the first call
// on the device; null on failure.
uint8_t* scratch_ptr() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static uint8_t* ptrs[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = static_cast<uint8_t*>(p);
  }
  return ptrs[dev];
}

template <class S>
int launch_generic(const gen::Launch& g, hipStream_t s) {
  dev::Args a{};
  a.x = static_cast<const uint16_t*>(g.x);
  a.idx = const_cast<int32_t*>(g.idx);
  a.wts = const_cast<float*>(g.wts);
  a.weights = static_cast<const uint8_t*>(g.weights);
  a.experts = g.experts;
  a.shared = g.shared;
  a.h = g.h32;
  a.part = g.part;
  a.gen = g.gen;
  a.gen_n = g.gen_n;
  a.map_gu = g.map_gu;
  a.map_dn = g.map_dn;
  a.list = g.list;
  a.cnt = g.cnt;
  a.mfma = g.mfma;
  a.R = g.rows;
  a.k = g.top_k;
  a.E = g.n_experts;
  hipLaunchKernelGGL(dev::k_gen_plan<S>, dim3(1), dim3(dev::kThreads), 0, s, a);
  hipLaunchKernelGGL(dev::k_gen_fill<S>, dim3(g.max_gen), dim3(dev::kThreads), 0, s, a);
  hipLaunchKernelGGL((dev::k_gen_ffn<S, true>), dim3(item_grid(g.max_items_gu)), dim3(dev::kThreads),
                     S::LDS_WITH_STAGE, s, a);
  hipLaunchKernelGGL((dev::k_gen_ffn<S, false>), dim3(item_grid(g.max_items_dn)), dim3(dev::kThreads),
                     S::LDS_WITH_STAGE, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

}  // namespace

namespace gen {
int launch(const moe_dims* d, const Launch& g, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (shape_class(d)) {
    case 1: return launch_generic<dev::Shape<5120, 2304>>(g, s);
    case 2: return launch_generic<dev::Shape<512, 256>>(g, s);
    default: return MOE_ESHAPE;
  }
}
}  // namespace gen
}  // namespace moe

extern "C" {

int moe_workspace_status(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 16) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t err = 0;
  // the error word is the first word of every workspace (layout.h)
  if (hipMemcpyAsync(&err, ws, sizeof(err), hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_EDEVICE;
  if (err == 0) return MOE_OK;
  if (hipMemsetAsync(ws, 0, sizeof(err), s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return MOE_EDEVICE;
  return MOE_ETIMEOUT;
}

int32_t moe_set_spin_limit(int32_t polls) {
  if (polls < 0) return MOE_EINVAL;
  return moe::g_spin_limit.exchange(polls, std::memory_order_relaxed);
}

int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, int32_t unroll,
                    void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) || grid < 1 || grid > 65536)
    return MOE_EINVAL;
  const auto* p = static_cast<const moe::dev::u32x4*>(buf);
  const size_t n16 = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(static_cast<unsigned>(grid)), b(moe::dev::kThreads);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(moe::dev::k_stream_read<1>, g, b, 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(moe::dev::k_stream_read<2>, g, b, 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(moe::dev::k_stream_read<4>, g, b, 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(moe::dev::k_stream_read<8>, g, b, 0, s, p, n16, sink); break;
    default: return MOE_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

int moe_add_chain(float* y, const float* add, const float* noise, void* x_next, int32_t rows, int32_t hidden,
                  void* stream) {
  if (!y || rows < 0 || hidden <= 0) return MOE_EINVAL;
  if (rows == 0 || (!add && !x_next)) return MOE_OK;
  hipLaunchKernelGGL(moe::dev::k_chain_rows, dim3(static_cast<unsigned>(rows)), dim3(moe::dev::kThreads), 0,
                     static_cast<hipStream_t>(stream), y, add, noise, static_cast<uint16_t*>(x_next), hidden);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

int moe_quant_mxfp8(const void* x_bf16, int32_t rows, int32_t k, void* codes, void* scales,
                    void* stream) {
  return moe::pf::quant(x_bf16, rows, k, codes, scales, stream);
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
  if (rows > MOE_MAX_DECODE_ROWS) {
    if (int st = moe::check_many_row_dims(dims, rows)) return st;
    return moe::pf::run(dims, x_bf16, rows, idx, wts, weights, experts, shared, y, ws, ws_bytes,
                        stream);
  }
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

int moe_layer_noalloc(const moe_dims* dims, const void* x_bf16, int32_t rows, const float* w_router,
                      const float* sel_bias, const void* weights, const moe_expert_ref* experts,
                      const moe_expert_ref* shared, int32_t* idx, float* wts, float* y, void* stream) {
  if (int st = moe::check_dims(dims, rows)) return st;
  if (rows == 0) return MOE_OK;
  if (moe::lay::fused_layout(*dims).total > moe::kScratchBytes) return MOE_EWORKSPACE;
  uint8_t* ws = moe::scratch_ptr();
  if (!ws) return MOE_EDEVICE;
  return moe::run(dims, x_bf16, rows, w_router, sel_bias, weights, experts, shared, idx, wts, y, ws,
                  moe::kScratchBytes, stream, true, true, nullptr, 0, true);
}

int moe_layer_profiled(const moe_dims* dims, const void* x_bf16, int32_t rows,
                       const float* w_router, const float* sel_bias, const void* weights,
                       const moe_expert_ref* experts, const moe_expert_ref* shared,
                       int32_t* idx, float* wts, float* y, void* ws, size_t ws_bytes,
                       void* stream, void* const* events, int32_t n_events) {
  if (!events || n_events < 2) return MOE_EINVAL;
  return moe::run(dims, x_bf16, rows, w_router, sel_bias, weights, experts, shared, idx, wts, y,
                  ws, ws_bytes, stream, true, true, events, n_events);
}

int moe_stack_decode(const moe_dims* dims, int32_t n_layers, const moe_layer_weights* layers,
                     int32_t rows, void* x_all, const float* noise, float* y_all, int32_t* idx_all,
                     float* wts_all, void* ws, size_t ws_bytes, void* stream) {
  if (n_layers < 0 || (n_layers > 0 && (!layers || !x_all || !y_all))) return MOE_EINVAL;
  if (int st = moe::check_dims(dims, rows)) return st;
  const size_t xy = static_cast<size_t>(rows) * dims->hidden;
  const size_t ik = static_cast<size_t>(rows) * dims->top_k;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_weights& w = layers[l];
    if (!w.w_router || !w.weights || !w.experts) return MOE_EINVAL;
  }
  uint16_t* x = static_cast<uint16_t*>(x_all);
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_weights& w = layers[l];
    const int st = moe::run(dims, x + l * xy, rows, w.w_router, w.sel_bias, w.weights, w.experts, w.shared,
                            idx_all ? idx_all + l * ik : nullptr, wts_all ? wts_all + l * ik : nullptr,
                            y_all + l * xy, ws, ws_bytes, stream, true, true, nullptr, 0, false,
                            noise ? noise + l * xy : nullptr, x + (l + 1) * xy);
    if (st) return st;
  }
  return MOE_OK;
}

}  // extern "C"
