// gfx950 many-row (prefill) path of the routed-MoE expert FFN: many rows per
// call (a prompt, thousands of tokens).  MXFP4 experts run here on the
// matrix cores; every other expert, and the shared expert, runs the decode
// tiles on the same expert-grouped pair lists (moe_kernels.hip).
//
// The experts become a grouped, dense contraction here -- each selected
// expert sees tens to hundreds of rows -- so the products run on the scaled
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4: fp8 e4m3 activations times
// fp4 e2m1 weights, one e8m0 scale per 32 elements on both sides).  The
// activations enter as MXFP8: x is quantised per 32 consecutive elements of a
// row (scale exponent floor(log2 amax) - 8 + 127, elements rounded to nearest
// even and saturated at 448).  h stays f16 and the down projection runs on the
// f16 matrix cores (v_mfma_f32_16x16x32_f16) with the fp4 weights widened to
// f16 by the hardware converter: re-quantising h to 8 bits would make its
// rounding decisions depend on the last bits of an fp32 accumulation.
//
//   quant     x [R x H] bf16 -> MXFP8 codes + scales
//   count     rows per expert
//   place     pairs (row, slot) grouped by expert, ascending pair index;
//             chunks of at most kChunk pairs of one expert
//   gateup    per (chunk, 256 channels): G = Xq W_gate^T, V = Xq W_up^T on the
//             scaled matrix cores, h = silu(G) * V stored as f16
//   down      per (chunk, 256 outputs): w * (h W_down^T) into per-pair partials
//   combine   y[r] = the row's partials in ascending expert id
//
// Method: "DeepSeek-V4.1-Flash served three ways on 4xL20" (lcz.me/topic/2356),
// section 1 (the layer) and the FP4 expert checkpoint it names; "[Strata]
// DeepSeek V4.1 Flash on a single 4090" (lcz.me/post/25274), section 4 (prefill
// runs the experts as dense products).  Element and scale encodings follow the
// OCP Microscaling Formats (MX) v1.0 specification.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/moe.h"
#include "dev_common.h"
#include "prefill.h"

namespace moe {
namespace pf {

using dev::Buf;
using dev::bload128;
using dev::bload8;
using dev::make_buf;
using dev::u32x4;
using dev::u32x2;
using dev::bload64;
using dev::uniform;

constexpr int kThreads = 256;
constexpr int kChunk = lay::kChunk;      // pairs of one expert per work item
constexpr int kRowTiles = kChunk / 16;   // 16-row matrix-core tiles per chunk
constexpr int kStepK = 128;              // K per matrix-core instruction
// LDS row pitch of the staged activation tiles: one 16-byte slot more than a
// row, so the 16 rows that one lane group reads per fragment start in
// different banks (an unpadded 128- or 256-byte pitch maps them all to the
// same banks)
constexpr int kAPitch = kStepK + 16;     // fp8 codes, bytes
constexpr int kHPitch = kStepK + 8;      // f16 values
constexpr int kGuThreads = 512;          // gate/up workgroup: 8 waves
constexpr int kGuCh = kGuThreads / 2;    // gate/up channels per work item (8 waves x 32)
constexpr int kDnCh = 256;               // down outputs per work item (4 waves x 64)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

using lay::Chunk;

struct Args {
  const uint16_t* x;              // [R x H] bf16
  const int32_t* idx;             // [R x k]
  const float* wts;               // [R x k]
  const uint8_t* weights;
  const moe_expert_ref* experts;  // [E]
  float* y;                       // [R x H]
  uint8_t* xq;                    // [R x H] e4m3
  uint8_t* xs;                    // [R x H/32] e8m0
  int32_t* cnt;                   // [E]
  int32_t* list;                  // [R k]: pair ids grouped by expert, ascending within
  Chunk* chunks;                  // [max_chunks]
  int32_t* n_chunks;              // [1]
  uint16_t* hq;                   // [R k x I] f16 h, expert-sorted positions
  float* part;                    // [(R k + R) x H] per-pair partial outputs (pair id
                                  // order; the shared expert's rows last)
  int R, k, E, H, I;
  int has_shared;                 // the combine adds the shared expert's partials
};

// ---------------------------------------------------------------------------
// MXFP8 encoding
// ---------------------------------------------------------------------------
// Nearest e4m3 (OCP FN variant) code of v, ties to the even significand,
// magnitudes at or above 448 saturating to 448.  Normal binade [2^e, 2^(e+1))
// with e >= -6 has quantum 2^(e-3); below 2^-6 the subnormal quantum 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __builtin_fabsf(v);
  if (!(a < 448.0f)) return sign | 0x7Eu;           // saturate (NaN inputs too)
  int e = static_cast<int>((bits >> 23) & 0xFFu) - 127;
  if (e < -6) e = -6;
  float m = __builtin_rintf(__builtin_ldexpf(a, 3 - e));   // exact scaling, then RNE
  if (m >= 16.0f) {                                  // rounded up into the next binade
    m = 8.0f;
    ++e;
  }
  const uint32_t mi = static_cast<uint32_t>(m);
  if (mi < 8u) return sign | mi;                      // subnormal (only when e == -6)
  return sign | (static_cast<uint32_t>(e + 7) << 3) | (mi - 8u);
}

// e8m0 scale exponent of a block with largest magnitude amax:
// floor(log2 amax) - 8 + 127 clamped to [0, 254]; 0 for an all-zero block.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  (void)__builtin_frexpf(amax, &ex);                 // amax = f * 2^ex, f in [0.5, 1)
  int E = (ex - 1) - 8 + 127;
  return E < 0 ? 0 : (E > 254 ? 254 : E);
}

// Quantises 32 values to MXFP8; returns the scale exponent, codes in q[8].
__device__ __forceinline__ int mx_quant32(const float (&v)[32], uint32_t (&q)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const int E = mx_scale_exp(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t u = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) u |= e4m3_code(__builtin_ldexpf(v[4 * w + b], 127 - E)) << (8 * b);
    q[w] = u;
  }
  return E;
}

// x [rows x K] bf16 -> codes [rows x K] e4m3 + scales [rows x K/32] e8m0;
// one thread per block of 32.
__global__ __launch_bounds__(kThreads) void k_quant(const uint16_t* x, int rows, int K, uint8_t* codes,
                                                    uint8_t* scales) {
  const int nb = K / 32;
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= rows * nb) return;
  const int r = b / nb, c = b - r * nb;
  const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<size_t>(r) * K + 32 * c);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = src[i];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[8 * i + 2 * t] = dev::bf16_bits_to_f32(w[t] & 0xFFFFu);
      v[8 * i + 2 * t + 1] = dev::bf16_bits_to_f32(w[t] >> 16);
    }
  }
  uint32_t q[8];
  const int E = mx_quant32(v, q);
  uint4* dst = reinterpret_cast<uint4*>(codes + static_cast<size_t>(r) * K + 32 * c);
  dst[0] = uint4{q[0], q[1], q[2], q[3]};
  dst[1] = uint4{q[4], q[5], q[6], q[7]};
  scales[static_cast<size_t>(r) * nb + c] = static_cast<uint8_t>(E);
}

// ---------------------------------------------------------------------------
// dispatch: pairs grouped by expert, deterministic order
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wg_sum(int v, int* red) {
  v = wave_sum_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < kThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// count: workgroup e counts the pairs that chose expert e.
__global__ __launch_bounds__(kThreads) void k_count(Args a) {
  __shared__ int red[kThreads / 64];
  const int e = blockIdx.x, n = a.R * a.k;
  int c = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) c += a.idx[i] == e;
  c = wg_sum(c, red);
  if (threadIdx.x == 0) a.cnt[e] = c;
}

// place: workgroup e writes its pairs in ascending pair order at its offset
// and its chunks at its chunk offset; the last workgroup records the total.
__global__ __launch_bounds__(kThreads) void k_place(Args a) {
  __shared__ int red[kThreads / 64];
  __shared__ int wave_cnt[kThreads / 64];
  const int e = blockIdx.x, n = a.R * a.k;
  int off = 0, coff = 0;
  for (int q = threadIdx.x; q < e; q += kThreads) {
    const int c = a.cnt[q];
    off += c;
    coff += (c + kChunk - 1) / kChunk;
  }
  off = wg_sum(off, red);
  coff = wg_sum(coff, red);
  const int ce = a.cnt[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = off;
  for (int i0 = 0; i0 < n; i0 += kThreads) {
    const int i = i0 + threadIdx.x;
    const bool hit = i < n && a.idx[i] == e;
    const uint64_t m = __ballot(hit);
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      before += w < wave ? wave_cnt[w] : 0;
      tot += wave_cnt[w];
    }
    if (hit) a.list[base + before + __popcll(m & ((1ull << lane) - 1ull))] = i;
    base += tot;
    __syncthreads();
  }
  const int nch = (ce + kChunk - 1) / kChunk;
  for (int c = threadIdx.x; c < nch; c += kThreads) {
    const int m = ce - c * kChunk < kChunk ? ce - c * kChunk : kChunk;
    a.chunks[coff + c] = Chunk{e, off + c * kChunk, m};
  }
  if (e == a.E - 1 && threadIdx.x == 0) *a.n_chunks = coff + nch;
}

// ---------------------------------------------------------------------------
// grouped products on the scaled matrix cores
// ---------------------------------------------------------------------------
// Operand layouts of v_mfma_scale_f32_16x16x128_f8f6f4 (lane l, g = l / 16):
//   A (fp8, 16 x 128): row l % 16; bytes 0..15 hold K 16g .. 16g+15, bytes
//                      16..31 hold K 64+16g .. 64+16g+15; the lane's scale is
//                      the row's block g (K 32g .. 32g+31)
//   B (fp4, 128 x 16): column l % 16; nibbles (low first) hold K 32g .. 32g+31,
//                      one block, whose scale the lane carries
//   D (f32, 16 x 16):  register r holds row 4g + r, column l % 16
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const u32x4& b, const v4f& c, uint32_t sa,
                                       uint32_t sb) {
  const v8i bb = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
                  static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, static_cast<int>(sa), 0,
                                                           static_cast<int>(sb));
}

// One fp4 weight fragment of an MXFP4 matrix [N x K] (planar: codes, then
// scales): row `row`, K-step s (128 wide), block g of the step.
struct WFrag {
  u32x4 q;
  uint32_t s;
};
__device__ __forceinline__ WFrag load_wfrag(const Buf& m, int N, int K, int row, int s, int g) {
  const uint32_t nb = static_cast<uint32_t>(K / 32);
  const uint32_t blk = static_cast<uint32_t>(row) * nb + static_cast<uint32_t>(s * 4 + g);
  WFrag f;
  f.q = bload128(m, blk * 16u);
  f.s = bload8(m, static_cast<uint32_t>(N) * nb * 16u + blk);
  return f;
}

// Largest value over the 16 lanes of a DPP row (lanes 16q .. 16q+15).
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  return v;
}

// The activation tile of one K-step: kChunk rows x 128 fp8 codes + 4 scale
// bytes per row, staged in LDS by all T threads of the workgroup (16-byte
// chunks, kChunk * 8 / T each).
template <int T>
struct ATile {
  static constexpr int N = kChunk * 8 / T;
  u32x4 v[N];
  uint32_t sc;
};
template <int T>
__device__ __forceinline__ void a_load(ATile<T>& t, const Buf& codes, const Buf& scales, const int* src,
                                       int K, int s) {
  constexpr uint32_t kNone = 0x7FFFFFF0u;   // past every buffer: reads as zeros
#pragma unroll
  for (int i = 0; i < ATile<T>::N; ++i) {
    const int q = threadIdx.x + T * i, row = q >> 3, part = q & 7;
    const int r = src[row];
    const uint32_t off = r >= 0 ? static_cast<uint32_t>(r) * K + s * kStepK + part * 16 : kNone;
    t.v[i] = bload128(codes, off);
  }
  if (threadIdx.x < kChunk) {
    const int r = src[threadIdx.x];
    t.sc = r >= 0 ? dev::bload32(scales, static_cast<uint32_t>(r) * (K / 32) + 4 * s) : 0u;
  }
}
template <int T>
__device__ __forceinline__ void a_store(const ATile<T>& t, uint8_t (*codes)[kAPitch], uint32_t* sc) {
#pragma unroll
  for (int i = 0; i < ATile<T>::N; ++i) {
    const int q = threadIdx.x + T * i, row = q >> 3, part = q & 7;
    *reinterpret_cast<u32x4*>(&codes[row][part * 16]) = t.v[i];
  }
  if (threadIdx.x < kChunk) sc[threadIdx.x] = t.sc;
}
// The lane's A fragment of row tile rt (16 rows) from the staged tile.
__device__ __forceinline__ v8i a_frag(const uint8_t (*codes)[kAPitch], const uint32_t* sc, int rt,
                                      int j, int g, uint32_t& sa) {
  const int row = rt * 16 + j;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(&codes[row][16 * g]);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(&codes[row][64 + 16 * g]);
  sa = (sc[row] >> (8 * g)) & 0xFFu;
  return v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
             static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// Work items are placed by XCD.  The dispatcher hands workgroups to the eight
// XCDs round-robin by id, so id b runs on XCD b % 8, as the (b / 8)-th of that
// XCD.  XCD x takes the x-th eighth of the chunk list (chunks are in expert
// order) and walks it chunk by chunk, the NT tiles of a chunk back to back:
// a chunk's activation tile, and the weight tile nt of an expert's
// consecutive chunks, are read by workgroups that run together on one XCD,
// so its L2 serves the repeats.  ci = -1: no item for this id.
constexpr int kXcd = 8;
__device__ __forceinline__ void item_of_block(int b, int NT, int n_chunks, int& ci, int& nt) {
  const int x = b % kXcd, l = b / kXcd, per = (n_chunks + kXcd - 1) / kXcd;
  nt = l % NT;
  const int c = l / NT;
  ci = c < per ? x * per + c : -1;
  if (ci >= n_chunks) ci = -1;
}

// gate/up: work item (chunk, 256 channels); wave w of eight owns channels
// c0 .. c0+31 of gate and up (four B fragments per K-step), every row tile of
// the chunk.  The eight waves share one staged activation tile, so a chunk's
// activations are read by I / 256 workgroups.  h = silu(G) * V goes out as
// f16 (round to nearest even) at the pairs' expert-sorted positions.
template <int H, int I>
__global__ __launch_bounds__(kGuThreads, 1) void k_gateup(Args a) {
  constexpr int NT = I / kGuCh, S = H / kStepK;
  static_assert(I % kGuCh == 0, "whole channel tiles");
  __shared__ __align__(16) uint8_t at[2][kChunk][kAPitch];
  __shared__ uint32_t asc[2][kChunk];
  __shared__ int src[kChunk];
  int ci, nt;
  item_of_block(blockIdx.x, NT, uniform(*a.n_chunks), ci, nt);
  if (ci < 0) return;
  const Chunk ch = a.chunks[ci];
  const int m = uniform(ch.m), s0 = uniform(ch.s0);
  const moe_expert_ref ref = a.experts[uniform(ch.expert)];
  if (uniform(static_cast<int>(ref.fmt)) != MOE_FMT_MXFP4) return;   // a generic entry's pairs
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15, g = lane >> 4;
  if (threadIdx.x < kChunk) src[threadIdx.x] = threadIdx.x < m ? a.list[s0 + threadIdx.x] / a.k : -1;
  __syncthreads();
  const int mt = (m + 15) / 16;
  const uint32_t mbytes = static_cast<uint32_t>(I) * (H / 32) * 17u;
  const Buf mg = make_buf(a.weights + ref.gate, mbytes);
  const Buf mu = make_buf(a.weights + ref.up, mbytes);
  const Buf xb = make_buf(a.xq, static_cast<uint32_t>(a.R) * H);
  const Buf xsb = make_buf(a.xs, static_cast<uint32_t>(a.R) * (H / 32));
  const int c0 = nt * kGuCh + wave * 32;
  const int brow[4] = {c0 + j, c0 + 16 + j, c0 + j, c0 + 16 + j};
  v4f acc[kRowTiles][4];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[rt][f] = v4f{0.f, 0.f, 0.f, 0.f};
  // Software pipeline over the K-steps:
  //   weight codes   a lane's 16-byte pieces of steps 2t and 2t+1 are the two
  //                  halves of one 128-byte line: both are loaded together,
  //                  on step 2t-2, into a ring of four steps.  Loaded a step
  //                  apart, a line could leave L2 between its halves and be
  //                  fetched twice
  //   e8m0 scales    four K-steps per aligned 16-byte load of the row (lane
  //                  group g uses byte g of dword s % 4), a group ahead
  //   activations    two steps ahead into registers, stored to the LDS
  //                  double buffer one step before use
  // Within a step the loads go out in the order of their use, so the wait
  // for one never drains a load needed later (the counter is in order).
  static_assert(S % 4 == 0, "scales are loaded four K-steps at a time");
  constexpr int kRing = 4;
  const uint32_t nbk = static_cast<uint32_t>(H / 32), splane = static_cast<uint32_t>(I) * nbk * 16u;
  auto scale_group = [&](int f, int q) {
    return bload128(f < 2 ? mg : mu, splane + static_cast<uint32_t>(brow[f]) * nbk + 16u * q);
  };
  auto codes = [&](int f, int s) {
    return bload128(f < 2 ? mg : mu, (static_cast<uint32_t>(brow[f]) * nbk + static_cast<uint32_t>(4 * s + g)) * 16u);
  };
  u32x4 bq[kRing][4], sg[2][4];
  ATile<kGuThreads> ta[2];
#pragma unroll
  for (int f = 0; f < 4; ++f) sg[0][f] = scale_group(f, 0);
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int f = 0; f < 4; ++f) bq[p][f] = codes(f, p);
  a_load(ta[0], xb, xsb, src, H, 0);
  if (S > 1) a_load(ta[1], xb, xsb, src, H, 1);
  a_store(ta[0], at[0], asc[0]);
  __syncthreads();
  // eight steps per iteration: every ring index is a compile-time constant
#pragma unroll 1
  for (int s8 = 0; s8 < S; s8 += 8) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int s = s8 + d;
      if (S % 8 != 0 && s >= S) break;
      const int gq = d / 4;   // scale group slot of this step
      if (d % 4 == 0 && s + 4 < S) {
#pragma unroll
        for (int f = 0; f < 4; ++f) sg[gq ^ 1][f] = scale_group(f, s / 4 + 1);
      }
      if (s + 2 < S) a_load(ta[d % 2], xb, xsb, src, H, s + 2);
      if (d % 2 == 0 && s + 2 < S) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          bq[(d + 2) % kRing][f] = codes(f, s + 2);
          bq[(d + 3) % kRing][f] = codes(f, s + 3);
        }
      }
      uint32_t sb[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const u32x4 w = sg[gq][f];
        sb[f] = ((d % 4 == 0 ? w.x : d % 4 == 1 ? w.y : d % 4 == 2 ? w.z : w.w) >> (8 * g)) & 0xFFu;
      }
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        if (rt < mt) {
          uint32_t sa;
          const v8i af = a_frag(at[d % 2], asc[d % 2], rt, j, g, sa);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[rt][f] = mfma_mx(af, bq[d % kRing][f], acc[rt][f], sa, sb[f]);
        }
      }
      if (s + 1 < S) a_store(ta[(d + 1) % 2], at[(d + 1) % 2], asc[(d + 1) % 2]);
      __syncthreads();
    }
  }
  // epilogue: SwiGLU, h stored as f16 (round to nearest even)
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    if (rt < mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * g + r;
        const float g0 = acc[rt][0][r], g1 = acc[rt][1][r];
        const float h0 = g0 / (1.0f + __expf(-g0)) * acc[rt][2][r];
        const float h1 = g1 / (1.0f + __expf(-g1)) * acc[rt][3][r];
        if (row < m) {
          uint16_t* hrow = a.hq + static_cast<size_t>(s0 + row) * I;
          hrow[c0 + j] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(h0));
          hrow[c0 + 16 + j] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(h1));
        }
      }
    }
  }
}

// down: work item (chunk, 256 outputs); wave w owns outputs c0 .. c0+63 (four
// 16-output tiles), every row tile; w_pair * (h W_down^T) goes to the partials.
// f16 matrix cores, 32 K per instruction: in sub-step q of a 128-wide K-step,
// lane group g supplies K 32g + 8q .. 32g + 8q + 7 of both operands, so a
// lane's weight bytes for the whole step are one 16-byte run of one MX block.
template <int H, int I>
__global__ __launch_bounds__(kThreads, 2) void k_down(Args a) {
  constexpr int NT = H / kDnCh, S = I / kStepK;
  __shared__ __align__(16) uint16_t at[2][kChunk][kHPitch];
  __shared__ int src[kChunk];
  int ci, nt;
  item_of_block(blockIdx.x, NT, uniform(*a.n_chunks), ci, nt);
  if (ci < 0) return;
  const Chunk ch = a.chunks[ci];
  const int m = uniform(ch.m), s0 = uniform(ch.s0);
  const moe_expert_ref ref = a.experts[uniform(ch.expert)];
  if (uniform(static_cast<int>(ref.fmt)) != MOE_FMT_MXFP4) return;   // a generic entry's pairs
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15, g = lane >> 4;
  if (threadIdx.x < kChunk) src[threadIdx.x] = threadIdx.x < m ? s0 + threadIdx.x : -1;
  __syncthreads();
  const int mt = (m + 15) / 16;
  const uint32_t mbytes = static_cast<uint32_t>(H) * (I / 32) * 17u;
  const Buf md = make_buf(a.weights + ref.down, mbytes);
  const Buf hb = make_buf(reinterpret_cast<const uint8_t*>(a.hq), static_cast<uint32_t>(a.R * a.k) * I * 2u);
  const int c0 = nt * kDnCh + wave * 64;
  // h tile loader: kChunk rows x 128 f16 = 16 KB, four 16-byte chunks per thread
  constexpr uint32_t kNone = 0x7FFFFFF0u;
  auto h_load = [&](int s, u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = threadIdx.x + kThreads * i, row = q >> 4, part = q & 15;
      const int r = src[row];
      v[i] = bload128(hb, r >= 0 ? (static_cast<uint32_t>(r) * I + s * kStepK + part * 8) * 2u : kNone);
    }
  };
  auto h_store = [&](int buf, const u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = threadIdx.x + kThreads * i, row = q >> 4, part = q & 15;
      *reinterpret_cast<u32x4*>(&at[buf][row][part * 8]) = v[i];
    }
  };
  v4f acc[kRowTiles][4];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[rt][f] = v4f{0.f, 0.f, 0.f, 0.f};
  // Software pipeline as in the gate/up kernel: the codes of steps 2t and
  // 2t+1 (one 128-byte line) loaded together on step 2t-2 into a ring of four
  // steps; scales two K-steps per aligned 8-byte load of the row
  // (lane group g uses byte g of dword s % 2), a group ahead; the h tile two
  // steps ahead into registers, stored to the LDS double buffer one step
  // before use.  Loads go out in the order of their use.
  static_assert(S % 2 == 0, "scales are loaded two K-steps at a time");
  constexpr int kRing = 4;
  const uint32_t nbk = static_cast<uint32_t>(I / 32), splane = static_cast<uint32_t>(H) * nbk * 16u;
  auto scale_group = [&](int f, int q) {
    return bload64(md, splane + static_cast<uint32_t>(c0 + 16 * f + j) * nbk + 8u * q);
  };
  auto codes = [&](int f, int s) {
    return bload128(md, (static_cast<uint32_t>(c0 + 16 * f + j) * nbk + static_cast<uint32_t>(4 * s + g)) * 16u);
  };
  u32x4 bq[kRing][4], hv[2][4];
  u32x2 sg[2][4];
#pragma unroll
  for (int f = 0; f < 4; ++f) sg[0][f] = scale_group(f, 0);
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int f = 0; f < 4; ++f) bq[p][f] = codes(f, p);
  h_load(0, hv[0]);
  h_load(1, hv[1]);
  h_store(0, hv[0]);
  __syncthreads();
  // four steps per iteration: every ring index is a compile-time constant
#pragma unroll 1
  for (int s4 = 0; s4 < S; s4 += 4) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int s = s4 + d;
    if (S % 4 != 0 && s >= S) break;
    const int gq = d / 2;   // scale group slot of this step
    if (d % 2 == 0 && s + 2 < S) {
#pragma unroll
      for (int f = 0; f < 4; ++f) sg[gq ^ 1][f] = scale_group(f, s / 2 + 1);
    }
    if (s + 2 < S) h_load(s + 2, hv[d % 2]);
    if (d % 2 == 0 && s + 2 < S) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        bq[(d + 2) % kRing][f] = codes(f, s + 2);
        bq[(d + 3) % kRing][f] = codes(f, s + 3);
      }
    }
    float sc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t sw = d % 2 == 0 ? sg[gq][f].x : sg[gq][f].y;
      sc[f] = __builtin_ldexpf(1.0f, static_cast<int>((sw >> (8 * g)) & 0xFFu) - 127);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v8h b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t w = bq[d % kRing][f][q];
        const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[f], 0);
        const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[f], 1);
        const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[f], 2);
        const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc[f], 3);
        b[f] = v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        if (rt < mt) {
          const v8h af = *reinterpret_cast<const v8h*>(&at[d % 2][rt * 16 + j][32 * g + 8 * q]);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[rt][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b[f], acc[rt][f], 0, 0, 0);
        }
      }
    }
    if (s + 1 < S) h_store((d + 1) % 2, hv[(d + 1) % 2]);
    __syncthreads();
  }
  }
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    if (rt < mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * g + r;
        if (row < m) {
          const int pair = a.list[s0 + row];
          const float w = a.wts[pair];
          float* out = a.part + static_cast<size_t>(pair) * H + c0 + j;
#pragma unroll
          for (int f = 0; f < 4; ++f) out[16 * f] = acc[rt][f][r] * w;
        }
      }
    }
  }
}

// y[r] = the row's k partials in ascending expert id, then the shared
// expert's (a fixed order, so y is bitwise reproducible); an id outside
// [0, E) yields NaN.
template <int H>
__global__ __launch_bounds__(kThreads) void k_combine(Args a) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.R * H) return;
  const int r = i / H, n = i - r * H;
  int id[MOE_MAX_TOP_K], rank[MOE_MAX_TOP_K];
  float v[MOE_MAX_TOP_K];
  bool bad = false;
#pragma unroll
  for (int q = 0; q < MOE_MAX_TOP_K; ++q) {
    id[q] = q < a.k ? a.idx[r * a.k + q] : 0x7fffffff;
    // -1: a pair the caller computes elsewhere (no list entry, adds 0); any
    // other id outside [0, E) is invalid and makes the row NaN
    bad = bad || (q < a.k && (id[q] < -1 || id[q] >= a.E));
    v[q] = (q < a.k && id[q] >= 0) ? a.part[static_cast<size_t>(r * a.k + q) * H + n] : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < MOE_MAX_TOP_K; ++q) {
    rank[q] = 0;
#pragma unroll
    for (int p = 0; p < MOE_MAX_TOP_K; ++p) rank[q] += id[p] < id[q];
  }
  float s = 0.0f;
#pragma unroll
  for (int pos = 0; pos < MOE_MAX_TOP_K; ++pos) {
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < MOE_MAX_TOP_K; ++q) t = rank[q] == pos ? v[q] : t;
    if (pos < a.k) s += t;
  }
  if (a.has_shared) s += a.part[static_cast<size_t>(a.R * a.k + r) * H + n];
  a.y[i] = bad ? __builtin_nanf("") : s;
}

// k_combine with four consecutive outputs per thread: 16-byte loads of the
// partials, issued before the ids are known (a pair marked -1 or invalid
// still has its slot in the partials; its value is dropped afterwards), and
// each output summed in the same order as k_combine, so y is bitwise the
// same.  Used when R * H is a multiple of 4 and y is 16-byte aligned.
template <int H>
__global__ __launch_bounds__(kThreads) void k_combine4(Args a) {
  static_assert(H % 4 == 0, "whole float4 groups per row");
  const int i = (blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i >= a.R * H) return;
  const int r = i / H, n = i - r * H;
  const int k = a.k;
  int id[MOE_MAX_TOP_K], rank[MOE_MAX_TOP_K];
  float4 v[MOE_MAX_TOP_K];
#pragma unroll
  for (int q = 0; q < MOE_MAX_TOP_K; ++q)
    v[q] = q < k ? *reinterpret_cast<const float4*>(a.part + static_cast<size_t>(r * k + q) * H + n)
                 : float4{0.f, 0.f, 0.f, 0.f};
  const float4 sh = a.has_shared ? *reinterpret_cast<const float4*>(a.part + static_cast<size_t>(a.R * k + r) * H + n)
                                 : float4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
#pragma unroll
  for (int q = 0; q < MOE_MAX_TOP_K; ++q) {
    id[q] = q < k ? a.idx[r * k + q] : 0x7fffffff;
    bad = bad || (q < k && (id[q] < -1 || id[q] >= a.E));
  }
#pragma unroll
  for (int q = 0; q < MOE_MAX_TOP_K; ++q) {
    rank[q] = 0;
#pragma unroll
    for (int p = 0; p < MOE_MAX_TOP_K; ++p) rank[q] += id[p] < id[q];
  }
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int pos = 0; pos < MOE_MAX_TOP_K; ++pos) {
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < MOE_MAX_TOP_K; ++q) {
      const bool take = rank[q] == pos && id[q] >= 0;
      const bool here = rank[q] == pos;
      t[0] = here ? (take ? v[q].x : 0.f) : t[0];
      t[1] = here ? (take ? v[q].y : 0.f) : t[1];
      t[2] = here ? (take ? v[q].z : 0.f) : t[2];
      t[3] = here ? (take ? v[q].w : 0.f) : t[3];
    }
    if (pos < k) {
      s[0] += t[0];
      s[1] += t[1];
      s[2] += t[2];
      s[3] += t[3];
    }
  }
  if (a.has_shared) {
    s[0] += sh.x;
    s[1] += sh.y;
    s[2] += sh.z;
    s[3] += sh.w;
  }
  const float nan = __builtin_nanf("");
  *reinterpret_cast<float4*>(a.y + i) =
      bad ? float4{nan, nan, nan, nan} : float4{s[0], s[1], s[2], s[3]};
}

}  // namespace pf

// ===========================================================================
// host side
// ===========================================================================
namespace {

template <int H, int I>
int launch_prefill(const moe_dims* d, int rows, pf::Args a, const lay::ManyRowLayout& l, const gen::Launch& g,
                   hipStream_t s) {
  const bool mfma = (d->flags & MOE_ACT_MXFP8) != 0;
  if (mfma) {
    const int nb = (rows * (H / 32) + pf::kThreads - 1) / pf::kThreads;
    hipLaunchKernelGGL(pf::k_quant, dim3(nb), dim3(pf::kThreads), 0, s, a.x, rows, H, a.xq, a.xs);
  }
  hipLaunchKernelGGL(pf::k_count, dim3(d->n_experts), dim3(pf::kThreads), 0, s, a);
  hipLaunchKernelGGL(pf::k_place, dim3(d->n_experts), dim3(pf::kThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return MOE_EDEVICE;
  if (int st = gen::launch(d, g, s)) return st;
  if (mfma) {
    const int chunk_groups = (l.max_chunks + pf::kXcd - 1) / pf::kXcd;   // ids cover every chunk slot
    hipLaunchKernelGGL((pf::k_gateup<H, I>), dim3(chunk_groups * pf::kXcd * (I / pf::kGuCh)),
                       dim3(pf::kGuThreads), 0, s, a);
    hipLaunchKernelGGL((pf::k_down<H, I>), dim3(chunk_groups * pf::kXcd * (H / pf::kDnCh)),
                       dim3(pf::kThreads), 0, s, a);
  }
  if (reinterpret_cast<uintptr_t>(a.y) % 16 == 0)
    hipLaunchKernelGGL(pf::k_combine4<H>, dim3((rows * H / 4 + pf::kThreads - 1) / pf::kThreads),
                       dim3(pf::kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(pf::k_combine<H>, dim3((rows * H + pf::kThreads - 1) / pf::kThreads),
                       dim3(pf::kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

}  // namespace

namespace pf {

int run(const moe_dims* d, const void* x, int rows, const int32_t* idx, const float* wts,
        const void* weights, const moe_expert_ref* experts, const moe_expert_ref* shared, float* y,
        void* ws, size_t ws_bytes, void* stream) {
  if (!x || !idx || !wts || !weights || !experts || !y || !ws) return MOE_EINVAL;
  const lay::ManyRowLayout l = lay::many_row_layout(*d, rows);
  if (ws_bytes < l.total) return MOE_EWORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.idx = idx;
  a.wts = wts;
  a.weights = static_cast<const uint8_t*>(weights);
  a.experts = experts;
  a.y = y;
  a.xq = w8 + l.xq;
  a.xs = w8 + l.xs;
  a.cnt = reinterpret_cast<int32_t*>(w8 + l.cnt);
  a.list = reinterpret_cast<int32_t*>(w8 + l.list);
  a.chunks = reinterpret_cast<Chunk*>(w8 + l.chunks);
  a.n_chunks = reinterpret_cast<int32_t*>(w8 + l.n_chunks);
  a.hq = reinterpret_cast<uint16_t*>(w8 + l.hq);
  a.part = reinterpret_cast<float*>(w8 + l.part);
  a.R = rows;
  a.k = d->top_k;
  a.E = d->n_experts;
  a.H = d->hidden;
  a.I = d->inter;
  a.has_shared = shared != nullptr;
  gen::Launch g{};
  g.x = x;
  g.idx = idx;
  g.wts = wts;
  g.weights = weights;
  g.experts = experts;
  g.shared = shared;
  g.cnt = a.cnt;
  g.list = a.list;
  g.gen = reinterpret_cast<lay::GenEntry*>(w8 + l.gen);
  g.gen_n = reinterpret_cast<int32_t*>(w8 + l.n_gen);
  g.map_gu = reinterpret_cast<int32_t*>(w8 + l.map_gu);
  g.map_dn = reinterpret_cast<int32_t*>(w8 + l.map_dn);
  g.h32 = reinterpret_cast<float*>(w8 + l.h32);
  g.part = a.part;
  g.rows = rows;
  g.top_k = d->top_k;
  g.n_experts = d->n_experts;
  g.mfma = (d->flags & MOE_ACT_MXFP8) ? 1 : 0;
  g.max_gen = l.max_gen;
  g.max_items_gu = l.max_items_gu;
  g.max_items_dn = l.max_items_dn;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->hidden == 5120 && d->inter == 2304) return launch_prefill<5120, 2304>(d, rows, a, l, g, s);
  if (d->hidden == 512 && d->inter == 256) return launch_prefill<512, 256>(d, rows, a, l, g, s);
  return MOE_ESHAPE;
}

int quant(const void* x, int rows, int K, void* codes, void* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ESHAPE;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_EINVAL;
  const int nb = (rows * (K / 32) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_quant, dim3(nb), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), rows, K, static_cast<uint8_t*>(codes),
                     static_cast<uint8_t*>(scales));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

}  // namespace pf
}  // namespace moe
