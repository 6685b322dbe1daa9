// Per-format decode-and-dot engines for the gfx950 expert kernels.
//
// Every engine works on "units": a fixed run of consecutive weights of one
// matrix row whose codes one lane fetches with a single 16-byte load (Q8:
// two).  Activations are staged once per workgroup in LDS as an "x' record"
// per unit: f16 pairs ordered and pre-scaled so that a code, dropped into the
// mantissa of an f16 1.0 by one AND-OR, multiplies its activation with one
// v_dot2c_f32_f16:
//
//   decoded pair value   v = 1 + c * 2^(p-10)          (c: code at bit p)
//   record pair value    x' = f16(sigma * x * 2^(10-p)) (sigma: power of two)
//   sum_i v_i x'_i       = sum_i x'_i + sum_i c_i x~_i,  x~_i = x'_i 2^(p_i-10)
//
// so the block's true dot product sum_i (c_i - OFF) x~_i is the dot2 chain
// minus S = sum_i x~_i (2^(10-p_i) + OFF), which the record carries.  S is
// built from the rounded x' values, so the large offset term cancels exactly.
// The result is then scaled by the block scale and, at the end, by 1/sigma.
//
// The code offsets and block scales are those of the formats defined in
// include/moe.h ("[Strata] DeepSeek V4.1 Flash on a single 4090", section
// 5.1 names the ternary / Q2_0 / Q3 formats and their bit rates; OCP MX v1.0
// defines e2m1 / e8m0; Q8_0 is the dense-half format of section 2).
#pragma once
#include "dev_common.h"

namespace moe {
namespace dev {

constexpr uint32_t kMag = 0x3C003C00u;  // f16 1.0 in both halves

// Records are built in sub-units (SUBS per unit, SUBV values each) so one
// thread holds only a few values; each sub-unit writes its own pairs and its
// own partial S (the dot sums the partials).

__device__ __forceinline__ void rec_store(uint8_t* rec, int dw, uint32_t v) {
  reinterpret_cast<uint32_t*>(rec)[dw] = v;
}

// f16(g * v * 2^(10-p)) for a pair (g: the row's power-of-two sigma);
// accumulates S += x~ * (2^(10-p) + off) = x' * (1 + off * 2^(p-10)) over the
// pair with one dot2: the factor is exact in f16 for every format's (p, off),
// so both products are exact and S sees the rounded x' values, as the dot does.
__device__ __forceinline__ uint32_t make_pair(float lo, float hi, float g, int p, float off, float& s) {
  const float sc = g * __builtin_ldexpf(1.0f, 10 - p);
  const uint32_t pr = pack_h2(lo * sc, hi * sc);
  const float k = 1.0f + off * __builtin_ldexpf(1.0f, p - 10);
  s = dot2(pr, pack_h2(k, k), s);
  return pr;
}

// =========================================================================
// Q2_0: unit = one block of 64 weights, 16 code bytes + fp16 d.
// Per code dword w (codes i at bits 2i), pair (i, i+8) is taken from
// w << 4 (i = 0,1,2 at p = 4,6,8), w (i = 3,4 at p = 6,8) or
// w >> 6 (i = 5,6,7 at p = 4,6,8).
// =========================================================================
struct FmtQ2 {
  static constexpr uint32_t bytes(int n, int k) { return static_cast<uint32_t>(n * (k / 64) * 18); }
  static constexpr int TAG = 2;
  static constexpr int UNIT = 64, XREC = 144, PSHIFT = 6, SUBS = 4, SUBV = 16;
  static constexpr int units(int k) { return k / 64; }
  static constexpr int kP[8] = {4, 6, 8, 6, 8, 4, 6, 8};
  struct Raw {
    uint32_t c[4];
    uint32_t s;
  };
  __device__ static __forceinline__ void load(Raw& r, const Buf& m, int nrows, int nbu, int n,
                                              int b) {
    const uint32_t bi = static_cast<uint32_t>(n * nbu + b);
    const u32x4 q = bload128(m, bi * 16u);
    r.c[0] = q.x; r.c[1] = q.y; r.c[2] = q.z; r.c[3] = q.w;
    r.s = bload16(m, static_cast<uint32_t>(nrows * nbu * 16) + bi * 2u);
  }
  // sub-unit d = code dword d: values 16d .. 16d+15
  __device__ static __forceinline__ void prep_sub(const float (&v)[16], float g, int d, uint8_t* rec) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) rec_store(rec, d * 8 + i, make_pair(v[i], v[i + 8], g, kP[i], 2.0f, s));
    reinterpret_cast<float*>(rec)[32 + d] = s;
  }
  template <int RT, int NT>
  __device__ static __forceinline__ void dot(const Raw (&raw)[RT], const uint8_t* xr, int rstride,
                                             int nt, float (&acc)[RT][NT]) {
    constexpr uint32_t M4 = 0x00300030u, M6 = 0x00C000C0u, M8 = 0x03000300u;
    float bd[RT][NT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) bd[r][t] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t pr[RT][8];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const uint32_t w = raw[r].c[d], wl = w << 4, wr = w >> 6;
        pr[r][0] = andor(wl, M4, kMag);
        pr[r][1] = andor(wl, M6, kMag);
        pr[r][2] = andor(wl, M8, kMag);
        pr[r][3] = andor(w, M6, kMag);
        pr[r][4] = andor(w, M8, kMag);
        pr[r][5] = andor(wr, M4, kMag);
        pr[r][6] = andor(wr, M6, kMag);
        pr[r][7] = andor(wr, M8, kMag);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          const uint4 xa = *reinterpret_cast<const uint4*>(xr + t * rstride + d * 32);
          const uint4 xb = *reinterpret_cast<const uint4*>(xr + t * rstride + d * 32 + 16);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            float a = bd[r][t];
            a = dot2(pr[r][0], xa.x, a);
            a = dot2(pr[r][1], xa.y, a);
            a = dot2(pr[r][2], xa.z, a);
            a = dot2(pr[r][3], xa.w, a);
            a = dot2(pr[r][4], xb.x, a);
            a = dot2(pr[r][5], xb.y, a);
            a = dot2(pr[r][6], xb.z, a);
            a = dot2(pr[r][7], xb.w, a);
            bd[r][t] = a;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        const float4 sp = *reinterpret_cast<const float4*>(xr + t * rstride + 128);
        const float S = (sp.x + sp.y) + (sp.z + sp.w);
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][t] = fmaf(f16_bits_to_f32(raw[r].s), bd[r][t] - S, acc[r][t]);
      }
    }
  }
};

// =========================================================================
// Q8: unit = one block of 32 int8 + fp16 d.  Codes are biased to
// u = q + 128 (xor 0x80 per byte); bytes (0,2) and (1,3) of a dword become
// f16 pairs at p = 2 via (w << 2) and (w >> 6).
// =========================================================================
struct FmtQ8 {
  static constexpr uint32_t bytes(int n, int k) { return static_cast<uint32_t>(n * (k / 32) * 34); }
  static constexpr int TAG = 5;
  static constexpr int UNIT = 32, XREC = 80, PSHIFT = 8, SUBS = 2, SUBV = 16;
  static constexpr int units(int k) { return k / 32; }
  struct Raw {
    uint32_t c[8];
    uint32_t s;
  };
  __device__ static __forceinline__ void load(Raw& r, const Buf& m, int nrows, int nbu, int n,
                                              int b) {
    const uint32_t bi = static_cast<uint32_t>(n * nbu + b);
    const u32x4 q0 = bload128(m, bi * 32u);
    const u32x4 q1 = bload128(m, bi * 32u + 16u);
    r.c[0] = q0.x; r.c[1] = q0.y; r.c[2] = q0.z; r.c[3] = q0.w;
    r.c[4] = q1.x; r.c[5] = q1.y; r.c[6] = q1.z; r.c[7] = q1.w;
    r.s = bload16(m, static_cast<uint32_t>(nrows * nbu * 32) + bi * 2u);
  }
  // sub-unit h = code dwords 4h .. 4h+3: values 16h .. 16h+15
  __device__ static __forceinline__ void prep_sub(const float (&v)[16], float g, int h, uint8_t* rec) {
    float s = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      rec_store(rec, 8 * h + 2 * d, make_pair(v[4 * d], v[4 * d + 2], g, 2, 128.0f, s));
      rec_store(rec, 8 * h + 2 * d + 1, make_pair(v[4 * d + 1], v[4 * d + 3], g, 2, 128.0f, s));
    }
    reinterpret_cast<float*>(rec)[16 + h] = s;
  }
  template <int RT, int NT>
  __device__ static __forceinline__ void dot(const Raw (&raw)[RT], const uint8_t* xr, int rstride,
                                             int nt, float (&acc)[RT][NT]) {
    constexpr uint32_t M = 0x03FC03FCu;
    float bd[RT][NT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) bd[r][t] = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t pr[RT][8];
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t w = raw[r].c[4 * h + d] ^ 0x80808080u;
          pr[r][2 * d] = andor(w << 2, M, kMag);
          pr[r][2 * d + 1] = andor(w >> 6, M, kMag);
        }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          const uint4 xa = *reinterpret_cast<const uint4*>(xr + t * rstride + h * 32);
          const uint4 xb = *reinterpret_cast<const uint4*>(xr + t * rstride + h * 32 + 16);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            float a = bd[r][t];
            a = dot2(pr[r][0], xa.x, a);
            a = dot2(pr[r][1], xa.y, a);
            a = dot2(pr[r][2], xa.z, a);
            a = dot2(pr[r][3], xa.w, a);
            a = dot2(pr[r][4], xb.x, a);
            a = dot2(pr[r][5], xb.y, a);
            a = dot2(pr[r][6], xb.z, a);
            a = dot2(pr[r][7], xb.w, a);
            bd[r][t] = a;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        const float2 sp = *reinterpret_cast<const float2*>(xr + t * rstride + 64);
        const float S = sp.x + sp.y;
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][t] = fmaf(f16_bits_to_f32(raw[r].s), bd[r][t] - S, acc[r][t]);
      }
    }
  }
};

// =========================================================================
// MXFP4: unit = one block of 32 e2m1 + e8m0.  v_cvt_scalef32_pk_f16_fp4
// turns the two nibbles of one code byte into an exact f16 pair (scale 1);
// the block scale 2^(E-127) is applied to the fp32 block sum.
// =========================================================================
struct FmtMXFP4 {
  static constexpr uint32_t bytes(int n, int k) { return static_cast<uint32_t>(n * (k / 32) * 17); }
  static constexpr int TAG = 4;
  static constexpr int UNIT = 32, XREC = 80, PSHIFT = 0, SUBS = 2, SUBV = 16;
  static constexpr int units(int k) { return k / 32; }
  struct Raw {
    uint32_t c[4];
    uint32_t s;
  };
  __device__ static __forceinline__ void load(Raw& r, const Buf& m, int nrows, int nbu, int n,
                                              int b) {
    const uint32_t bi = static_cast<uint32_t>(n * nbu + b);
    const u32x4 q = bload128(m, bi * 16u);
    r.c[0] = q.x; r.c[1] = q.y; r.c[2] = q.z; r.c[3] = q.w;
    r.s = bload8(m, static_cast<uint32_t>(nrows * nbu * 16) + bi);
  }
  __device__ static __forceinline__ void prep_sub(const float (&v)[16], float g, int h, uint8_t* rec) {
#pragma unroll
    for (int k = 0; k < 8; ++k) rec_store(rec, 8 * h + k, pack_h2(v[2 * k] * g, v[2 * k + 1] * g));
  }
  template <int RT, int NT>
  __device__ static __forceinline__ void dot(const Raw (&raw)[RT], const uint8_t* xr, int rstride,
                                             int nt, float (&acc)[RT][NT]) {
    float bd[RT][NT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) bd[r][t] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t pr[RT][4];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        pr[r][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[r].c[d], 1.0f, 0));
        pr[r][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[r].c[d], 1.0f, 1));
        pr[r][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[r].c[d], 1.0f, 2));
        pr[r][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[r].c[d], 1.0f, 3));
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          const uint4 xa = *reinterpret_cast<const uint4*>(xr + t * rstride + d * 16);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            float a = bd[r][t];
            a = dot2(pr[r][0], xa.x, a);
            a = dot2(pr[r][1], xa.y, a);
            a = dot2(pr[r][2], xa.z, a);
            a = dot2(pr[r][3], xa.w, a);
            bd[r][t] = a;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r][t] = fmaf(__builtin_ldexpf(1.0f, static_cast<int>(raw[r].s) - 127), bd[r][t], acc[r][t]);
      }
    }
  }
};

// =========================================================================
// TERN160: unit = half a block: 16 code bytes = 80 trits; the block's fp16
// d is shared by its two units.  Each code byte is looked up in an LDS table
// that spreads its five digits (t + 1) into f16 mantissa fields:
// digit0 -> bits 8, digit1 -> 24, digit2 -> 6, digit3 -> 22, digit4 -> 4 and 20.
// Per pair of bytes (A, B): (t0,t1)_A, (t2,t3)_A, (t0,t1)_B, (t2,t3)_B at
// p = 8,6,8,6 and (t4_A, t4_B) at p = 4.
// =========================================================================
struct FmtTern {
  static constexpr uint32_t bytes(int n, int k) { return static_cast<uint32_t>(n * ((k + 159) / 160) * 34); }
  static constexpr int TAG = 1;
  static constexpr int UNIT = 80, XREC = 176, PSHIFT = 6, SUBS = 4, SUBV = 20;
  static constexpr int units(int k) { return 2 * ((k + 159) / 160); }
  struct Raw {
    uint32_t c[4];
    uint32_t s;
  };
  __device__ static __forceinline__ void load(Raw& r, const Buf& m, int nrows, int nbu, int n,
                                              int b) {
    const uint32_t bi = static_cast<uint32_t>(n * nbu + b);  // unit index; block = unit / 2
    const u32x4 q = bload128(m, bi * 16u);
    r.c[0] = q.x; r.c[1] = q.y; r.c[2] = q.z; r.c[3] = q.w;
    r.s = bload16(m, static_cast<uint32_t>(nrows * nbu * 16) + (bi >> 1) * 2u);
  }
  // table entry for byte value b (< 243); larger values decode as all-zero trits
  __device__ static __forceinline__ uint32_t table_entry(int b) {
    int d[5] = {1, 1, 1, 1, 1};
    if (b < 243) {
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        d[m] = b % 3;
        b /= 3;
      }
    }
    return (static_cast<uint32_t>(d[0]) << 8) | (static_cast<uint32_t>(d[1]) << 24) |
           (static_cast<uint32_t>(d[2]) << 6) | (static_cast<uint32_t>(d[3]) << 22) |
           (static_cast<uint32_t>(d[4]) << 4) | (static_cast<uint32_t>(d[4]) << 20);
  }
  // sub-unit q = code dword q = byte pairs 2q, 2q+1: values 20q .. 20q+19
  __device__ static __forceinline__ void prep_sub(const float (&vv)[20], float g, int q, uint8_t* rec) {
    float s = 0.0f;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = 2 * q + mm;
      const float* v = vv + 10 * mm;
      rec_store(rec, 5 * m + 0, make_pair(v[0], v[1], g, 8, 1.0f, s));
      rec_store(rec, 5 * m + 1, make_pair(v[2], v[3], g, 6, 1.0f, s));
      rec_store(rec, 5 * m + 2, make_pair(v[5], v[6], g, 8, 1.0f, s));
      rec_store(rec, 5 * m + 3, make_pair(v[7], v[8], g, 6, 1.0f, s));
      rec_store(rec, 5 * m + 4, make_pair(v[4], v[9], g, 4, 1.0f, s));
    }
    reinterpret_cast<float*>(rec)[40 + q] = s;
  }
  template <int RT, int NT>
  __device__ static __forceinline__ void dot(const Raw (&raw)[RT], const uint8_t* xr, int rstride,
                                             int nt, float (&acc)[RT][NT], const uint32_t* table) {
    constexpr uint32_t M01 = 0x03000300u, M23 = 0x00C000C0u, M4A = 0x00000030u, M4B = 0x00300000u;
    float bd[RT][NT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) bd[r][t] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {           // code dword q = bytes 4q..4q+3 = byte pairs 2q, 2q+1
      uint32_t pr[RT][10];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const uint32_t w = raw[r].c[q];
        const uint32_t t0 = table[w & 0xFFu], t1 = table[(w >> 8) & 0xFFu];
        const uint32_t t2 = table[(w >> 16) & 0xFFu], t3 = table[w >> 24];
        pr[r][0] = andor(t0, M01, kMag);
        pr[r][1] = andor(t0, M23, kMag);
        pr[r][2] = andor(t1, M01, kMag);
        pr[r][3] = andor(t1, M23, kMag);
        pr[r][4] = andor(t1, M4B, andor(t0, M4A, kMag));
        pr[r][5] = andor(t2, M01, kMag);
        pr[r][6] = andor(t2, M23, kMag);
        pr[r][7] = andor(t3, M01, kMag);
        pr[r][8] = andor(t3, M23, kMag);
        pr[r][9] = andor(t3, M4B, andor(t2, M4A, kMag));
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          const uint32_t* x = reinterpret_cast<const uint32_t*>(xr + t * rstride) + 10 * q;
          uint32_t xv[10];
#pragma unroll
          for (int i = 0; i < 10; ++i) xv[i] = x[i];
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            float a = bd[r][t];
#pragma unroll
            for (int i = 0; i < 10; ++i) a = dot2(pr[r][i], xv[i], a);
            bd[r][t] = a;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        const float4 sp = *reinterpret_cast<const float4*>(xr + t * rstride + 160);
        const float S = (sp.x + sp.y) + (sp.z + sp.w);
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][t] = fmaf(f16_bits_to_f32(raw[r].s), bd[r][t] - S, acc[r][t]);
      }
    }
  }
};

// =========================================================================
// Q3: unit = a quarter block: 64 weights = 4 sub-blocks of 16; 24 code bytes
// (six words), the block's fp16 d and the unit's four 6-bit sub-scales (24
// bits of the 96).  Pair i of sub-block j is (weight i, weight i+8); its
// codes are 3-bit fields at the same place in both halves of a word: field f
// at bit 1 + 3f.  Pairs 0-2 of every sub-block sit in fields 0 / 3 (p = 1),
// pairs 3-5 in fields 1 / 4 (p = 4), pairs 6-7 in field 2 (p = 7) or, for
// the last two of the unit, spread over bit 0 of each half of three words
// (assembled at p = 7).  Fields 0-2 are taken in place, 3-4 from the word
// shifted right by 9: one v_and_or_b32 per pair, and every pair's p depends
// only on its index in the sub-block, so records are built with constant
// scales.
// =========================================================================
struct FmtQ3 {
  static constexpr uint32_t bytes(int n, int k) { return static_cast<uint32_t>(n * (k / 256) * 110); }
  static constexpr int TAG = 3;
  static constexpr int UNIT = 64, XREC = 144, PSHIFT = 9, SUBS = 4, SUBV = 16;
  static constexpr int units(int k) { return k / 64; }
  static constexpr int kP[8] = {1, 1, 1, 4, 4, 4, 7, 7};
  struct Raw {
    uint32_t c[6];
    uint32_t d;
    uint32_t u24;  // the unit's four 6-bit sub-scales
  };
  __device__ static __forceinline__ void load(Raw& r, const Buf& m, int nrows, int nbu, int n,
                                              int b) {
    const uint32_t ku = static_cast<uint32_t>(b & 3);
    const uint32_t nb = static_cast<uint32_t>(nbu) >> 2;
    const uint32_t blk = static_cast<uint32_t>(n) * nb + static_cast<uint32_t>(b >> 2);
    const u32x4 l = bload128(m, blk * 96u + 24u * ku);
    const u32x2 h = bload64(m, blk * 96u + 24u * ku + 16u);
    r.c[0] = l.x; r.c[1] = l.y; r.c[2] = l.z; r.c[3] = l.w;
    r.c[4] = h.x; r.c[5] = h.y;
    const uint32_t dplane = static_cast<uint32_t>(nrows) * nb * 96u;
    r.d = bload16(m, dplane + blk * 2u);
    const uint32_t w0 = ku >= 2 ? 1u : 0u;
    const uint32_t uo = dplane + static_cast<uint32_t>(nrows) * nb * 2u + blk * 12u + 4u * w0;
    const uint32_t u0 = bload32(m, uo);
    const uint32_t u1 = bload32(m, uo + 4u);
    const uint64_t pair = static_cast<uint64_t>(u0) | (static_cast<uint64_t>(u1) << 32);
    r.u24 = static_cast<uint32_t>(pair >> (24u * ku - 32u * w0)) & 0xFFFFFFu;
  }
  // sub-unit j = sub-block j: values 16j .. 16j+15
  __device__ static __forceinline__ void prep_sub(const float (&v)[16], float g, int j, uint8_t* rec) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) rec_store(rec, j * 8 + i, make_pair(v[i], v[i + 8], g, kP[i], 4.0f, s));
    reinterpret_cast<float*>(rec)[32 + j] = s;
  }
  // the f16 pair of pair i of sub-block j (both compile-time after unrolling)
  __device__ static __forceinline__ uint32_t pair_of(const uint32_t (&w)[6], const uint32_t (&sp)[2], int j,
                                                     int i) {
    constexpr uint32_t F0 = 0x000E000Eu, F1 = 0x00700070u, F2 = 0x03800380u;
    if (i < 6) {
      const int q = 3 * j + i % 3, m = q % 6;
      const uint32_t mask = i < 3 ? F0 : F1;
      return andor(q < 6 ? w[m] : w[m] >> 9, mask, kMag);
    }
    const int q = 2 * j + i - 6;
    return q < 6 ? andor(w[q], F2, kMag) : sp[q - 6];
  }
  template <int RT, int NT>
  __device__ static __forceinline__ void dot(const Raw (&raw)[RT], const uint8_t* xr, int rstride,
                                             int nt, float (&acc)[RT][NT]) {
    uint32_t sp[RT][2];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        sp[r][q] = andor(raw[r].c[3 * q] << 7, 0x00800080u,
                         andor(raw[r].c[3 * q + 1] << 8, 0x01000100u,
                               andor(raw[r].c[3 * q + 2] << 9, 0x02000200u, kMag)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float bd[RT][NT];
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) bd[r][t] = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          const uint4 xa = *reinterpret_cast<const uint4*>(xr + t * rstride + j * 32);
          const uint4 xb = *reinterpret_cast<const uint4*>(xr + t * rstride + j * 32 + 16);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            float a = 0.0f;
            a = dot2(pair_of(raw[r].c, sp[r], j, 0), xa.x, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 1), xa.y, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 2), xa.z, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 3), xa.w, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 4), xb.x, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 5), xb.y, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 6), xb.z, a);
            a = dot2(pair_of(raw[r].c, sp[r], j, 7), xb.w, a);
            bd[r][t] = a;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          const float S = *reinterpret_cast<const float*>(xr + t * rstride + 128 + 4 * j);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            const int sj = static_cast<int>((raw[r].u24 >> (6 * j)) & 63u) - 32;
            const float ds = f16_bits_to_f32(raw[r].d) * static_cast<float>(sj);
            acc[r][t] = fmaf(ds, bd[r][t] - S, acc[r][t]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

}  // namespace dev
}  // namespace moe
