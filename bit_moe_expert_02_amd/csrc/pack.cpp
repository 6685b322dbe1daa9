// Host-side packer / unpacker for the library's low-bit weight formats.
//
// Formats (block layouts defined in include/moe.h): Q2_0, TERN160, Q3, MXFP4
// (OCP MX v1.0 e2m1 + e8m0), Q8.  The pages name the formats and their bit
// rates ("[Strata] DeepSeek V4.1 Flash on a single 4090", section 5.1 table;
// "DeepSeek-V4.1-Flash served three ways on 4xL20", section 1 for the FP4
// experts with a per-32 scale); the RTN rules below are this library's.
//
// All packing arithmetic is IEEE fp32 with round-to-nearest-even, and fp16
// conversion is round-to-nearest-even with saturation at +-65504, so the
// bytes produced are a pure function of the fp32 input.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "host_common.h"

namespace moe {

// ---------------------------------------------------------------- fp16
uint16_t f32_to_f16_sat(float f) {
  if (f > 65504.0f) f = 65504.0f;
  if (f < -65504.0f) f = -65504.0f;
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax > 0x7f800000u) return static_cast<uint16_t>(sign | 0x7e00u);  // NaN
  const int e = static_cast<int>(ax >> 23);
  const uint32_t m = (ax & 0x7fffffu) | 0x800000u;                    // 24-bit significand
  if (e >= 113) {                                                     // |f| >= 2^-14: normal
    uint32_t h = (static_cast<uint32_t>(e - 112) << 10) | ((ax & 0x7fffffu) >> 13);
    const uint32_t rem = ax & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;           // may carry into exponent
    return static_cast<uint16_t>(sign | h);
  }
  if (e < 102) return static_cast<uint16_t>(sign);                    // below half the smallest subnormal
  const int s = 126 - e;                                              // value = m * 2^(e-150) = h * 2^-24
  uint32_t h = m >> s;
  const uint32_t rem = m & ((1u << s) - 1u), half = 1u << (s - 1);
  if (rem > half || (rem == half && (h & 1u))) ++h;
  return static_cast<uint16_t>(sign | h);
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  float v;
  if (e == 0) {
    v = std::ldexp(static_cast<float>(m), -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<float>(m | 1024u), static_cast<int>(e) - 25);
  }
  uint32_t b;
  std::memcpy(&b, &v, 4);
  b |= sign;
  std::memcpy(&v, &b, 4);
  return v;
}

// ---------------------------------------------------------------- shapes
FormatInfo format_info(int fmt) {
  switch (fmt) {
    case MOE_FMT_Q2_0: return {64, 16, 2};
    case MOE_FMT_TERN160: return {160, 32, 2};
    case MOE_FMT_Q3: return {256, 96, 14};
    case MOE_FMT_MXFP4: return {32, 16, 1};
    case MOE_FMT_Q8: return {32, 32, 2};
    default: return {0, 0, 0};
  }
}

int64_t blocks_per_row(int fmt, int64_t k) {
  const FormatInfo fi = format_info(fmt);
  if (fi.block == 0 || k <= 0) return -1;
  if (fmt != MOE_FMT_TERN160 && k % fi.block) return -1;
  return (k + fi.block - 1) / fi.block;
}

size_t packed_bytes(int fmt, int64_t n, int64_t k) {
  const int64_t nb = blocks_per_row(fmt, k);
  if (nb < 0 || n <= 0) return 0;
  const FormatInfo fi = format_info(fmt);
  return static_cast<size_t>(n) * static_cast<size_t>(nb) * (fi.code_bytes + fi.scale_bytes);
}

namespace {

template <class F>
void parallel_rows(int64_t n, int nthreads, F&& body) {
  int t = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  t = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(t, n)));
  if (t == 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (n + t - 1) / t;
  for (int i = 0; i < t; ++i) {
    const int64_t a = i * per, b = std::min(n, a + per);
    if (a < b) pool.emplace_back([&body, a, b] { body(a, b); });
  }
  for (auto& th : pool) th.join();
}

inline float rintf_even(float v) { return std::nearbyint(v); }   // default mode: ties to even

inline float div_or_zero(float w, float d) { return d == 0.0f ? 0.0f : w / d; }

// Q3 code bit b of weight i (0..255) of a block, as a bit index into the
// block's 96 code bytes.  By quarter block u (64 weights, six little-endian
// words at byte 24u): weight t of the quarter's sub-block j is in half
// h = t / 8 of pair p = t % 8; field f of a word is the 3 bits at 16h + 1 + 3f.
// Pairs p < 6 go to field p / 3 (+ 3 from the second six on) of word q % 6,
// q = 3j + p % 3; pairs p >= 6 to field 2 of word q = 2j + p - 6 for q < 6,
// else code bit b sits in bit 16h of word 3(q - 6) + b.
inline int q3_code_bit(int i, int b) {
  const int u = i >> 6, w = i & 63, j = w >> 4, t = w & 15, h = t >> 3, p = t & 7;
  if (p < 6) {
    const int q = 3 * j + p % 3, f = p / 3 + (q < 6 ? 0 : 3);
    return 192 * u + 32 * (q % 6) + 16 * h + 1 + 3 * f + b;
  }
  const int q = 2 * j + p - 6;
  if (q < 6) return 192 * u + 32 * q + 16 * h + 1 + 3 * 2 + b;
  return 192 * u + 32 * (3 * (q - 6) + b) + 16 * h;
}

// element of largest magnitude, sign kept; the first one on ties
inline float signed_absmax(const float* b, int n) {
  float best = b[0];
  for (int i = 1; i < n; ++i)
    if (std::fabs(b[i]) > std::fabs(best)) best = b[i];
  return best;
}

inline void put_f16(uint8_t* p, uint16_t h) {
  p[0] = static_cast<uint8_t>(h & 0xff);
  p[1] = static_cast<uint8_t>(h >> 8);
}
inline uint16_t get_f16(const uint8_t* p) { return static_cast<uint16_t>(p[0] | (p[1] << 8)); }

// one block of fp32 inputs (zero padded for the ternary tail)
inline void load_block(const float* row, int64_t k, int64_t start, int bsz, float* out) {
  for (int i = 0; i < bsz; ++i) out[i] = (start + i < k) ? row[start + i] : 0.0f;
}

// --------------------------------------------------------------- packers
void pack_rows(int fmt, const float* w, int64_t n, int64_t k, uint8_t* dst, int64_t r0,
               int64_t r1) {
  const FormatInfo fi = format_info(fmt);
  const int64_t nb = blocks_per_row(fmt, k);
  uint8_t* codes = dst;
  uint8_t* scales = dst + static_cast<size_t>(n * nb) * fi.code_bytes;
  float blk[256];
  for (int64_t r = r0; r < r1; ++r) {
    const float* row = w + r * k;
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t bi = r * nb + b;
      uint8_t* c = codes + bi * fi.code_bytes;
      load_block(row, k, b * fi.block, fi.block, blk);
      std::memset(c, 0, fi.code_bytes);
      switch (fmt) {
        case MOE_FMT_Q2_0: {
          const uint16_t dh = f32_to_f16_sat(signed_absmax(blk, 64) / -2.0f);
          const float d = f16_to_f32(dh);
          for (int i = 0; i < 64; ++i) {
            float q = rintf_even(div_or_zero(blk[i], d)) + 2.0f;
            const int ci = static_cast<int>(std::min(3.0f, std::max(0.0f, q)));
            c[i >> 2] |= static_cast<uint8_t>(ci << ((i & 3) * 2));
          }
          put_f16(scales + bi * 2, dh);
          break;
        }
        case MOE_FMT_TERN160: {
          float amax = 0.0f;
          for (int i = 0; i < 160; ++i) amax = std::max(amax, std::fabs(blk[i]));
          const uint16_t dh = f32_to_f16_sat(amax);
          const float d = f16_to_f32(dh);
          for (int j = 0; j < 32; ++j) {
            int byte = 0, p3 = 1;
            for (int m = 0; m < 5; ++m) {
              float t = rintf_even(div_or_zero(blk[5 * j + m], d));
              t = std::min(1.0f, std::max(-1.0f, t));
              byte += (static_cast<int>(t) + 1) * p3;
              p3 *= 3;
            }
            c[j] = static_cast<uint8_t>(byte);
          }
          put_f16(scales + bi * 2, dh);
          break;
        }
        case MOE_FMT_Q3: {
          float sigma[16], smax = 0.0f;
          for (int j = 0; j < 16; ++j) {
            sigma[j] = signed_absmax(blk + 16 * j, 16) / -4.0f;
            smax = std::max(smax, std::fabs(sigma[j]));
          }
          const uint16_t dh = f32_to_f16_sat(smax / 31.0f);
          const float d = f16_to_f32(dh);
          uint8_t* ub = scales + static_cast<size_t>(n * nb) * 2 + bi * 12;
          std::memset(ub, 0, 12);
          for (int j = 0; j < 16; ++j) {
            float s = rintf_even(div_or_zero(sigma[j], d));
            s = std::min(31.0f, std::max(-31.0f, s));
            const int u = static_cast<int>(s) + 32;
            for (int bit = 0; bit < 6; ++bit)
              if ((u >> bit) & 1) ub[(6 * j + bit) >> 3] |= static_cast<uint8_t>(1u << ((6 * j + bit) & 7));
            const float ds = d * s;
            for (int i = 0; i < 16; ++i) {
              float q = rintf_even(div_or_zero(blk[16 * j + i], ds)) + 4.0f;
              const int qi = static_cast<int>(std::min(7.0f, std::max(0.0f, q)));
              for (int b = 0; b < 3; ++b) {
                const int pos = q3_code_bit(16 * j + i, b);
                c[pos >> 3] |= static_cast<uint8_t>(((qi >> b) & 1) << (pos & 7));
              }
            }
          }
          put_f16(scales + bi * 2, dh);
          break;
        }
        case MOE_FMT_MXFP4: {
          float amax = 0.0f;
          for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(blk[i]));
          int e = 0;
          if (amax > 0.0f) {
            int ex;
            std::frexp(amax, &ex);                              // amax = f * 2^ex, f in [0.5, 1)
            e = std::min(254, std::max(0, (ex - 1) - 2 + 127));
          }
          for (int i = 0; i < 32; ++i) {
            const float v = static_cast<float>(std::ldexp(static_cast<double>(blk[i]), 127 - e));
            const float a = std::fabs(v);
            int code;
            if (a <= 0.25f) code = 0;
            else if (a < 0.75f) code = 1;
            else if (a <= 1.25f) code = 2;
            else if (a < 1.75f) code = 3;
            else if (a <= 2.5f) code = 4;
            else if (a < 3.5f) code = 5;
            else if (a <= 5.0f) code = 6;
            else code = 7;
            if (std::signbit(v)) code |= 8;
            c[i >> 1] |= static_cast<uint8_t>(code << ((i & 1) * 4));
          }
          scales[bi] = static_cast<uint8_t>(e);
          break;
        }
        case MOE_FMT_Q8: {
          float amax = 0.0f;
          for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(blk[i]));
          const uint16_t dh = f32_to_f16_sat(amax / 127.0f);
          const float d = f16_to_f32(dh);
          for (int i = 0; i < 32; ++i) {
            float q = rintf_even(div_or_zero(blk[i], d));
            q = std::min(127.0f, std::max(-127.0f, q));
            c[i] = static_cast<uint8_t>(static_cast<int8_t>(q));
          }
          put_f16(scales + bi * 2, dh);
          break;
        }
      }
    }
  }
}

// --------------------------------------------------------------- unpack
const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

}  // namespace

// Rows [r0, r1) of a packed [n x k] matrix decoded to fp32 (exact), row r at
// out + (r - r0) * k.  False if a code is invalid.
bool unpack_rows(int fmt, const uint8_t* src, int64_t n, int64_t k, float* out, int64_t r0, int64_t r1) {
  const FormatInfo fi = format_info(fmt);
  const int64_t nb = blocks_per_row(fmt, k);
  const uint8_t* codes = src;
  const uint8_t* scales = src + static_cast<size_t>(n * nb) * fi.code_bytes;
  float v[256];
  for (int64_t r = r0; r < r1; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t bi = r * nb + b;
      const uint8_t* c = codes + bi * fi.code_bytes;
      switch (fmt) {
        case MOE_FMT_Q2_0: {
          const float d = f16_to_f32(get_f16(scales + bi * 2));
          for (int i = 0; i < 64; ++i)
            v[i] = d * static_cast<float>(((c[i >> 2] >> ((i & 3) * 2)) & 3) - 2);
          break;
        }
        case MOE_FMT_TERN160: {
          const float d = f16_to_f32(get_f16(scales + bi * 2));
          for (int j = 0; j < 32; ++j) {
            int byte = c[j];
            if (byte > 242) return false;
            for (int m = 0; m < 5; ++m) {
              v[5 * j + m] = d * static_cast<float>(byte % 3 - 1);
              byte /= 3;
            }
          }
          break;
        }
        case MOE_FMT_Q3: {
          const float d = f16_to_f32(get_f16(scales + bi * 2));
          const uint8_t* ub = scales + static_cast<size_t>(n * nb) * 2 + bi * 12;
          for (int j = 0; j < 16; ++j) {
            int u = 0;
            for (int bit = 0; bit < 6; ++bit) u |= ((ub[(6 * j + bit) >> 3] >> ((6 * j + bit) & 7)) & 1) << bit;
            const float ds = d * static_cast<float>(u - 32);                 // exact: 11 x 6 bits
            for (int i = 0; i < 16; ++i) {
              const int wi = 16 * j + i;
              int q = 0;
              for (int b = 0; b < 3; ++b) {
                const int pos = q3_code_bit(wi, b);
                q |= ((c[pos >> 3] >> (pos & 7)) & 1) << b;
              }
              v[wi] = ds * static_cast<float>(q - 4);                         // exact: 17 x 3 bits
            }
          }
          break;
        }
        case MOE_FMT_MXFP4: {
          const int e = scales[bi];
          if (e == 255) return false;
          for (int i = 0; i < 32; ++i) {
            const int code = (c[i >> 1] >> ((i & 1) * 4)) & 15;
            const double mag = std::ldexp(static_cast<double>(kE2M1[code & 7]), e - 127);
            v[i] = static_cast<float>((code & 8) ? -mag : mag);               // exact: >= 2^-128
          }
          break;
        }
        case MOE_FMT_Q8: {
          const float d = f16_to_f32(get_f16(scales + bi * 2));
          for (int i = 0; i < 32; ++i) v[i] = d * static_cast<float>(static_cast<int8_t>(c[i]));
          break;
        }
      }
      const int64_t start = b * fi.block;
      const int64_t cnt = std::min<int64_t>(fi.block, k - start);
      std::memcpy(out + (r - r0) * k + start, v, static_cast<size_t>(cnt) * sizeof(float));
    }
  }
  return true;
}

}  // namespace moe

extern "C" size_t moe_packed_bytes(int fmt, int64_t n, int64_t k) {
  return moe::packed_bytes(fmt, n, k);
}

extern "C" int moe_pack(int fmt, const float* w, int64_t n, int64_t k, void* dst,
                        size_t dst_bytes, int nthreads) {
  if (moe::format_info(fmt).block == 0) return MOE_EFORMAT;
  if (!w || !dst || n <= 0 || k <= 0) return MOE_EINVAL;
  const size_t need = moe::packed_bytes(fmt, n, k);
  if (need == 0) return MOE_ESHAPE;
  if (dst_bytes < need) return MOE_EINVAL;
  moe::parallel_rows(n, nthreads, [&](int64_t a, int64_t b) {
    moe::pack_rows(fmt, w, n, k, static_cast<uint8_t*>(dst), a, b);
  });
  return MOE_OK;
}

extern "C" int moe_unpack(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k,
                          float* w, int nthreads) {
  if (moe::format_info(fmt).block == 0) return MOE_EFORMAT;
  if (!w || !src || n <= 0 || k <= 0) return MOE_EINVAL;
  const size_t need = moe::packed_bytes(fmt, n, k);
  if (need == 0) return MOE_ESHAPE;
  if (src_bytes < need) return MOE_EINVAL;
  int t = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  t = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(t, n)));
  std::vector<uint8_t> status(static_cast<size_t>(t), 1);   // one slot per worker
  std::vector<std::thread> pool;
  const int64_t per = (n + t - 1) / t;
  for (int i = 0; i < t; ++i) {
    const int64_t a = i * per, b = std::min(n, a + per);
    if (a >= b) continue;
    pool.emplace_back([&, i, a, b] {
      status[static_cast<size_t>(i)] =
          moe::unpack_rows(fmt, static_cast<const uint8_t*>(src), n, k, w + a * k, a, b) ? 1 : 0;
    });
  }
  for (auto& th : pool) th.join();
  bool good = true;
  for (uint8_t st : status) good = good && st;
  return good ? MOE_OK : MOE_ECODE;
}
