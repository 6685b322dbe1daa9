// Device helpers for the gfx950 kernels: f16 pair packing, dot2, DPP
// reductions within a 16-lane row, coherent loads for cross-workgroup data.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace dev {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// fp32 accumulate of a two-element f16 dot product (v_dot2c_f32_f16): both
// products are exact in fp32, so only the accumulation rounds.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// (v & mask) | magic: places two small integer codes into the mantissas of
// two f16 values whose exponent field comes from `magic`.  Written as one
// v_and_or_b32 (the compiler would otherwise split it into an AND and an OR
// with literal operands); mask and magic live in VGPRs.
__device__ __forceinline__ uint32_t andor(uint32_t v, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  f16x2 v;
  v.x = static_cast<_Float16>(lo);  // round to nearest even
  v.y = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float h2_lo(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(f16x2, v).x);
}
__device__ __forceinline__ float h2_hi(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(f16x2, v).y);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}

// Sum of v over groups of LPR consecutive lanes (LPR in {1,2,4,8,16}); every
// lane of a group ends with the group's sum.  DPP moves stay inside a row of
// 16 lanes: quad swaps, then half-row and full-row mirrors.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0xB1, 0xF, 0xF, false));
  if constexpr (LPR >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x4E, 0xF, 0xF, false));
  if constexpr (LPR >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x141, 0xF, 0xF, false));
  if constexpr (LPR >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x140, 0xF, 0xF, false));
  return v;
}

// Wave-wide (64 lanes) sum of a double via cross-lane shuffles.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t w = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64));
    v = v > w ? v : w;
  }
  return v;
}

// Loads that read what other workgroups published in this kernel (through
// device-scope release/acquire); they bypass non-coherent caches.
__device__ __forceinline__ float coherent_load_f32(const float* p) {
  return __builtin_bit_cast(
      float, __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ double coherent_load_f64(const double* p) {
  return __builtin_bit_cast(
      double, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT));
}

}  // namespace dev
}  // namespace moe
