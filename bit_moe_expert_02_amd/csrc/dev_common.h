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
// lane of a group ends with the group's sum.  Up to 16 lanes, DPP moves inside
// a row: quad swaps, then half-row and full-row mirrors.
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
  // wider groups leave the 16-lane row: lane permutes through LDS hardware
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Values every lane holds equally (read from LDS or computed from them),
// moved to scalar registers so addresses built on them stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}



typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A packed matrix as a buffer resource: a wave-uniform descriptor in scalar
// registers, addressed with 32-bit vector offsets.  Reads at or past `bytes`
// return zero instead of touching memory.
struct Buf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ Buf make_buf(const uint8_t* base, uint32_t bytes) {
  void* u = reinterpret_cast<void*>(uniform(reinterpret_cast<uint64_t>(base)));
  return Buf{__builtin_amdgcn_make_buffer_rsrc(u, 0, static_cast<int>(bytes), 0x00020000)};
}
__device__ __forceinline__ u32x4 bload128(const Buf& b, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, 0);
  return u32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ u32x2 bload64(const Buf& b, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(b.r, off, 0, 0);
  return u32x2{v[0], v[1]};
}
__device__ __forceinline__ uint32_t bload32(const Buf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(b.r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload16(const Buf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(b.r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(const Buf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(b.r, off, 0, 0);
}

// The work-item id through an empty asm statement.  Values derived from it are
// then computed where they are used: left to itself, the compiler hoists every
// lane-constant offset of every format's tile code to the kernel entry, where
// they outlive the register cap and are spilled to scratch, and each reload
// costs a memory round trip on the way to the weight loads.
__device__ __forceinline__ int tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Wave-wide (64 lanes) sum of a double via cross-lane shuffles.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One step of an unsigned max across lanes: lanes of rows outside ROWMASK, or
// whose source lane does not exist, take 0, the identity of the max.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, ROWMASK, 0xF, false);
  return v > o ? v : o;
}
// Wave-wide max of a u32; every lane gets it.  Four in-row steps (quad
// swaps, half-row and row mirrors), then the row broadcasts of lanes 15 and 31
// carry the rows' maxima into row 3, whose lane 63 holds the wave's.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v = dpp_max_u32<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v = dpp_max_u32<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_max_u32<0x140, 0xF>(v);   // row_mirror
  v = dpp_max_u32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_u32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// Loads that read what other workgroups published in this kernel (through
// device-scope release/acquire); they bypass non-coherent caches.
// ---------------------------------------------------------------------------
// Tagged words: hand-offs between workgroups of one launch without fences.
// A word is (tag << 32) | payload, written and read with relaxed atomics at
// agent scope, which keep every single word coherent across the XCDs' L2s.
// A consumer takes a word once its tag equals the call's tag, so no ordering
// between different words is needed and no cache write-back is issued.  The
// tag is per call (an epoch kept in the workspace), so words left by earlier
// calls never look ready.
// ---------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 16;   // default polls before a wait gives up (tens of ms)

__device__ __forceinline__ uint64_t tload(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tstore(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// N words at once: addr(j) gives word j's address, or null for none (then its
// payload reads 0).  All loads are issued together; only the words not yet
// carrying `tag` are polled again.  Payloads land in out[].  After `limit`
// polls the wait ends, *err is set to `tag` and false is returned (the
// payloads of the words that never came are stale).
template <int N, class AddrF>
__device__ __forceinline__ bool await_batch(AddrF addr, uint32_t tag, uint32_t* err,
                                            uint32_t (&out)[N], int limit) {
  bool all = true;
  uint64_t w[N];
  const uint64_t ready0 = static_cast<uint64_t>(tag) << 32;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint64_t* p = addr(j);
    w[j] = p ? tload(p) : ready0;
  }
  for (int it = 0;; ++it) {
    all = true;
#pragma unroll
    for (int j = 0; j < N; ++j) all = all && static_cast<uint32_t>(w[j] >> 32) == tag;
    if (all) break;
    if (it >= limit) {
      __hip_atomic_store(err, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (static_cast<uint32_t>(w[j] >> 32) != tag) w[j] = tload(addr(j));
  }
#pragma unroll
  for (int j = 0; j < N; ++j) out[j] = static_cast<uint32_t>(w[j]);
  return all;
}

// await_batch with two polls in flight, for waits whose wave has nothing
// else in flight (twice the registers): the second set of loads is issued
// while the first is out, and each set is issued again as soon as it has been
// checked, so a word is seen about half a round trip sooner.  Every word's
// address must be valid; the words wanted are the bits of `need`.  The loads
// are issued by the whole wave without branches and the loop ends when no
// lane of the wave waits any more, so the compiler counts the loads in flight
// instead of waiting for all of them.
template <int N>
__device__ __forceinline__ void take_ready(const uint64_t (&w)[N], uint32_t tag, uint32_t& done,
                                           uint32_t (&out)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const bool now = !(done >> j & 1u) && static_cast<uint32_t>(w[j] >> 32) == tag;
    out[j] = now ? static_cast<uint32_t>(w[j]) : out[j];
    done |= now ? 1u << j : 0u;
  }
}

template <int N, class AddrF>
__device__ __forceinline__ bool await_batch2(AddrF addr, uint32_t need, uint32_t tag, uint32_t* err,
                                             uint32_t (&out)[N], int limit) {
  static_assert(N < 32, "one bit per word");
  constexpr uint32_t kAll = (1u << N) - 1u;
  uint64_t wa[N], wb[N];
  uint32_t done = ~need & kAll;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    wa[j] = tload(addr(j));
    out[j] = 0;
  }
  // each set is issued again when it returns, so the two stay as far apart
  // as they start: about half a round trip under load (~1.3 us)
  __builtin_amdgcn_s_sleep(48);
#pragma unroll
  for (int j = 0; j < N; ++j) wb[j] = tload(addr(j));
  // both sets are issued again on every pass, and a pass that found the
  // words in the second set ends at the top of the next one, before it waits
  // for anything: no set changes registers on the way round
  bool all = false;
  for (int it = 0;; it += 2) {
    if (all) break;
    take_ready<N>(wa, tag, done, out);
    all = __builtin_amdgcn_ballot_w64(done != kAll) == 0;
    if (all || it >= limit) break;
#pragma unroll
    for (int j = 0; j < N; ++j) wa[j] = tload(addr(j));
    __builtin_amdgcn_sched_barrier(0);   // the first set is out before the second is waited for
    take_ready<N>(wb, tag, done, out);
    all = __builtin_amdgcn_ballot_w64(done != kAll) == 0;
#pragma unroll
    for (int j = 0; j < N; ++j) wb[j] = tload(addr(j));
  }
  if (!all) __hip_atomic_store(err, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return done == kAll;
}

// Payload of *p once it carries `tag`.  After `limit` polls the wait ends,
// *err is set to `tag` and 0 is returned: a launch always drains, and the
// failure is recorded for that call in the error word.
__device__ __forceinline__ uint32_t await_word(const uint64_t* p, uint32_t tag, uint32_t* err,
                                               int limit) {
  for (int i = 0; i < limit; ++i) {
    const uint64_t w = tload(p);
    if (static_cast<uint32_t>(w >> 32) == tag) return static_cast<uint32_t>(w);
    __builtin_amdgcn_s_sleep(8);
  }
  __hip_atomic_store(err, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0u;
}

}  // namespace dev
}  // namespace moe
