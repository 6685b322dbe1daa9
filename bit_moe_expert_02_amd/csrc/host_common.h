// Host-side helpers shared by the packer and the C-ABI shell.
#pragma once
#include <cstddef>
#include <cstdint>

namespace moe {

struct FormatInfo {
  int block;        // weights per block
  int code_bytes;   // code bytes per block
  int scale_bytes;  // scale bytes per block
};

FormatInfo format_info(int fmt);             // {0,0,0} for an unknown tag
int64_t blocks_per_row(int fmt, int64_t k);  // -1 when K is not allowed
size_t packed_bytes(int fmt, int64_t n, int64_t k);
uint16_t f32_to_f16_sat(float f);
float f16_to_f32(uint16_t h);
// rows [r0, r1) of a packed [n x k] matrix to fp32, row r at out + (r - r0) * k;
// false if a code is invalid
bool unpack_rows(int fmt, const uint8_t* src, int64_t n, int64_t k, float* out, int64_t r0, int64_t r1);

}  // namespace moe
