// Block-scaled FP4 (E2M1 values, one E4M3 scale per 16 input-dim elements)
// decoded to bf16 in registers.  Format: "Nemotron 3 Super", section 3.6 (a
// per-tensor and a per-block scale); "Nemotron 3 Ultra" (E2M1 elements, E4M3
// block scales).  Every E2M1 value times every E4M3 scale is a bf16 number,
// so the decoded operand is exact; the per-tensor fp32 scale is applied to the
// fp32 accumulator instead.
#pragma once
#include "common.hpp"

namespace lmoe {

// FP4 E2M1 nibble -> fp32 bits (sign, 2-bit exponent with bias 1, 1-bit mantissa)
__device__ __forceinline__ uint32_t e2m1_f32_bits(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  return mag | ((c & 8u) << 28);
}

// eight E2M1 codes (low nibble first) times a block scale -> eight bf16 (exact)
__device__ __forceinline__ u32x4_t fp4x8_to_bf16(uint32_t codes, float scale) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __uint_as_float(e2m1_f32_bits((codes >> (8 * i)) & 15u)) * scale;
    const float b = __uint_as_float(e2m1_f32_bits((codes >> (8 * i + 4)) & 15u)) * scale;
    // the products are bf16 numbers, so dropping the low half is exact
    r[i] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
  }
  return r;
}

}  // namespace lmoe
