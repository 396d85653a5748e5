// Block-scaled FP4 (E2M1 values, one E4M3 scale per 16 input-dim elements)
// decoded to bf16 in registers; the E4M3 block scales go through the exact
// hardware FP8 -> fp32 conversion (fp8.hpp).  Format: "Nemotron 3 Super", section 3.6 (a
// per-tensor and a per-block scale); "Nemotron 3 Ultra" (E2M1 elements, E4M3
// block scales).  Every E2M1 value times every E4M3 scale is a bf16 number,
// so the decoded operand is exact; the per-tensor fp32 scale is applied to the
// fp32 accumulator instead.
#pragma once
#include "common.hpp"
#include "fp8.hpp"

namespace lmoe {

// the two E2M1 codes of byte I of `codes` (low nibble first) times a block scale
// -> two bf16 in one word.  The conversion with a unit scale gives the exact
// E2M1 values in fp32; the products are bf16 numbers, so keeping the upper
// halves is exact.
template <int I>
__device__ __forceinline__ uint32_t fp4x2_to_bf16(uint32_t codes, float scale) {
  const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, I);
  const float a = v.x * scale, b = v.y * scale;
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// eight E2M1 codes (low nibble first) times a block scale -> eight bf16 (exact)
__device__ __forceinline__ u32x4_t fp4x8_to_bf16(uint32_t codes, float scale) {
  u32x4_t r;
  r[0] = fp4x2_to_bf16<0>(codes, scale);
  r[1] = fp4x2_to_bf16<1>(codes, scale);
  r[2] = fp4x2_to_bf16<2>(codes, scale);
  r[3] = fp4x2_to_bf16<3>(codes, scale);
  return r;
}

}  // namespace lmoe
