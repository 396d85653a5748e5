// E4M3FN weight bytes decoded to bf16 in registers.  Every finite E4M3 value
// (4 significant bits, exponents 2^-9 .. 2^8) is a bf16 number, so the decode is
// exact; the per-tensor fp32 scale is applied to the fp32 accumulator.  The
// format is one of the released precision mix ("Nemotron 3.5 Super and
// Lightning", section on keeping accuracy under 4-bit quantisation).
#pragma once
#include "common.hpp"

namespace lmoe {

// bytes 2*SEL and 2*SEL+1 of w -> two bf16 in one word (lower byte in the low half);
// the gfx950 conversion with a unit scale
template <bool SEL>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL));
}

// bytes 2*SEL and 2*SEL+1 of w as E4M3FN -> two fp32 (exact), e.g. FP4 block scales
template <bool SEL>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, SEL);
}

// eight E4M3FN bytes (w0 = bytes 0..3, w1 = bytes 4..7) -> eight bf16
__device__ __forceinline__ u32x4_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4_t r;
  r[0] = fp8x2_to_bf16<false>(w0);
  r[1] = fp8x2_to_bf16<true>(w0);
  r[2] = fp8x2_to_bf16<false>(w1);
  r[3] = fp8x2_to_bf16<true>(w1);
  return r;
}

}  // namespace lmoe
