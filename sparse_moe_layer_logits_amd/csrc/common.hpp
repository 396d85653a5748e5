// Shared device helpers for the LatentMoE kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));


// D[16x16] += A[16 x 32] * B[32 x 16] on the matrix cores, bf16 in, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B with eight k values
// (the k set of lane group l / 16); lane l receives D[4*(l/16) + r][l % 16], r = 0..3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bf16 on gfx950's converter (one v_cvt_pk_bf16_f32
// per pair).  For every non-NaN input it returns what the bit formula
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16 gives, denormals and overflow to infinity
// included (all 2^32 patterns compared on the device).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// 128-bit global load / store helpers
__device__ __forceinline__ u32x4_t ld128(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st128(void* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

__device__ __forceinline__ u32x4_t zero128() { u32x4_t z = {0u, 0u, 0u, 0u}; return z; }
