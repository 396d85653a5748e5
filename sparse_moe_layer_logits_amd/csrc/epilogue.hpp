// GEMM epilogues: four consecutive output columns (n .. n+3) of one output row.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace lmoe {

__device__ __forceinline__ void store_bf16x4(void* C, long long off, float a, float b, float c, float d) {
  u32x2_t w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(C) + off) = w;
}

template <int EPI>
__device__ __forceinline__ void epi4(const GemmParams& p, int expert, int split, int row, int n,
                                     f32x4_t v) {
  const long long off = (long long)row * p.ldc + n;
  if constexpr (EPI == EPI_PARTIAL) {
    float* dst = p.partial + (long long)split * p.partial_stride + (long long)row * p.N + n;
    *reinterpret_cast<f32x4_t*>(dst) = v;
  } else if constexpr (EPI == EPI_BF16) {
    store_bf16x4(p.C, off, v[0], v[1], v[2], v[3]);
  } else if constexpr (EPI == EPI_SQRELU_BF16 || EPI == EPI_SQRELU_HILO) {
    const float ts = p.b_tscale ? p.b_tscale[expert] : 1.0f;
    float hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = fmaxf(v[i] * ts, 0.0f);
      const float sq = u * u;
      hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(sq));
      lo[i] = sq - hi[i];
    }
    store_bf16x4(p.C, off, hi[0], hi[1], hi[2], hi[3]);
    if constexpr (EPI == EPI_SQRELU_HILO) store_bf16x4(p.C2, off, lo[0], lo[1], lo[2], lo[3]);
  } else if constexpr (EPI == EPI_BF16_HILO) {
    const float ts = p.b_tscale ? p.b_tscale[expert] : 1.0f;
    float hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = v[i] * ts;
      hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(u));
      lo[i] = u - hi[i];
    }
    store_bf16x4(p.C, off, hi[0], hi[1], hi[2], hi[3]);
    store_bf16x4(p.C2, off, lo[0], lo[1], lo[2], lo[3]);
  } else if constexpr (EPI == EPI_F32) {
    f32x4_t w = v * (p.b_tscale ? p.b_tscale[expert] : 1.0f);
    if (p.bias) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] += p.bias[n + i];
    }
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off) = w;
  } else if constexpr (EPI == EPI_F32_ADD) {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off);
    *dst = *dst + v * (p.b_tscale ? p.b_tscale[expert] : 1.0f);
  } else if constexpr (EPI == EPI_GATE_F32 || EPI == EPI_GATE_BF16) {
    const float ts = p.b_tscale ? p.b_tscale[expert] : 1.0f;
    const float gg = (p.row_scale ? p.row_scale[row] : 1.0f) * ts;
    if constexpr (EPI == EPI_GATE_F32)
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off) = v * gg;
    else
      store_bf16x4(p.C, off, v[0] * gg, v[1] * gg, v[2] * gg, v[3] * gg);
  }
}

// calls f(std::integral_constant<int, EPI>) once for the runtime epilogue kind,
// so a whole tile's stores are compiled per kind without per-element branches
template <class F>
__device__ __forceinline__ void epi_dispatch(int epi, F&& f) {
  switch (epi) {
    case EPI_PARTIAL: f(std::integral_constant<int, EPI_PARTIAL>{}); break;
    case EPI_BF16: f(std::integral_constant<int, EPI_BF16>{}); break;
    case EPI_SQRELU_BF16: f(std::integral_constant<int, EPI_SQRELU_BF16>{}); break;
    case EPI_SQRELU_HILO: f(std::integral_constant<int, EPI_SQRELU_HILO>{}); break;
    case EPI_F32: f(std::integral_constant<int, EPI_F32>{}); break;
    case EPI_F32_ADD: f(std::integral_constant<int, EPI_F32_ADD>{}); break;
    case EPI_GATE_F32: f(std::integral_constant<int, EPI_GATE_F32>{}); break;
    case EPI_GATE_BF16: f(std::integral_constant<int, EPI_GATE_BF16>{}); break;
    case EPI_BF16_HILO: f(std::integral_constant<int, EPI_BF16_HILO>{}); break;
    default: break;
  }
}

// runtime-kind form for kernels with few stores per lane
__device__ __forceinline__ void epilogue4(const GemmParams& p, int expert, int split, int row, int n,
                                          f32x4_t v) {
  epi_dispatch(p.epi, [&](auto E) { epi4<decltype(E)::value>(p, expert, split, row, n, v); });
}

}  // namespace lmoe
