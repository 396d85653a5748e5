// GEMM epilogues: four consecutive output columns (n .. n+3) of one output row.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {

__device__ __forceinline__ void store_bf16x4(void* C, long long off, float a, float b, float c, float d) {
  u32x2_t w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(C) + off) = w;
}

__device__ __forceinline__ void epilogue4(const GemmParams& p, int expert, int split, int row, int n,
                                          f32x4_t v) {
  const long long off = (long long)row * p.ldc + n;
  switch (p.epi) {
    case EPI_PARTIAL: {
      float* dst = p.partial + (long long)split * p.partial_stride + (long long)row * p.N + n;
      *reinterpret_cast<f32x4_t*>(dst) = v;
      break;
    }
    case EPI_BF16:
      store_bf16x4(p.C, off, v[0], v[1], v[2], v[3]);
      break;
    case EPI_SQRELU_BF16: {
      const float ts = p.b_tscale ? p.b_tscale[expert] : 1.0f;
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float u = fmaxf(v[i] * ts, 0.0f);
        r[i] = u * u;
      }
      store_bf16x4(p.C, off, r[0], r[1], r[2], r[3]);
      break;
    }
    case EPI_SQRELU_HILO: {
      const float ts = p.b_tscale ? p.b_tscale[expert] : 1.0f;
      float hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float u = fmaxf(v[i] * ts, 0.0f);
        float s = u * u;
        hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(s));
        lo[i] = s - hi[i];
      }
      store_bf16x4(p.C, off, hi[0], hi[1], hi[2], hi[3]);
      store_bf16x4(p.C2, off, lo[0], lo[1], lo[2], lo[3]);
      break;
    }
    case EPI_BF16_HILO: {
      float hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(v[i]));
        lo[i] = v[i] - hi[i];
      }
      store_bf16x4(p.C, off, hi[0], hi[1], hi[2], hi[3]);
      store_bf16x4(p.C2, off, lo[0], lo[1], lo[2], lo[3]);
      break;
    }
    case EPI_F32: {
      f32x4_t w = v;
      if (p.bias) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] += p.bias[n + i];
      }
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off) = w;
      break;
    }
    case EPI_F32_ADD: {
      f32x4_t* dst = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off);
      f32x4_t w = *dst;
      *dst = w + v;
      break;
    }
    case EPI_GATE_F32:
    case EPI_GATE_BF16: {
      const float ts = p.b_tscale ? p.b_tscale[expert] : 1.0f;
      const float g = (p.row_scale ? p.row_scale[row] : 1.0f) * ts;
      if (p.epi == EPI_GATE_F32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off) = v * g;
      } else {
        store_bf16x4(p.C, off, v[0] * g, v[1] * g, v[2] * g, v[3] * g);
      }
      break;
    }
    default:
      break;
  }
}

}  // namespace lmoe
