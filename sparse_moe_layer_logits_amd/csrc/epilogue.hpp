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

// A tile's stores take every value they need besides the accumulators as
// arguments: the weight tensor scale `ts` (one per expert), the row factor `rf`
// (the gate weight of a gated row) and `add` (the bias of EPI_F32, the old output
// of EPI_F32_ADD).  Callers load those before the stores: vmcnt counts loads and
// stores alike, so a load between two stores makes the second wait until the
// first has completed, and a tile of 32 stores per lane would run one at a time.
__device__ __forceinline__ float epi_tscale(const GemmParams& p, int expert) {
  return p.b_tscale ? p.b_tscale[expert] : 1.0f;
}

template <int EPI>
__device__ __forceinline__ float epi_rowf(const GemmParams& p, int row) {
  if constexpr (EPI == EPI_GATE_F32 || EPI == EPI_GATE_BF16) return p.row_scale ? p.row_scale[row] : 1.0f;
  else return 1.0f;
}

template <int EPI>
__device__ __forceinline__ f32x4_t epi_add(const GemmParams& p, int row, int n) {
  if constexpr (EPI == EPI_F32) {
    if (p.bias) return *reinterpret_cast<const f32x4_t*>(p.bias + n);
  } else if constexpr (EPI == EPI_F32_ADD) {
    return *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(p.C) + (long long)row * p.ldc + n);
  }
  return f32x4_t{0.f, 0.f, 0.f, 0.f};
}

template <int EPI>
constexpr bool epi_has_add() { return EPI == EPI_F32 || EPI == EPI_F32_ADD; }

// waits for every vector-memory operation of this wave.  Issued as the wait
// instruction itself, so that the compiler's wait insertion knows the loaded
// values are ready on every path: otherwise a value loaded under a branch stays
// "maybe pending" and each guarded store gets a full wait of its own.
__device__ __forceinline__ void epi_wait_all() {
  // s_waitcnt: vmcnt (bits 3:0, 15:14) = 0; expcnt (6:4) and lgkmcnt (11:8) at max
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// The values of one 4-column group before they go to memory: v0 is the output in
// fp32 (bf16 kinds round it when packing, and a hi/lo pair's low part is formed
// there from the packed high part).  EPI_F32_ADD gives the addend acc * ts; the
// store adds the old value.
struct Epi4 {
  f32x4_t v0;
};

template <int EPI>
__device__ __forceinline__ Epi4 epi_math(const GemmParams& p, f32x4_t v, float ts, float rf, f32x4_t add) {
  Epi4 o;
  if constexpr (EPI == EPI_PARTIAL || EPI == EPI_BF16) {
    o.v0 = v;
  } else if constexpr (EPI == EPI_SQRELU_BF16 || EPI == EPI_SQRELU_HILO || EPI == EPI_BF16_HILO) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float u = v[i] * ts;
      if constexpr (EPI != EPI_BF16_HILO) {
        u = fmaxf(u, 0.0f);
        u = u * u;
      }
      o.v0[i] = u;
    }
  } else if constexpr (EPI == EPI_F32) {
    o.v0 = v * ts;
    if (p.bias) o.v0 += add;
  } else if constexpr (EPI == EPI_F32_ADD) {
    o.v0 = v * ts;
  } else if constexpr (EPI == EPI_GATE_F32 || EPI == EPI_GATE_BF16) {
    o.v0 = v * (rf * ts);
  }
  return o;
}

// output arrays (hi and lo for the pair kinds) and bytes per element
template <int EPI>
constexpr int epi_planes() { return EPI == EPI_SQRELU_HILO || EPI == EPI_BF16_HILO ? 2 : 1; }

// bf16 planes of a 4-column group: hi = bf16(u) (round to nearest even) and, for
// the pair kinds, lo = bf16(u - hi) (u - hi is exact in fp32)
template <int EPI>
__device__ __forceinline__ void epi_pack(const f32x4_t& u, u32x2_t& hi, u32x2_t& lo) {
  hi = u32x2_t{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3])};
  if constexpr (epi_planes<EPI>() == 2) {
    const f32x4_t h = {__uint_as_float(hi.x << 16), __uint_as_float(hi.x & 0xFFFF0000u),
                       __uint_as_float(hi.y << 16), __uint_as_float(hi.y & 0xFFFF0000u)};
    const f32x4_t l = u - h;
    lo = u32x2_t{pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3])};
  }
}
template <int EPI>
constexpr int epi_bytes() {
  return EPI == EPI_PARTIAL || EPI == EPI_F32 || EPI == EPI_F32_ADD || EPI == EPI_GATE_F32 ? 4 : 2;
}

template <int EPI>
__device__ __forceinline__ void epi4(const GemmParams& p, int split, int row, int n, f32x4_t v, float ts,
                                     float rf, f32x4_t add) {
  const long long off = (long long)row * p.ldc + n;
  const Epi4 o = epi_math<EPI>(p, v, ts, rf, add);
  if constexpr (EPI == EPI_PARTIAL) {
    float* dst = p.partial + (long long)split * p.partial_stride + (long long)row * p.N + n;
    *reinterpret_cast<f32x4_t*>(dst) = o.v0;
  } else if constexpr (epi_bytes<EPI>() == 2) {
    u32x2_t hi, lo;
    epi_pack<EPI>(o.v0, hi, lo);
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(p.C) + off) = hi;
    if constexpr (epi_planes<EPI>() == 2) *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(p.C2) + off) = lo;
  } else if constexpr (EPI == EPI_F32_ADD) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off) = add + o.v0;
  } else {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + off) = o.v0;
  }
}

// Stores a lane's NA x NB accumulator fragments: fragment (a, b) is output
// column ncol(a) .. + 3 of tile row mrow(b) (global row row0 + mrow(b)); it is
// stored when ncol(a) < p.N, mrow(b) < rows and b < nb.  Loads come first: the
// tile's scale and row factors once, the addends of one column group at a time.
template <int EPI, int NA, int NB, class NC, class MR>
__device__ __forceinline__ void epi_tile(const GemmParams& p, int expert, int split, int row0, int rows,
                                         int nb, NC ncol, MR mrow, const f32x4_t (&acc)[NA][NB]) {
  const float ts = epi_tscale(p, expert);
  float rf[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) rf[b] = (b < nb && mrow(b) < rows) ? epi_rowf<EPI>(p, row0 + mrow(b)) : 1.0f;
  epi_wait_all();
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int n = ncol(a);
    if (n >= p.N) continue;
    f32x4_t add[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      add[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (epi_has_add<EPI>())
        if (b < nb && mrow(b) < rows) add[b] = epi_add<EPI>(p, row0 + mrow(b), n);
    }
    if constexpr (epi_has_add<EPI>()) epi_wait_all();
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < nb && mrow(b) < rows) epi4<EPI>(p, split, row0 + mrow(b), n, acc[a][b], ts, rf[b], add[b]);
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

// runtime-kind form of one store (loads, then the store)
__device__ __forceinline__ void epilogue4(const GemmParams& p, int expert, int split, int row, int n,
                                          f32x4_t v) {
  epi_dispatch(p.epi, [&](auto E) {
    constexpr int EPI = decltype(E)::value;
    epi4<EPI>(p, split, row, n, v, epi_tscale(p, expert), epi_rowf<EPI>(p, row), epi_add<EPI>(p, row, n));
  });
}

}  // namespace lmoe
