// Grouped MFMA GEMM for tiles of up to 64 activation rows with weights read
// once per tile (experts that see tens of tokens; the FP4 workload).
//
// Block: four waves; wave w owns NT 16-row MFMA tiles of weight rows
// (n0 + 16*NT*w ..) against the tile's activation rows in 16-row groups (a
// tile of r rows runs ceil(r/16) groups, no more).  The activation tile (bf16
// hi + lo, 64 k per stage) is staged once per block in LDS and read by all
// four waves; each wave loads its own weight fragments straight into
// registers, two 64-wide k blocks ahead, so every weight byte crosses HBM once
// and is decoded once.
//
// Block-scaled FP4 weights ("Nemotron 3 Super", section 3.6; E2M1 elements
// and E4M3 block scales per "Nemotron 3 Ultra") are decoded in registers: the
// packed FP4 -> bf16 conversion with a unit scale gives the exact E2M1 values,
// and an fp32 multiply by the E4M3 block scale is exact as well (every such
// product is a bf16 number).  The per-matrix fp32 scale multiplies the
// accumulator in the epilogue.
//
// MFMA roles and the k layout follow the other kernels: weight tile = MFMA A
// operand (rows = output columns n), activations = B operand; inside each
// 64-wide k block lane group g holds k = 16g .. 16g+15 (one FP4 scale block)
// and MFMA step j uses 16g + 8j .. +7.
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

#include <type_traits>

#ifndef LMOE_MID_NT_FP4
#define LMOE_MID_NT_FP4 4
#endif

namespace lmoe {

constexpr int MD_ROWS = 64;                  // activation rows per tile
constexpr int MD_PARTB = MD_ROWS * 128;      // one part of one stage: 64 rows x 64 k bf16 = 8 KB
constexpr int MD_STAGEB = 2 * MD_PARTB;      // hi + lo

__device__ __forceinline__ int md_off(int part, int row, int piece) {
  return part * MD_PARTB + row * 128 + ((piece ^ (row & 7)) << 4);
}

// wait for this wave's LDS operations (its stores) before a barrier; vector
// memory loads stay in flight
__device__ __forceinline__ void md_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// one wave's activation slice of one stage: two 16-byte pieces of hi and lo
struct MdX {
  u32x4_t v[2][2];  // [chunk][part]
};

// one wave's weight fragments for one 64-wide k block
template <bool FP4, int NT>
struct MdW;
template <int NT>
struct MdW<false, NT> {
  u32x4_t v[NT][2];  // [n tile][step]
};
template <int NT>
struct MdW<true, NT> {
  u32x2_t codes[NT];   // 16 E2M1 codes per n tile
  uint32_t scale[NT];  // E4M3 byte per n tile
};

// two E2M1 codes (byte I of `codes`) times an E4M3 block scale -> two bf16
template <int I>
__device__ __forceinline__ uint32_t md_fp4x2(uint32_t codes, float s) {
  const bf16x2_t q = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, I);  // exact E2M1
  const uint32_t qb = __builtin_bit_cast(uint32_t, q);
  const float lo = __uint_as_float(qb << 16) * s;
  const float hi = __uint_as_float(qb & 0xFFFF0000u) * s;
  // the products are bf16 numbers: keep the upper halves
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// eight E2M1 codes times an E4M3 block scale (already as float) -> eight bf16
__device__ __forceinline__ u32x4_t md_fp4x8(uint32_t codes, float s) {
  u32x4_t r;
  r[0] = md_fp4x2<0>(codes, s);
  r[1] = md_fp4x2<1>(codes, s);
  r[2] = md_fp4x2<2>(codes, s);
  r[3] = md_fp4x2<3>(codes, s);
  return r;
}

// The pipelined main loop for a tile whose rows fill MT 16-row groups.
// Stage s (one 64-wide k block) is loaded into register set s % 3 two steps
// ahead: the activation part is written to LDS slot s % 2 at step s, the
// weight part is used from registers.  Every step issues the same loads (past
// the last k block it re-reads the last one), so the compiler's in-order wait
// counts are exact on every path and the loads of two later stages stay in
// flight while a stage is multiplied.
template <bool FP4, int NT, int EPI, int MT>
__device__ __forceinline__ void mid_body(const GemmParams& p, uint8_t* smem, int expert, int row0,
                                         int rows, int nbase, bool active) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int P = p.seg[0].K >> 6;  // 64-wide k blocks

  // activations: this wave moves chunks wave and wave + 4 (1 KB = 8 rows x
  // 128 B each) of both parts.  Lane l handles row 8c + l/8, logical piece l%8,
  // stored at piece (l%8) ^ (row & 7).
  uint32_t x_off[2], x_lds[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (wave + 4 * i) + (lane >> 3);
    const int xr = min(row, rows - 1);
    const int src = p.row_index ? p.row_index[row0 + xr] : row0 + xr;
    x_off[i] = ((uint32_t)src * (uint32_t)p.lda + (lane & 7) * 8) * 2u;  // bytes
    x_lds[i] = md_off(0, row, lane & 7);
  }
  const uint8_t* Xhi = reinterpret_cast<const uint8_t*>(p.seg[0].A);
  const uint8_t* Xlo = reinterpret_cast<const uint8_t*>(p.a_lo);

  // weights: uniform expert base + 32-bit per-lane offsets (row n, k = 16g ..);
  // waves past the end read a valid slab they never use (p.N is a multiple of 16 * NT)
  const int wrow0 = min(nbase, p.N - 16 * NT);
  const uint8_t* Wb;
  const uint8_t* Sb = nullptr;
  uint32_t w_off[NT], s_off[NT];
  if constexpr (FP4) {
    Wb = reinterpret_cast<const uint8_t*>(p.seg[0].B) + (size_t)expert * (size_t)(p.b_stride / 2);
    Sb = p.b_scale + (size_t)expert * (size_t)p.N * (size_t)(p.ldb / 16);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t n = wrow0 + nt * 16 + r16;
      w_off[nt] = n * (uint32_t)(p.ldb / 2) + 8u * g;
      s_off[nt] = n * (uint32_t)(p.ldb / 16) + g;
    }
  } else {
    Wb = reinterpret_cast<const uint8_t*>(p.seg[0].B) + (size_t)expert * (size_t)p.b_stride * 2;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t n = wrow0 + nt * 16 + r16;
      w_off[nt] = (n * (uint32_t)p.ldb + 16u * g) * 2u;
      s_off[nt] = 0;
    }
  }

  auto issue = [&](MdX& xv, MdW<FP4, NT>& wv, int ps) {
    const uint8_t* xh = Xhi + ps * 128;
    const uint8_t* xl = Xlo + ps * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      xv.v[i][0] = *reinterpret_cast<const u32x4_t*>(xh + x_off[i]);
      xv.v[i][1] = *reinterpret_cast<const u32x4_t*>(xl + x_off[i]);
    }
    if constexpr (FP4) {
      const uint8_t* wb = Wb + ps * 32;
      const uint8_t* sb = Sb + ps * 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        wv.codes[nt] = *reinterpret_cast<const u32x2_t*>(wb + w_off[nt]);
        wv.scale[nt] = sb[s_off[nt]];
      }
    } else {
      const uint8_t* wb = Wb + ps * 128;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        wv.v[nt][0] = *reinterpret_cast<const u32x4_t*>(wb + w_off[nt]);
        wv.v[nt][1] = *reinterpret_cast<const u32x4_t*>(wb + w_off[nt] + 16);
      }
    }
  };
  auto stash = [&](const MdX& xv, int s) {
    uint8_t* st = smem + (s & 1) * MD_STAGEB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<u32x4_t*>(st + x_lds[i]) = xv.v[i][0];
      *reinterpret_cast<u32x4_t*>(st + MD_PARTB + x_lds[i]) = xv.v[i][1];
    }
  };

  f32x4_t acc[NT][MT];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < MT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const MdW<FP4, NT>& wv, int s) {
    const uint8_t* st = smem + (s & 1) * MD_STAGEB;
    float sc[NT];
    if constexpr (FP4) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc[nt] = e4m3_to_f32(wv.scale[nt]);
    }
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      u32x4_t xf[2][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int part = 0; part < 2; ++part)
          xf[part][mt] = *reinterpret_cast<const u32x4_t*>(st + md_off(part, mt * 16 + r16, 2 * g + js));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        u32x4_t wf;
        if constexpr (FP4)
          wf = md_fp4x8(wv.codes[nt][js], sc[nt]);
        else
          wf = wv.v[nt][js];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[nt][mt] = mfma_16x16x32(wf, xf[0][mt], acc[nt][mt]);
          acc[nt][mt] = mfma_16x16x32(wf, xf[1][mt], acc[nt][mt]);
        }
      }
    }
  };

  MdX x0, x1, x2;
  MdW<FP4, NT> w0, w1, w2;
  // sched_barrier keeps each stage's loads together and in stage order, so a
  // stage's loads are never behind the next stage's in the in-order counter
  issue(x0, w0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue(x1, w1, min(1, P - 1));
  __builtin_amdgcn_sched_barrier(0);
  auto step = [&](MdX& xc, MdW<FP4, NT>& wc, MdX& xn, MdW<FP4, NT>& wn, int s) {
    stash(xc, s);  // slot s % 2 was last read at step s - 2, before the previous barrier
    md_wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
    issue(xn, wn, min(s + 2, P - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (active && s < P) compute(wc, s);
  };
  // the trip count is padded to a multiple of three (one loop exit; the
  // padding steps only move data) so the register sets stay static
  const int P3 = (P + 2) / 3 * 3;
  for (int s = 0; s < P3; s += 3) {
    step(x0, w0, x2, w2, s);
    step(x1, w1, x0, w0, s + 1);
    step(x2, w2, x1, w1, s + 2);
  }

  if (!active) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nbase + nt * 16 + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      if (m < rows) epi4<EPI>(p, expert, 0, row0 + m, n, acc[nt][mt]);
    }
  }
}

template <bool FP4, int NT, int EPI>
__global__ __launch_bounds__(256) void gemm_mid_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int BN = 4 * 16 * NT;  // weight rows per block
  const int NQ = (p.N + BN - 1) / BN;
  const int j = blockIdx.x / NQ;
  const int q = blockIdx.x % NQ;
  if (j >= p.n_tiles[0]) return;
  const int expert = p.tile_expert[j];
  const int row0 = p.tile_row0[j];
  const int rows = p.tile_rows[j];
  const int nbase = q * BN + (threadIdx.x >> 6) * 16 * NT;
  const bool active = nbase < p.N;  // wave-uniform; inactive waves still stage activations
  switch ((rows + 15) >> 4) {
    case 1: mid_body<FP4, NT, EPI, 1>(p, smem, expert, row0, rows, nbase, active); break;
    case 2: mid_body<FP4, NT, EPI, 2>(p, smem, expert, row0, rows, nbase, active); break;
    case 3: mid_body<FP4, NT, EPI, 3>(p, smem, expert, row0, rows, nbase, active); break;
    default: mid_body<FP4, NT, EPI, 4>(p, smem, expert, row0, rows, nbase, active); break;
  }
}

template <bool FP4, int NT, int EPI>
static void mid_launch(const GemmParams& p, hipStream_t s) {
  constexpr int BN = 4 * 16 * NT;
  const long long blocks = (long long)p.max_tiles * ((p.N + BN - 1) / BN);
  if (blocks <= 0) return;
  gemm_mid_kernel<FP4, NT, EPI><<<(unsigned)blocks, 256, 2 * MD_STAGEB, s>>>(p);
}

constexpr int MD_NT_FP4 = LMOE_MID_NT_FP4;
constexpr int MD_NT_BF16 = 4;

bool gemm_mid_supports(const GemmParams& p, bool fp4) {
  const int nt = fp4 ? MD_NT_FP4 : MD_NT_BF16;
  return p.tile_expert && p.rows_per_tile <= MD_ROWS && p.a_lo && p.nseg == 1 &&
         p.N % (16 * nt) == 0 && p.seg[0].K % 64 == 0 && p.seg[0].K >= 64 &&
         (p.epi == EPI_SQRELU_HILO || p.epi == EPI_GATE_F32);
}

void launch_gemm_mid(const GemmParams& p, bool fp4, hipStream_t s) {
  if (fp4) {
    if (p.epi == EPI_SQRELU_HILO) mid_launch<true, MD_NT_FP4, EPI_SQRELU_HILO>(p, s);
    else mid_launch<true, MD_NT_FP4, EPI_GATE_F32>(p, s);
  } else {
    if (p.epi == EPI_SQRELU_HILO) mid_launch<false, MD_NT_BF16, EPI_SQRELU_HILO>(p, s);
    else mid_launch<false, MD_NT_BF16, EPI_GATE_F32>(p, s);
  }
}

}  // namespace lmoe
