// Large-tile MFMA GEMM for many rows per tile (prefill-like shapes).
//
// Block tile: 256 weight rows (output columns n) x 256 activation rows, k step
// 32, eight waves in a 2 x 4 arrangement, each wave 128 x 64 = 8 x 4 MFMA
// 16x16x32 tiles (128 fp32 accumulators per lane), two waves per SIMD so that
// one wave's LDS reads and waits overlap the other's MFMAs (one wave per SIMD
// with 128 x 128 wave tiles ran 11 % slower at prefill).  Per k step a wave
// reads 12 (16 in dual mode) 16-byte fragments for 32 (64) MFMAs.
//
// Operand tiles go from global memory straight into a ring of STAGES LDS
// buffers (global_load_lds, 16 bytes per lane, no staging registers): while
// step k computes, the loads of steps k+1 .. k+STAGES-1 are in flight.  Each
// step waits for its own loads (vmcnt), then one barrier makes every wave's
// loads visible and frees the buffer the next issue overwrites.
//
// LDS rows are 64 bytes (32 bf16 of one k step); the 16-byte piece p of row r
// is stored at piece p ^ ((r >> 2) & 3), so the 16 rows a lane group reads in
// one MFMA operand land in distinct 16-byte slots.  A direct load writes lane l
// of a wave to slot l of a 1 KB chunk (16 rows), so each lane fetches the
// global piece that belongs in its slot.
//
// k layout inside a 32-wide k step: lane group g = lane / 16 holds k = 8g .. 8g+7
// for both operands.  DUAL: the activation tile comes as two bf16 parts (hi + lo)
// and every weight fragment feeds both.
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace lmoe {

constexpr int BG_BN = 256;
constexpr int BG_BM = 256;
constexpr int BG_BK = 32;
constexpr int BG_ROWB = BG_BK * 2;          // 64 bytes per LDS row
constexpr int BG_TILEB = 256 * BG_ROWB;     // 16 KB per operand tile

__device__ __forceinline__ int bg_off(int row, int piece) {
  return row * BG_ROWB + ((piece ^ ((row >> 2) & 3)) << 4);
}

template <bool DUAL>
constexpr int bg_stages() { return DUAL ? 3 : 4; }

// waves per block: 4 (2 x 2 waves of 128 x 128) or 8 (2 x 4 waves of 128 x 64, two
// waves per SIMD: one wave's LDS reads and waits overlap the other's MFMAs)
#ifndef LMOE_BIG_WAVES
#define LMOE_BIG_WAVES 8
#endif
constexpr int BG_WAVES = LMOE_BIG_WAVES;
constexpr int BG_THREADS = 64 * BG_WAVES;
constexpr int BG_WM = BG_WAVES / 2;        // waves along the activation rows
constexpr int BG_MB = BG_BM / BG_WM / 16;  // 16-row activation tiles per wave
constexpr int BG_CPW = 16 / BG_WAVES;      // 1 KB chunks per wave per operand tile

// wait until at most n of this wave's vector-memory loads are outstanding
__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at max
#define LMOE_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
  switch (n) {
    case 0: LMOE_VMCNT(0); break;
    case 4: LMOE_VMCNT(4); break;
    case 6: LMOE_VMCNT(6); break;
    case 8: LMOE_VMCNT(8); break;
    case 12: LMOE_VMCNT(12); break;
    case 16: LMOE_VMCNT(16); break;
    case 24: LMOE_VMCNT(24); break;
    default: LMOE_VMCNT(0); break;
  }
#undef LMOE_VMCNT
}

template <bool DUAL, int EPI>
__global__ __launch_bounds__(BG_THREADS, 1) void gemm_big_kernel(GemmParams p) {
  constexpr int NPART = DUAL ? 2 : 1;
  constexpr int STAGES = bg_stages<DUAL>();
  constexpr int STAGEB = BG_TILEB * (1 + NPART);  // weights + activation part(s)
  constexpr int LOADS = BG_CPW * (1 + NPART);     // direct loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;  // 128 weight rows x BG_MB * 16 activation rows
  const int r16 = lane & 15, g = lane >> 4;

  const int NQ = (p.N + BG_BN - 1) / BG_BN;
  int item = blockIdx.x;
  const int split = item % p.splits;
  item /= p.splits;
  const int q = item % NQ;
  int j = item / NQ;
  int expert = 0, row0, rows;
  if (p.tile_expert) {
    if (j >= p.n_tiles[0]) return;
    if (p.tile_first) j += p.tile_first[0];
    expert = p.tile_expert[j];
    row0 = p.tile_row0[j];
    rows = p.tile_rows[j];
  } else {
    row0 = j * BG_BM;
    rows = min(BG_BM, p.M - row0);
    if (rows <= 0) return;
  }
  const int n0 = q * BG_BN;

  int Ktot = 0;
  for (int s = 0; s < p.nseg; ++s) Ktot += p.seg[s].K;
  const int kbeg = split * p.k_split;
  const int kend = min(Ktot, kbeg + p.k_split);
  if (kbeg >= kend) return;
  const int KT = (kend - kbeg) / BG_BK;
  const long long bexp = (long long)expert * p.b_stride;

  // This wave loads 1 KB chunks c = wave + BG_WAVES i of each 16 KB operand
  // tile: lane l fills slot l of the chunk, i.e. row 16c + l/4, stored piece
  // l%4, which holds logical piece (l%4) ^ ((row >> 2) & 3).  Rows past the
  // tile are clamped to a valid row: their products land in outputs that are
  // never stored.
  uint32_t w_off[BG_CPW], x_off[BG_CPW];
#pragma unroll
  for (int i = 0; i < BG_CPW; ++i) {
    const int row = 16 * (wave + BG_WAVES * i) + (lane >> 2);
    const int piece = (lane & 3) ^ ((row >> 2) & 3);
    const int wrow = min(n0 + row, p.N - 1) - n0;
    const int xr = min(row, rows - 1);
    const int src = p.row_index ? p.row_index[row0 + xr] : row0 + xr;
    w_off[i] = (uint32_t)wrow * (uint32_t)p.ldb + piece * 8;
    x_off[i] = (uint32_t)src * (uint32_t)p.lda + piece * 8;
  }

  // segment boundaries without indexing the parameter struct at run time
  const int K0 = p.seg[0].K, K1 = p.nseg > 1 ? p.seg[1].K : 0;
  const uint16_t* A0 = reinterpret_cast<const uint16_t*>(p.seg[0].A);
  const uint16_t* A1 = reinterpret_cast<const uint16_t*>(p.seg[1].A);
  const uint16_t* A2 = reinterpret_cast<const uint16_t*>(p.seg[2].A);
  const uint16_t* B0 = reinterpret_cast<const uint16_t*>(p.seg[0].B) + bexp + (long long)n0 * p.ldb;
  const uint16_t* B1 = reinterpret_cast<const uint16_t*>(p.seg[1].B) + bexp + (long long)n0 * p.ldb;
  const uint16_t* B2 = reinterpret_cast<const uint16_t*>(p.seg[2].B) + bexp + (long long)n0 * p.ldb;
  const uint16_t* Alo = reinterpret_cast<const uint16_t*>(p.a_lo);

  auto issue = [&](int kt) {
    int k = kbeg + kt * BG_BK;
    const uint16_t* A = A0;
    const uint16_t* B = B0;
    if (k >= K0 && p.nseg > 1) {
      k -= K0;
      A = A1;
      B = B1;
      if (k >= K1 && p.nseg > 2) {
        k -= K1;
        A = A2;
        B = B2;
      }
    }
    uint8_t* st = smem + (kt % STAGES) * STAGEB;
#pragma unroll
    for (int i = 0; i < BG_CPW; ++i) {
      const int chunk = (wave + BG_WAVES * i) * 1024;
      __builtin_amdgcn_global_load_lds(B + k + w_off[i], st + chunk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(A + k + x_off[i], st + BG_TILEB + chunk, 16, 0, 0);
      if constexpr (DUAL)
        __builtin_amdgcn_global_load_lds(Alo + k + x_off[i], st + 2 * BG_TILEB + chunk, 16, 0, 0);
    }
  };

  f32x4_t acc[8][BG_MB];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < BG_MB; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt) {
    const uint8_t* base = smem + (kt % STAGES) * STAGEB;
    u32x4_t wf[8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
      wf[a] = *reinterpret_cast<const u32x4_t*>(base + bg_off(wn * 128 + a * 16 + r16, g));
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      u32x4_t xf[BG_MB];
#pragma unroll
      for (int b = 0; b < BG_MB; ++b)
        xf[b] = *reinterpret_cast<const u32x4_t*>(base + (1 + part) * BG_TILEB +
                                                  bg_off(wm * (BG_MB * 16) + b * 16 + r16, g));
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < BG_MB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xf[b], acc[a][b]);
    }
  };

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    // stages issued after step kt: min(STAGES - 2, KT - 1 - kt)
    const int later = min(STAGES - 2, KT - 1 - kt);
    wait_vmcnt(later * LOADS);
    // a plain barrier: the step's own loads were waited for above; a fenced
    // __syncthreads would wait for every load in flight, draining the ring
    asm volatile("s_barrier" ::: "memory");
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
    compute(kt);
  }

#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int n = n0 + wn * 128 + a * 16 + 4 * g;
#pragma unroll
    for (int b = 0; b < BG_MB; ++b) {
      const int m = wm * (BG_MB * 16) + b * 16 + r16;
      if (n < p.N && m < rows) epi4<EPI>(p, expert, split, row0 + m, n, acc[a][b]);
    }
  }
}

template <bool DUAL>
constexpr int big_lds_bytes() { return bg_stages<DUAL>() * BG_TILEB * (1 + (DUAL ? 2 : 1)); }

template <bool DUAL, int EPI>
static hipError_t big_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_big_kernel<DUAL, EPI>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, big_lds_bytes<DUAL>());
}

// the (dual, epilogue) instances the host launches
template <class F>
static void big_for_each_epi(int epi, F&& f) {
  switch (epi) {
    case EPI_PARTIAL: f(std::integral_constant<int, EPI_PARTIAL>{}); break;
    case EPI_BF16_HILO: f(std::integral_constant<int, EPI_BF16_HILO>{}); break;
    case EPI_SQRELU_HILO: f(std::integral_constant<int, EPI_SQRELU_HILO>{}); break;
    case EPI_SQRELU_BF16: f(std::integral_constant<int, EPI_SQRELU_BF16>{}); break;
    case EPI_F32: f(std::integral_constant<int, EPI_F32>{}); break;
    case EPI_F32_ADD: f(std::integral_constant<int, EPI_F32_ADD>{}); break;
    case EPI_GATE_F32: f(std::integral_constant<int, EPI_GATE_F32>{}); break;
    default: break;
  }
}

int gemm_big_setup() {
  const int kinds[] = {EPI_PARTIAL, EPI_BF16_HILO, EPI_SQRELU_HILO, EPI_SQRELU_BF16,
                       EPI_F32, EPI_F32_ADD, EPI_GATE_F32};
  hipError_t e = hipSuccess;
  for (int k : kinds) {
    big_for_each_epi(k, [&](auto E) {
      if (e == hipSuccess) e = big_attr<true, decltype(E)::value>();
      if (e == hipSuccess) e = big_attr<false, decltype(E)::value>();
    });
  }
  return (int)e;
}

bool gemm_big_supports(int epi) {
  return epi == EPI_PARTIAL || epi == EPI_BF16_HILO || epi == EPI_SQRELU_HILO ||
         epi == EPI_SQRELU_BF16 || epi == EPI_F32 || epi == EPI_F32_ADD || epi == EPI_GATE_F32;
}

void launch_gemm_big(const GemmParams& p, hipStream_t s) {
  const int NQ = (p.N + BG_BN - 1) / BG_BN;
  const long long tiles = p.tile_expert ? p.max_tiles : (p.M + BG_BM - 1) / BG_BM;
  const long long blocks = tiles * NQ * p.splits;
  if (blocks <= 0) return;
  if (p.a_lo)
    big_for_each_epi(p.epi, [&](auto E) {
      gemm_big_kernel<true, decltype(E)::value><<<(unsigned)blocks, BG_THREADS, big_lds_bytes<true>(), s>>>(p);
    });
  else
    big_for_each_epi(p.epi, [&](auto E) {
      gemm_big_kernel<false, decltype(E)::value><<<(unsigned)blocks, BG_THREADS, big_lds_bytes<false>(), s>>>(p);
    });
}

}  // namespace lmoe
