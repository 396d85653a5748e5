// LDS-tiled MFMA GEMM for many rows per tile (prefill-like shapes).
//
// Block tile: 128 weight rows (output columns n) x 128 activation rows, k step
// 64, four waves in a 2 x 2 arrangement, each wave 64 x 64 with 4 x 4 MFMA
// 16x16x32 tiles.  Both operand tiles are staged through LDS in two buffers
// (global loads of step k+1 are in flight while step k computes).  In grouped
// mode the activation rows are gathered through a row index (the expert
// permutation) while they are loaded.
//
// The k layout inside a 64-wide k block is the one the weight-streaming kernel
// uses: lane group g holds k = 16g .. 16g+15, MFMA step j uses 16g + 8j .. +7.
//
// DUAL: the activation tile is staged as two bf16 parts (hi + lo) and every
// weight fragment feeds both, so the product carries about 16 bits of the
// activation at twice the MFMA work and the same weight traffic.
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace lmoe {

constexpr int TL_BN = 128;  // weight rows per block
constexpr int TL_BM = 128;  // activation rows per block
constexpr int TL_BK = 64;
constexpr int TL_ROWB = TL_BK * 2;  // bytes per LDS row

__device__ __forceinline__ void seg_at_tile(const GemmParams& p, int kg, const uint16_t*& A,
                                            const uint16_t*& B, int& kl) {
  int k = kg, s = 0;
  while (s + 1 < p.nseg && k >= p.seg[s].K) {
    k -= p.seg[s].K;
    ++s;
  }
  A = reinterpret_cast<const uint16_t*>(p.seg[s].A);
  B = reinterpret_cast<const uint16_t*>(p.seg[s].B);
  kl = k;
}

template <bool DUAL>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmParams p) {
  constexpr int NPART = DUAL ? 2 : 1;
  constexpr int WBYTES = TL_BN * TL_ROWB;
  constexpr int XBYTES = TL_BM * TL_ROWB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // [buf][weights | activation part 0 | activation part 1]
  auto Wbuf = [&](int buf) { return smem + buf * (WBYTES + NPART * XBYTES); };
  auto Xbuf = [&](int buf, int part) { return Wbuf(buf) + WBYTES + part * XBYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;

  const int NQ = (p.N + TL_BN - 1) / TL_BN;
  int item = blockIdx.x;
  const int split = item % p.splits;
  item /= p.splits;
  const int q = item % NQ;
  const int j = item / NQ;
  int expert = 0, row0, rows;
  if (p.tile_expert) {
    if (j >= p.n_tiles[0]) return;
    expert = p.tile_expert[j];
    row0 = p.tile_row0[j];
    rows = p.tile_rows[j];
  } else {
    row0 = j * TL_BM;
    rows = min(TL_BM, p.M - row0);
    if (rows <= 0) return;
  }
  const int n0 = q * TL_BN;

  int Ktot = 0;
  for (int s = 0; s < p.nseg; ++s) Ktot += p.seg[s].K;
  const int kbeg = split * p.k_split;
  const int kend = min(Ktot, kbeg + p.k_split);
  if (kbeg >= kend) return;
  const int KT = (kend - kbeg) / TL_BK;

  const long long bexp = (long long)expert * p.b_stride;

  // this thread's four pieces of each operand tile: row = i / 8, piece = i % 8
  int x_src[4];
  int w_row[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + u * 256;
    const int row = i >> 3;
    x_src[u] = (row < rows) ? (p.row_index ? p.row_index[row0 + row] : row0 + row) : -1;
    w_row[u] = (n0 + row < p.N) ? n0 + row : -1;
  }
  const int pc = tid & 7;

  const uint16_t* Alo = reinterpret_cast<const uint16_t*>(p.a_lo);
  u32x4_t wr[4], xr[NPART][4];
  auto load = [&](int kt) {
    const uint16_t *A, *B;
    int kl;
    seg_at_tile(p, kbeg + kt * TL_BK, A, B, kl);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wr[u] = w_row[u] >= 0 ? ld128(B + bexp + (long long)w_row[u] * p.ldb + kl + pc * 8) : zero128();
      xr[0][u] = x_src[u] >= 0 ? ld128(A + (long long)x_src[u] * p.lda + kl + pc * 8) : zero128();
      if constexpr (DUAL)
        xr[1][u] = x_src[u] >= 0 ? ld128(Alo + (long long)x_src[u] * p.lda + kl + pc * 8) : zero128();
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (tid + u * 256) >> 3;
      const int off = row * TL_ROWB + ((pc ^ (row & 7)) << 4);
      *reinterpret_cast<u32x4_t*>(Wbuf(buf) + off) = wr[u];
#pragma unroll
      for (int part = 0; part < NPART; ++part)
        *reinterpret_cast<u32x4_t*>(Xbuf(buf, part) + off) = xr[part][u];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const int piece = 2 * g + js;
      u32x4_t wf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int rw = wn * 64 + t * 16 + r16;
        wf[t] = *reinterpret_cast<const u32x4_t*>(Wbuf(buf) + rw * TL_ROWB + ((piece ^ (rw & 7)) << 4));
      }
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        u32x4_t xf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int rx = wm * 64 + t * 16 + r16;
          xf[t] = *reinterpret_cast<const u32x4_t*>(Xbuf(buf, part) + rx * TL_ROWB + ((piece ^ (rx & 7)) << 4));
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma_16x16x32(wf[a], xf[b], acc[a][b]);
      }
    }
  };

  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load(kt + 1);
    compute(cur);
    if (kt + 1 < KT) store(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int n = n0 + wn * 64 + a * 16 + 4 * g;
    if (n >= p.N) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int m = wm * 64 + b * 16 + r16;
      if (m < rows) epilogue4(p, expert, split, row0 + m, n, acc[a][b]);
    }
  }
}

constexpr int tile_lds_bytes(bool dual) {
  return 2 * (TL_BN * TL_ROWB + (dual ? 2 : 1) * TL_BM * TL_ROWB);
}

int gemm_tile_setup() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tile_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, tile_lds_bytes(true));
  if (e != hipSuccess) return (int)e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tile_kernel<false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, tile_lds_bytes(false));
  return (int)e;
}

void launch_gemm_tile(const GemmParams& p, hipStream_t s) {
  const int NQ = (p.N + TL_BN - 1) / TL_BN;
  const long long tiles = p.tile_expert ? p.max_tiles : (p.M + TL_BM - 1) / TL_BM;
  const long long blocks = tiles * NQ * p.splits;
  if (blocks <= 0) return;
  if (p.a_lo)
    gemm_tile_kernel<true><<<(unsigned)blocks, 256, tile_lds_bytes(true), s>>>(p);
  else
    gemm_tile_kernel<false><<<(unsigned)blocks, 256, tile_lds_bytes(false), s>>>(p);
}

}  // namespace lmoe
