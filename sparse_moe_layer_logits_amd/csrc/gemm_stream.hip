// Weight-streaming MFMA GEMM for tiles of at most ROWS activation rows.
//
// In decode-like shapes every expert sees a few tokens, so the cost is reading
// the weights once from HBM (low-latency MoE inference is bound by expert
// weight reads: "Nemotron 3 Super", section 2 and section 3.2 principle 1).
// Each wave streams 16*NT weight rows straight from HBM into registers
// (double-buffered chunks) and multiplies them with the tile's activation rows,
// which the block stages once per chunk in LDS.
//
// The weight tile is the MFMA "A" operand (rows = output columns n) and the
// activations are the MFMA "B" operand (columns = token rows), so each lane
// ends with four consecutive n of one row and stores them as one vector.
//
// k layout inside every 64-wide k block: lane group g = lane / 16 holds
// k = 16g .. 16g+15; MFMA step j (0, 1) uses k = 16g + 8j .. 16g + 8j + 7.  The
// same map is used for both operands, so the products pair up correctly, and a
// block-scaled FP4 lane group covers exactly one 16-element scale block.
//
// DUAL: the activation comes as two bf16 parts (hi + lo); each weight
// fragment feeds two MFMAs, so the weights are still read once.
//
// FMT: the stored weight format (bf16, block-scaled FP4, per-tensor FP8); FP4
// and FP8 weights are decoded to exact bf16 in registers after the load.
#include "common.hpp"
#include "epilogue.hpp"
#include "fp4.hpp"
#include "fp8.hpp"
#include "kernels.hpp"

namespace lmoe {

struct SegPtr {
  const uint16_t* A;
  const uint8_t* B;  // bytes
  int kl;            // k inside the segment
};

__device__ __forceinline__ SegPtr seg_at(const GemmParams& p, int kg) {
  int k = kg;
  int s = 0;
  while (s + 1 < p.nseg && k >= p.seg[s].K) {
    k -= p.seg[s].K;
    ++s;
  }
  SegPtr r;
  r.A = reinterpret_cast<const uint16_t*>(p.seg[s].A);
  r.B = reinterpret_cast<const uint8_t*>(p.seg[s].B);
  r.kl = k;
  return r;
}

template <int FMT>
struct BFrag;
template <>
struct BFrag<WF_BF16> {
  u32x4_t v[2];  // steps 0 and 1
};
template <>
struct BFrag<WF_FP4> {
  u32x2_t codes;   // 16 E2M1 codes
  uint32_t scale;  // E4M3 byte
};
template <>
struct BFrag<WF_FP8> {
  u32x4_t codes;   // 16 E4M3 bytes: step 0 in words 0-1, step 1 in words 2-3
};

template <int W, int NT, int ROWS, int PAIRS, int FMT, bool DUAL>
__global__ __launch_bounds__(W * 64) void gemm_stream_kernel(GemmParams p) {
  constexpr int MTMAX = ROWS / 16;
  constexpr int NPART = DUAL ? 2 : 1;
  constexpr int KC = 64 * PAIRS;                           // k per chunk
  constexpr int ROWB = KC * 2;                             // LDS bytes per row and part
  constexpr int PIECES = ROWS * 8 * PAIRS * NPART;         // 16-byte A pieces per chunk
  constexpr int THREADS = W * 64;
  constexpr int APT = (PIECES + THREADS - 1) / THREADS;    // A pieces per thread
  constexpr int PPR = 8 * PAIRS;                           // pieces per row and part
  __shared__ __attribute__((aligned(16))) uint8_t As[2][NPART * ROWS * ROWB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  // ---- work item ----
  const int NQ = (p.N + W * NT * 16 - 1) / (W * NT * 16);
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
    row0 = j * ROWS;
    rows = min(ROWS, p.M - row0);
    if (rows <= 0) return;
  }
  const int MT = (rows + 15) >> 4;

  int Ktot = 0;
  for (int s = 0; s < p.nseg; ++s) Ktot += p.seg[s].K;
  const int kbeg = split * p.k_split;
  const int kend = min(Ktot, kbeg + p.k_split);
  if (kbeg >= kend) return;
  const int npairs = (kend - kbeg) >> 6;
  const int nchunks = (npairs + PAIRS - 1) / PAIRS;

  // ---- this thread's A pieces: (part, row, piece) fixed across chunks ----
  int a_row[APT];
  int a_piece[APT];  // part * ROWS * PPR + row * PPR + piece, or -1
#pragma unroll
  for (int u = 0; u < APT; ++u) {
    const int i = threadIdx.x + u * THREADS;
    const int row = (i % (ROWS * PPR)) / PPR;
    int src = -1;
    if (i < PIECES && row < rows) src = p.row_index ? p.row_index[row0 + row] : row0 + row;
    a_row[u] = src;
    a_piece[u] = i < PIECES ? i : -1;
  }

  // ---- this wave's weight rows ----
  const int nbase = q * (W * NT * 16) + wave * (NT * 16);
  const bool wave_active = nbase < p.N;
  const long long bexp = (long long)expert * p.b_stride;  // elements
  const long long sexp = (long long)expert * p.N * (p.ldb / 16);

  f32x4_t acc[NT][MTMAX];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load_b = [&](BFrag<FMT> (&bf)[PAIRS][NT], int c) {
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int pg = c * PAIRS + pr;
      if (pg < npairs && wave_active) {
        const SegPtr sp = seg_at(p, kbeg + pg * 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = nbase + nt * 16 + r16;
          const long long kk = sp.kl + 16 * g;
          if constexpr (FMT == WF_FP4) {
            const uint8_t* bp = sp.B + (bexp + (long long)n * p.ldb + kk) / 2;
            bf[pr][nt].codes = *reinterpret_cast<const u32x2_t*>(bp);
            bf[pr][nt].scale = p.b_scale[sexp + (long long)n * (p.ldb / 16) + kk / 16];
          } else if constexpr (FMT == WF_FP8) {
            bf[pr][nt].codes = ld128(sp.B + bexp + (long long)n * p.ldb + kk);
          } else {
            const uint8_t* bp = sp.B + 2 * (bexp + (long long)n * p.ldb + kk);
            bf[pr][nt].v[0] = ld128(bp);
            bf[pr][nt].v[1] = ld128(bp + 16);
          }
        }
      }
    }
  };

  u32x4_t a_regs[APT];
  auto load_a = [&](int c) {
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      a_regs[u] = zero128();
      if (a_piece[u] < 0 || a_row[u] < 0) continue;
      const int part = a_piece[u] / (ROWS * PPR);
      const int pc = a_piece[u] % PPR;
      const int pg = c * PAIRS + (pc >> 3);
      if (pg < npairs) {
        const SegPtr sp = seg_at(p, kbeg + pg * 64);
        const uint16_t* base = (DUAL && part) ? reinterpret_cast<const uint16_t*>(p.a_lo) : sp.A;
        a_regs[u] = ld128(base + (long long)a_row[u] * p.lda + sp.kl + (pc & 7) * 8);
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      if (a_piece[u] < 0) continue;
      const int part = a_piece[u] / (ROWS * PPR);
      const int row = (a_piece[u] % (ROWS * PPR)) / PPR;
      const int pc = a_piece[u] % PPR;
      const int phys = pc ^ (row & 15);
      *reinterpret_cast<u32x4_t*>(&As[buf][(part * ROWS + row) * ROWB + phys * 16]) = a_regs[u];
    }
  };
  auto compute = [&](const BFrag<FMT> (&bf)[PAIRS][NT], int buf, int c) {
    if (!wave_active) return;
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int pg = c * PAIRS + pr;
      if (pg < npairs) {
#pragma unroll
        for (int js = 0; js < 2; ++js) {
          u32x4_t bw[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if constexpr (FMT == WF_FP4) {
              const float sc = e4m3_to_f32(bf[pr][nt].scale);
              bw[nt] = fp4x8_to_bf16(bf[pr][nt].codes[js], sc);
            } else if constexpr (FMT == WF_FP8) {
              bw[nt] = fp8x8_to_bf16(bf[pr][nt].codes[2 * js], bf[pr][nt].codes[2 * js + 1]);
            } else {
              bw[nt] = bf[pr][nt].v[js];
            }
          }
#pragma unroll
          for (int mt = 0; mt < MTMAX; ++mt) {
            if (mt < MT) {
              const int row = mt * 16 + r16;
              const int phys = (pr * 8 + 2 * g + js) ^ (row & 15);
#pragma unroll
              for (int part = 0; part < NPART; ++part) {
                const u32x4_t av = *reinterpret_cast<const u32x4_t*>(
                    &As[buf][(part * ROWS + row) * ROWB + phys * 16]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mfma_16x16x32(bw[nt], av, acc[nt][mt]);
              }
            }
          }
        }
      }
    }
  };

  BFrag<FMT> b0[PAIRS][NT], b1[PAIRS][NT];
  load_a(0);
  load_b(b0, 0);
  store_a(0);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    const bool has1 = c + 1 < nchunks;
    if (has1) {
      load_a(c + 1);
      load_b(b1, c + 1);
    }
    compute(b0, 0, c);
    if (has1) store_a(1);
    __syncthreads();
    if (!has1) break;
    const bool has2 = c + 2 < nchunks;
    if (has2) {
      load_a(c + 2);
      load_b(b0, c + 2);
    }
    compute(b1, 1, c + 1);
    if (has2) store_a(0);
    __syncthreads();
  }

  if (!wave_active) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nbase + nt * 16 + 4 * g;
    if (n >= p.N) continue;
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt) {
      const int m = mt * 16 + r16;
      if (mt < MT && m < rows) epilogue4(p, expert, split, row0 + m, n, acc[nt][mt]);
    }
  }
}

#ifndef LMOE_ST_W
#define LMOE_ST_W 8
#endif
#ifndef LMOE_ST_PAIRS16
#define LMOE_ST_PAIRS16 4
#endif

template <int ROWS, int PAIRS, int FMT, bool DUAL>
static void launch_rows(const GemmParams& p, long long blocks, hipStream_t s) {
  constexpr int W = LMOE_ST_W, NT = 1;
  gemm_stream_kernel<W, NT, ROWS, PAIRS, FMT, DUAL><<<(unsigned)blocks, W * 64, 0, s>>>(p);
}

template <int FMT, bool DUAL>
static void launch_fmt(const GemmParams& p, int rows, long long blocks, hipStream_t s) {
  if constexpr (FMT == WF_FP8) {
    // FP8 weights are the dense projections only: 64-row tiles
    launch_rows<64, DUAL ? 2 : 4, FMT, DUAL>(p, blocks, s);
  } else {
    if (rows == 16)
      launch_rows<16, LMOE_ST_PAIRS16, FMT, DUAL>(p, blocks, s);
    else if (rows == 32)
      launch_rows<32, DUAL ? 2 : 4, FMT, DUAL>(p, blocks, s);
    else
      launch_rows<64, DUAL ? 2 : 4, FMT, DUAL>(p, blocks, s);
  }
}

template <int FMT>
static void launch_dual(const GemmParams& p, int rows, long long blocks, hipStream_t s) {
  if (p.a_lo != nullptr)
    launch_fmt<FMT, true>(p, rows, blocks, s);
  else
    launch_fmt<FMT, false>(p, rows, blocks, s);
}

void launch_gemm_stream(const GemmParams& p, int fmt, hipStream_t s) {
  constexpr int W = LMOE_ST_W, NT = 1;
  // tile height: the grouped tile list's (16, 32 or 64 rows), 64 for dense GEMMs
  const int rows = !p.tile_expert ? 64 : p.rows_per_tile <= 16 ? 16 : p.rows_per_tile <= 32 ? 32 : 64;
  if (fmt == WF_FP8 && rows != 64) return;  // not offered (callers check gemm_stream_supports)
  const int NQ = (p.N + W * NT * 16 - 1) / (W * NT * 16);
  const long long tiles = p.tile_expert ? p.max_tiles : (p.M + rows - 1) / rows;
  const long long blocks = tiles * NQ * p.splits;
  if (blocks <= 0) return;
  if (fmt == WF_FP4)
    launch_dual<WF_FP4>(p, rows, blocks, s);
  else if (fmt == WF_FP8)
    launch_dual<WF_FP8>(p, rows, blocks, s);
  else
    launch_dual<WF_BF16>(p, rows, blocks, s);
}

}  // namespace lmoe
