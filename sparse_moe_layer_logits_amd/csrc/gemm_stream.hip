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
// k layout inside every 64-wide k block (bf16, FP8): lane group g = lane / 16
// holds k = 16g .. 16g+15; MFMA step j (0, 1) uses k = 16g + 8j .. 16g + 8j + 7.
// FP4: lane group g holds the contiguous k range [16 PAIRS g, 16 PAIRS (g+1)) of
// the chunk, so one lane reads its codes as 16-byte loads and all its block
// scales (one per 16 k) as one 2- or 4-byte load; the 4-bit weights would
// otherwise cost several times more memory requests per byte than bf16.
// Both operands use the same map, so the products pair up correctly.
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

// global-memory (address space 1) pointers: the segment pointers are picked with
// register selects, after which the compiler can no longer infer the address
// space of a generic pointer and would issue flat loads (counted against the LDS
// counter too, so every barrier would wait for the weight prefetches)
typedef const __attribute__((address_space(1))) uint8_t* gptr8;
typedef const __attribute__((address_space(1))) uint16_t* gptr16;
typedef const __attribute__((address_space(1))) u32x4_t* gptr128;

__device__ __forceinline__ u32x4_t gld128(gptr8 q) { return *reinterpret_cast<gptr128>(q); }
__device__ __forceinline__ u32x4_t gld128(gptr16 q) { return *reinterpret_cast<gptr128>(q); }

struct SegPtr {
  gptr16 A;
  gptr8 B;  // bytes
  int kl;   // k inside the segment
};

// a kernel-argument pointer as a plain (uniform) value: selecting between such
// values stays a register select, where a select between two argument loads may be
// turned into one per-lane load from a selected address
__device__ __forceinline__ uint64_t uniform_u64(const void* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// the segment holding global k index kg (at most three segments), branch-free: a
// lane-dependent index into p.seg would make the compiler fetch the descriptor per
// lane from memory and wait for every load in flight before using it
__device__ __forceinline__ SegPtr seg_at(const GemmParams& p, int kg) {
  const int k1 = p.seg[0].K, k2 = p.seg[0].K + p.seg[1].K;
  const bool s1 = p.nseg > 1 && kg >= k1;
  const bool s2 = p.nseg > 2 && kg >= k2;
  const uint64_t a0 = uniform_u64(p.seg[0].A), a1 = uniform_u64(p.seg[1].A),
                 a2 = uniform_u64(p.seg[2].A);
  const uint64_t b0 = uniform_u64(p.seg[0].B), b1 = uniform_u64(p.seg[1].B),
                 b2 = uniform_u64(p.seg[2].B);
  SegPtr r;
  r.A = (gptr16)(s2 ? a2 : s1 ? a1 : a0);
  r.B = (gptr8)(s2 ? b2 : s1 ? b1 : b0);
  r.kl = kg - (s2 ? k2 : s1 ? k1 : 0);
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
  uint32_t scale;  // the lane's E4M3 block scales, one byte per 16 k (byte pr for sub-block pr)
};
template <>
struct BFrag<WF_FP8> {
  u32x4_t codes;   // 16 E4M3 bytes: step 0 in words 0-1, step 1 in words 2-3
};

// LDS bytes of one block: two chunk buffers of the tile's activation rows
template <int ROWS, int PAIRS, bool DUAL>
constexpr int stream_lds_bytes() {
  return 2 * (DUAL ? 2 : 1) * ROWS * (64 * PAIRS * 2);
}

// One block's work item `block` of GEMM p; smem holds stream_lds_bytes() bytes.
template <int W, int NT, int ROWS, int PAIRS, int FMT, bool DUAL>
__device__ __forceinline__ void stream_tile(const GemmParams& p, const int block, uint8_t* smem) {
  constexpr int MTMAX = ROWS / 16;
  constexpr int NPART = DUAL ? 2 : 1;
  constexpr int KC = 64 * PAIRS;                           // k per chunk
  constexpr int ROWB = KC * 2;                             // LDS bytes per row and part
  constexpr int PIECES = ROWS * 8 * PAIRS * NPART;         // 16-byte A pieces per chunk
  constexpr int THREADS = W * 64;
  constexpr int APT = (PIECES + THREADS - 1) / THREADS;    // A pieces per thread
  constexpr int PPR = 8 * PAIRS;                           // pieces per row and part
  auto As = reinterpret_cast<uint8_t (*)[NPART * ROWS * ROWB]>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  // ---- work item ----
  const int NQ = (p.N + W * NT * 16 - 1) / (W * NT * 16);
  int item = block;
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

  static_assert(FMT != WF_FP4 || PAIRS == 2 || PAIRS == 4, "FP4 lane ranges need 2 or 4 pairs");
  // FP4: does this lane group's k range of chunk c hold weights (within the chunk's pairs)?
  auto fp4_live = [&](int c) { return g * PAIRS < 4 * min(PAIRS, npairs - c * PAIRS); };
  // FP4 GEMMs have one segment: the lane's weight-code and block-scale rows are set
  // once (rows past N clamped to N - 1) and every chunk only adds its k offset
  gptr8 w4_row[NT], s4_row[NT];
  if constexpr (FMT == WF_FP4) {
    const gptr8 B0 = (gptr8)uniform_u64(p.seg[0].B);
    const gptr8 S0 = (gptr8)uniform_u64(p.b_scale);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = min(nbase + nt * 16 + r16, p.N - 1);
      w4_row[nt] = B0 + (bexp + (long long)n * p.ldb) / 2;
      s4_row[nt] = S0 + sexp + (long long)n * (p.ldb / 16);
    }
  }
  auto load_b = [&](BFrag<FMT> (&bf)[PAIRS][NT], int c) {
    if constexpr (FMT == WF_FP4) {
      // lane group g: sub-block pr of its range is k0 + 16 pr .. k0 + 16 pr + 15.  Every
      // lane loads, so each chunk costs the same loads and the compiler's wait counts
      // stay exact: a lane without data (a wave past N, or a group past the pairs of a
      // short last chunk; PAIRS <= 4 makes groups wholly in or out) reads a valid
      // address instead, and compute() zeroes its scales.
      const int k0 = kbeg + c * PAIRS * 64 + (fp4_live(c) ? 16 * PAIRS * g : 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        u32x4_t cw[PAIRS / 2];
        uint32_t sw;
        const gptr8 bp = w4_row[nt] + k0 / 2;
#pragma unroll
        for (int i = 0; i < PAIRS / 2; ++i) cw[i] = gld128(bp + 16 * i);
        const gptr8 sb = s4_row[nt] + k0 / 16;
        if constexpr (PAIRS == 4)
          sw = *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(sb);
        else
          sw = *reinterpret_cast<const __attribute__((address_space(1))) uint16_t*>(sb);
#pragma unroll
        for (int pr = 0; pr < PAIRS; ++pr) {
          bf[pr][nt].codes = u32x2_t{cw[pr / 2][2 * (pr % 2)], cw[pr / 2][2 * (pr % 2) + 1]};
          bf[pr][nt].scale = sw;  // all PAIRS scale bytes; compute() decodes them from bf[0]
        }
      }
    } else {
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        const int pg = c * PAIRS + pr;
        if (pg < npairs && wave_active) {
          const SegPtr sp = seg_at(p, kbeg + pg * 64);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int n = nbase + nt * 16 + r16;
            const long long kk = sp.kl + 16 * g;
            if constexpr (FMT == WF_FP8) {
              bf[pr][nt].codes = gld128(sp.B + bexp + (long long)n * p.ldb + kk);
            } else {
              const gptr8 bp = sp.B + 2 * (bexp + (long long)n * p.ldb + kk);
              bf[pr][nt].v[0] = gld128(bp);
              bf[pr][nt].v[1] = gld128(bp + 16);
            }
          }
        }
      }
    }
  };

  u32x4_t a_regs[APT];
  const gptr16 a_lo = (gptr16)uniform_u64(p.a_lo);
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
        const gptr16 base = (DUAL && part) ? a_lo : sp.A;
        a_regs[u] = gld128(base + (long long)a_row[u] * p.lda + sp.kl + (pc & 7) * 8);
      }
    }
  };
  // FP4 path: every lane issues its loads (uniform load counts, as for the weights);
  // pieces without data read the tile's first row / the chunk's first pair instead and
  // store_a_sel writes zeros for them.  One segment: each piece's row pointer (with its
  // 8-element offset in the pair) and LDS address are set once.
  gptr16 a4_ptr[APT];
  int a4_pair[APT], a4_lds[APT];
  if constexpr (FMT == WF_FP4) {
    const int a_src0 = p.row_index ? p.row_index[row0] : row0;
    const gptr16 A0 = (gptr16)uniform_u64(p.seg[0].A);
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      const int piece = a_piece[u] < 0 ? 0 : a_piece[u];
      const int part = piece / (ROWS * PPR);
      const int row = (piece % (ROWS * PPR)) / PPR;
      const int pc = piece % PPR;
      const int src = a_row[u] < 0 ? a_src0 : a_row[u];
      a4_ptr[u] = ((DUAL && part) ? a_lo : A0) + (long long)src * p.lda + (pc & 7) * 8;
      a4_pair[u] = pc >> 3;
      a4_lds[u] = (part * ROWS + row) * ROWB + (pc ^ (row & 15)) * 16;
    }
  }
  auto load_a_all = [&](u32x4_t (&ar)[APT], int c) {
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      const int pg = c * PAIRS + a4_pair[u];
      ar[u] = gld128(a4_ptr[u] + kbeg + (pg < npairs ? pg : c * PAIRS) * 64);
    }
  };
  auto store_a_sel = [&](const u32x4_t (&ar)[APT], int buf, int c) {
#pragma unroll
    for (int u = 0; u < APT; ++u) {
      if (a_piece[u] < 0) continue;
      const bool ok = a_row[u] >= 0 && c * PAIRS + a4_pair[u] < npairs;
      *reinterpret_cast<u32x4_t*>(&As[buf][a4_lds[u]]) = ok ? ar[u] : zero128();
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
  // MFMAs of one 8-k step: bw holds the weights, `piece` the step's 16-byte column
  // of the activation rows in LDS (k = 8 piece .. 8 piece + 7 of the chunk)
  auto mfma_step = [&](const u32x4_t (&bw)[NT], int piece, int buf) {
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt) {
      if (mt < MT) {
        const int row = mt * 16 + r16;
        const int phys = piece ^ (row & 15);
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(
              &As[buf][(part * ROWS + row) * ROWB + phys * 16]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mfma_16x16x32(bw[nt], av, acc[nt][mt]);
        }
      }
    }
  };
  auto compute = [&](const BFrag<FMT> (&bf)[PAIRS][NT], int buf, int c) {
    if (!wave_active) return;
    if constexpr (FMT == WF_FP4) {
      // every step carries data from the live lane groups: no per-pair skip; the other
      // groups hold re-read weights, zeroed through their scales
      const bool live = fp4_live(c);
      // the lane's PAIRS block scales (bytes of one word, the same in every bf[pr])
      float scl[NT][PAIRS];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int h = 0; h < PAIRS / 2; ++h) {
          const f32x2_t v = h ? fp8x2_to_f32<true>(bf[0][nt].scale) : fp8x2_to_f32<false>(bf[0][nt].scale);
          scl[nt][2 * h] = live ? v.x : 0.0f;
          scl[nt][2 * h + 1] = live ? v.y : 0.0f;
        }
      }
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        float sc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sc[nt] = scl[nt][pr];
#pragma unroll
        for (int js = 0; js < 2; ++js) {
          u32x4_t bw[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) bw[nt] = fp4x8_to_bf16(bf[pr][nt].codes[js], sc[nt]);
          mfma_step(bw, 2 * PAIRS * g + 2 * pr + js, buf);
        }
      }
    } else {
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        const int pg = c * PAIRS + pr;
        if (pg < npairs) {
#pragma unroll
          for (int js = 0; js < 2; ++js) {
            u32x4_t bw[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              if constexpr (FMT == WF_FP8)
                bw[nt] = fp8x8_to_bf16(bf[pr][nt].codes[2 * js], bf[pr][nt].codes[2 * js + 1]);
              else
                bw[nt] = bf[pr][nt].v[js];
            }
            mfma_step(bw, pr * 8 + 2 * g + js, buf);
          }
        }
      }
    }
  };

  if constexpr (FMT == WF_FP4) {
    // FP4 fragments are small (3 registers per pair): rings of R chunks of weights and
    // activation pieces (registers) keep R - 1 chunks of loads in flight while a chunk
    // is computed.  Step cc loads chunk cc + R - 1 (activations first, then weights) and
    // moves chunk cc + 1's activations to LDS; loads complete in order, so that wait
    // leaves the younger chunks in flight.  Every step issues the same loads (clamped
    // to the last chunk past the end) and the loop has one exit, so the compiler's
    // wait counts stay exact.
    constexpr int R = 2;
    BFrag<FMT> ring[R][PAIRS][NT];
    u32x4_t aring[R][APT];
    const int last = nchunks - 1;
#pragma unroll
    for (int i = 0; i < R - 1; ++i) {
      load_a_all(aring[i], min(i, last));
      load_b(ring[i], min(i, last));
    }
    store_a_sel(aring[0], 0, 0);
    __syncthreads();
    for (int c = 0; c < nchunks; c += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int cc = c + u;
        load_a_all(aring[(u + R - 1) % R], min(cc + R - 1, last));
        load_b(ring[(u + R - 1) % R], min(cc + R - 1, last));
        if (cc < nchunks) compute(ring[u], u & 1, cc);
        store_a_sel(aring[(u + 1) % R], (u + 1) & 1, min(cc + 1, last));
        __syncthreads();
      }
    }
  } else {
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
  }

  if (!wave_active) return;
  epi_dispatch(p.epi, [&](auto E) {
    epi_tile<decltype(E)::value>(p, expert, split, row0, rows, MTMAX,
                                 [&](int nt) { return nbase + nt * 16 + 4 * g; },
                                 [&](int mt) { return mt * 16 + r16; }, acc);
  });
}

template <int W, int NT, int ROWS, int PAIRS, int FMT, bool DUAL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(1))) void gemm_stream_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[stream_lds_bytes<ROWS, PAIRS, DUAL>()];
  stream_tile<W, NT, ROWS, PAIRS, FMT, DUAL>(p, blockIdx.x, smem);
}

// Two GEMMs in one launch: blocks [0, q_blocks) run q, a dense GEMM of at most 64
// rows over its whole k range (bf16 weights, 128-k chunks; QDUAL: hi + lo
// activations), the rest run the grouped expert GEMM p.  A dense GEMM of a few
// tokens on its own is a short launch whose blocks wait on memory latency
// (a few chunks each, then split-K partial sums); inside a long weight-streaming
// launch its blocks start first, read their weights at the launch's rate and
// finish long before it ends.
template <int W, int NT, int ROWS, int PAIRS, int FMT, bool DUAL, bool QDUAL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(1))) void gemm_stream_pair_kernel(
    GemmParams p, GemmParams q, int q_blocks) {
  constexpr int LP = stream_lds_bytes<ROWS, PAIRS, DUAL>();
  constexpr int LQ = stream_lds_bytes<64, 2, QDUAL>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[LP > LQ ? LP : LQ];
  const int b = blockIdx.x;
  if (b < q_blocks)
    stream_tile<W, NT, 64, 2, WF_BF16, QDUAL>(q, b, smem);
  else
    stream_tile<W, NT, ROWS, PAIRS, FMT, DUAL>(p, b - q_blocks, smem);
}

// block shape: 8 waves of one 16-row weight tile each
constexpr int ST_W = 8, ST_NT = 1;

template <int ROWS, int PAIRS, int FMT, bool DUAL>
static void launch_rows(const GemmParams& p, long long tiles, hipStream_t s) {
  constexpr int W = ST_W, NT = ST_NT;
  const long long NQ = (p.N + W * NT * 16 - 1) / (W * NT * 16);
  const long long blocks = tiles * NQ * p.splits;
  if (blocks <= 0) return;
  gemm_stream_kernel<W, NT, ROWS, PAIRS, FMT, DUAL><<<(unsigned)blocks, W * 64, 0, s>>>(p);
}

template <int FMT, bool DUAL>
static void launch_fmt(const GemmParams& p, int rows, long long tiles, hipStream_t s) {
  if constexpr (FMT == WF_FP8) {
    // FP8 weights are the dense projections only: 64-row tiles
    launch_rows<64, DUAL ? 2 : 4, FMT, DUAL>(p, tiles, s);
  } else {
    // 16-row tiles take 4 pairs (256 k) per chunk; 32-row tiles 2 with a hi + lo
    // activation, 4 with one part; 64-row bf16 tiles 2 (with 4, one-part tiles took
    // 146 VGPRs: one 8-wave block per CU, whose load latency the dense decode GEMMs
    // could not hide; with 2, 90 VGPRs and two blocks per CU)
    constexpr int P16 = 4;
    constexpr int P = DUAL ? 2 : 4;
    if (rows == 16)
      launch_rows<16, P16, FMT, DUAL>(p, tiles, s);
    else if (rows == 32)
      launch_rows<32, P, FMT, DUAL>(p, tiles, s);
    else
      launch_rows<64, FMT == WF_BF16 ? 2 : P, FMT, DUAL>(p, tiles, s);
  }
}

template <int FMT>
static void launch_dual(const GemmParams& p, int rows, long long tiles, hipStream_t s) {
  if (p.a_lo != nullptr)
    launch_fmt<FMT, true>(p, rows, tiles, s);
  else
    launch_fmt<FMT, false>(p, rows, tiles, s);
}

void launch_gemm_stream(const GemmParams& p, int fmt, hipStream_t s) {
  // tile height: the grouped tile list's (16, 32 or 64 rows), 64 for dense GEMMs
  const int rows = !p.tile_expert ? 64 : p.rows_per_tile <= 16 ? 16 : p.rows_per_tile <= 32 ? 32 : 64;
  // FP8 weights come only as dense GEMMs (64-row tiles) and FP4 ones with one
  // segment (the FP4 path indexes seg[0] only); other shapes are not instantiated
  if ((fmt == WF_FP8 && rows != 64) || (fmt == WF_FP4 && p.nseg != 1)) return;
  const long long tiles = p.tile_expert ? p.max_tiles : (p.M + rows - 1) / rows;
  if (fmt == WF_FP4)
    launch_dual<WF_FP4>(p, rows, tiles, s);
  else if (fmt == WF_FP8)
    launch_dual<WF_FP8>(p, rows, tiles, s);
  else
    launch_dual<WF_BF16>(p, rows, tiles, s);
}

template <int ROWS, int PAIRS, bool QDUAL>
static void launch_pair_rows(const GemmParams& p, const GemmParams& q, hipStream_t s) {
  constexpr int W = ST_W, NT = ST_NT;
  const long long q_blocks = (long long)(q.N + W * NT * 16 - 1) / (W * NT * 16) * ((q.M + 63) / 64);
  const long long p_blocks = (long long)p.max_tiles * ((p.N + W * NT * 16 - 1) / (W * NT * 16)) * p.splits;
  if (q_blocks + p_blocks <= 0) return;
  gemm_stream_pair_kernel<W, NT, ROWS, PAIRS, WF_BF16, true, QDUAL>
      <<<(unsigned)(q_blocks + p_blocks), W * 64, 0, s>>>(p, q, (int)q_blocks);
}

template <bool QDUAL>
static void launch_pair_q(const GemmParams& p, const GemmParams& q, int rows, hipStream_t s) {
  if (rows == 16)
    launch_pair_rows<16, 4, QDUAL>(p, q, s);
  else if (rows == 32)
    launch_pair_rows<32, 2, QDUAL>(p, q, s);
  else
    launch_pair_rows<64, 2, QDUAL>(p, q, s);
}

void launch_gemm_stream_pair(const GemmParams& p, const GemmParams& q, hipStream_t s) {
  // the pair covers bf16 experts with hi + lo activations and a one-segment dense
  // bf16 GEMM of at most one 64-row tile in one split; anything else runs as two launches
  const bool ok = p.tile_expert && p.a_lo && p.nseg == 1 && !q.tile_expert && q.nseg == 1 &&
                  q.splits == 1 && q.M <= 64;
  if (!ok) {
    launch_gemm_stream(q, WF_BF16, s);
    launch_gemm_stream(p, WF_BF16, s);
    return;
  }
  const int rows = p.rows_per_tile <= 16 ? 16 : p.rows_per_tile <= 32 ? 32 : 64;
  if (q.a_lo)
    launch_pair_q<true>(p, q, rows, s);
  else
    launch_pair_q<false>(p, q, rows, s);
}

}  // namespace lmoe
