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
// is stored at piece p ^ ((r >> 1) & 3).  A 16-byte LDS read is served four
// lanes at a time over 32 four-byte banks, so the rows r .. r+7 that neighbouring
// lanes of a group read must fill the 128 bytes of banks without overlap: rows
// 2j and 2j+1 take the two 64-byte halves and bits 1..2 of r separate the four
// pairs.  (An XOR with bits 2..3 doubled up banks and read at 112 B/clk per CU
// against 198 B/clk conflict-free, measured.)  A direct load writes lane l of a
// wave to slot l of a 1 KB chunk (16 rows), so each lane fetches the global
// piece that belongs in its slot.
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
  return row * BG_ROWB + ((piece ^ ((row >> 1) & 3)) << 4);
}

#ifndef LMOE_BIG_STAGES
#define LMOE_BIG_STAGES 4
#endif
template <bool DUAL>
constexpr int bg_stages() { return DUAL ? 3 : LMOE_BIG_STAGES; }

// waves per block: 4 (2 x 2 waves of 128 x 128) or 8 (2 x 4 waves of 128 x 64, two
// waves per SIMD: one wave's LDS reads and waits overlap the other's MFMAs)
#ifndef LMOE_BIG_WAVES
#define LMOE_BIG_WAVES 8
#endif
constexpr int BG_WAVES = LMOE_BIG_WAVES;
#ifndef LMOE_BIG_PIPE
#define LMOE_BIG_PIPE 1
#endif
#ifndef LMOE_BIG_NT
#define LMOE_BIG_NT 1
#endif
#ifndef LMOE_BIG_XCD
#define LMOE_BIG_XCD 1
#endif
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

// Output tile through LDS.  A lane's accumulators hold 4 columns of one row, so
// direct stores write 32 (bf16) or 64 (fp32) bytes of each of 16 rows per
// instruction; L2 reads every line written that way before merging (measured:
// about as many bytes fetched as written).  Instead the finished tile goes to LDS,
// which the operand ring no longer needs, 128 rows at a time, and every thread
// then stores 16-byte chunks along rows: a wave covers whole 128-byte lines.
//
// Staged half: [plane][128 rows][BG_BN elements of EB bytes]; 16-byte chunk c of
// row r sits at chunk c ^ (r & 7), so that the writes of 8 neighbouring rows and
// the reads along a row fall in distinct banks.  N is a multiple of 8 (every width
// the layer accepts is a multiple of 16): a chunk is entirely inside or outside.
template <int EPI>
__device__ __forceinline__ void big_epilogue(const GemmParams& p, uint8_t* smem, const f32x4_t (&acc)[8][BG_MB],
                                             int expert, int split, int row0, int rows, int n0, int wn, int wm,
                                             int r16, int g, int tid) {
  constexpr int PL = epi_planes<EPI>();
  constexpr int EB = epi_bytes<EPI>();
  constexpr int HR = 128;                  // rows per half
  constexpr int RB = BG_BN * EB;           // staged bytes per row and plane
  constexpr int CPR = RB / 16;             // 16-byte chunks per row
  constexpr int PLANEB = HR * RB;
  constexpr int PER = PL * HR * CPR / BG_THREADS;  // chunks per thread and half
  static_assert(PL * HR * CPR % BG_THREADS == 0, "whole chunks per thread");
  // fp32 kinds with an addend (the bias, the old output) stage acc * ts and add it
  // on the way out, loading the addends of 4 chunks before their 4 stores
  constexpr bool ADD = EPI == EPI_F32 || EPI == EPI_F32_ADD;
  constexpr int SE = ADD ? EPI_F32_ADD : EPI;  // the kind whose values are staged
  constexpr int BATCH = ADD ? 4 : PER;
  static_assert(PER % BATCH == 0, "whole batches");
  const int wrow = wm * (BG_MB * 16);      // first tile row of this wave
  const float ts = epi_tscale(p, expert);
  float rf[BG_MB];
#pragma unroll
  for (int b = 0; b < BG_MB; ++b) {
    const int m = wrow + b * 16 + r16;
    rf[b] = m < rows ? epi_rowf<EPI>(p, row0 + m) : 1.0f;
  }
  epi_wait_all();
  // the staged values of all eight waves at once (the halves are staged in turn,
  // and a wave computing its values only in its own half left the other SIMD
  // slots idle): fp32, or bf16 pairs per plane
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t sf[EB == 4 ? 8 : 1][BG_MB];
  u32x2_t sb[EB == 2 ? PL : 1][EB == 2 ? 8 : 1][BG_MB];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < BG_MB; ++b) {
      const Epi4 o = epi_math<SE>(p, acc[a][b], ts, rf[b], zero);
      if constexpr (EB == 4) {
        sf[a][b] = o.v0;
      } else {
        epi_pack<SE>(o.v0, sb[0][a][b], sb[PL - 1][a][b]);
      }
    }
  __syncthreads();  // every wave has read its last operands from the ring

#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wrow / HR == half) {
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int col = wn * 128 + a * 16 + 4 * g;
#pragma unroll
        for (int b = 0; b < BG_MB; ++b) {
          const int r = wrow % HR + b * 16 + r16;
          if constexpr (EB == 4) {
            *reinterpret_cast<f32x4_t*>(smem + r * RB + (((col >> 2) ^ (r & 7)) << 4)) = sf[a][b];
          } else {
            const int at = r * RB + (((col >> 3) ^ (r & 7)) << 4) + ((col >> 2) & 1) * 8;
            *reinterpret_cast<u32x2_t*>(smem + at) = sb[0][a][b];
            if constexpr (PL == 2) *reinterpret_cast<u32x2_t*>(smem + PLANEB + at) = sb[PL - 1][a][b];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i0 = 0; i0 < PER; i0 += BATCH) {
      u32x4_t d[BATCH];
      f32x4_t ad[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int id = tid + (i0 + i) * BG_THREADS;
        const int plane = id / (HR * CPR), rem = id % (HR * CPR);
        const int r = rem / CPR, c = rem % CPR;
        d[i] = *reinterpret_cast<const u32x4_t*>(smem + plane * PLANEB + r * RB + ((c ^ (r & 7)) << 4));
        ad[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (ADD) {
          const int m = half * HR + r, n = n0 + c * 4;
          if (m < rows && n < p.N) {
            if constexpr (EPI == EPI_F32_ADD)
              ad[i] = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(p.C) +
                                                        (long long)(row0 + m) * p.ldc + n);
            else if (p.bias)
              ad[i] = *reinterpret_cast<const f32x4_t*>(p.bias + n);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int id = tid + (i0 + i) * BG_THREADS;
        const int plane = id / (HR * CPR), rem = id % (HR * CPR);
        const int r = rem / CPR, c = rem % CPR;
        const int m = half * HR + r, n = n0 + c * (16 / EB);
        if (m >= rows || n >= p.N) continue;
        const long long row = row0 + m;
        u32x4_t* dst;
        u32x4_t v = d[i];
        if constexpr (EPI == EPI_PARTIAL) {
          dst = reinterpret_cast<u32x4_t*>(p.partial + (long long)split * p.partial_stride + row * p.N + n);
        } else if constexpr (EB == 2) {
          dst = reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(plane ? p.C2 : p.C) + row * p.ldc + n);
        } else {
          dst = reinterpret_cast<u32x4_t*>(reinterpret_cast<float*>(p.C) + row * p.ldc + n);
          if constexpr (ADD) {
            f32x4_t w = __builtin_bit_cast(f32x4_t, d[i]);
            if (EPI == EPI_F32_ADD) w = ad[i] + w;
            else if (p.bias) w += ad[i];
            v = __builtin_bit_cast(u32x4_t, w);
          }
        }
#if LMOE_BIG_NT
        __builtin_nontemporal_store(v, dst);
#else
        *dst = v;
#endif
      }
    }
    if (half == 0) __syncthreads();  // the copy has read the staged half
  }
}

template <bool DUAL, int EPI>
__global__ __launch_bounds__(BG_THREADS, 1) void gemm_big_kernel(GemmParams p) {
  constexpr int NPART = DUAL ? 2 : 1;
  constexpr int STAGES = bg_stages<DUAL>();
  constexpr int STAGEB = BG_TILEB * (1 + NPART);  // weights + activation part(s)
  // the epilogue stages half a tile (128 rows, every plane) in the ring's LDS
  static_assert(epi_planes<EPI>() * 128 * BG_BN * epi_bytes<EPI>() <= STAGES * STAGEB,
                "the staged half of the output tile must fit in the ring");
  constexpr int LOADS = BG_CPW * (1 + NPART);     // direct loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;  // 128 weight rows x BG_MB * 16 activation rows
  const int r16 = lane & 15, g = lane >> 4;

  const int NQ = (p.N + BG_BN - 1) / BG_BN;
  int item = blockIdx.x;
  bool mapped = false;
  int j = 0, q = 0;
#if LMOE_BIG_XCD
  // Blocks are dealt to the 8 XCDs in turn (block b to XCD b % 8), and each XCD
  // has its own L2.  Expert tiles: XCD x takes the contiguous tile range
  // [x TPX, (x + 1) TPX) of the n_tiles listed, each tile's NQ column blocks in a
  // row, so that the tiles of one expert run on one XCD at about the same time and
  // share its weight slices (and each tile's activations) in that L2.  Row tiles
  // of a dense product: tile t on XCD t % 8, its column blocks in a row.
  if (p.splits == 1) {
    const int b = blockIdx.x, x = b % 8, sx = b / 8;
    if (p.tile_expert) {
      const int tpx = (p.n_tiles[0] + 7) / 8;
      const int tl = sx / NQ;
      if (tl >= tpx) return;
      j = x * tpx + tl;
      q = sx % NQ;
    } else {
      j = (b / (NQ * 8)) * 8 + x;
      q = sx % NQ;
    }
    mapped = true;
  }
#endif
  int split = 0;
  if (!mapped) {
    split = item % p.splits;
    item /= p.splits;
    q = item % NQ;
    j = item / NQ;
  }
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
  // l%4, which holds logical piece (l%4) ^ ((row >> 1) & 3).  Rows past the
  // tile are clamped to a valid row: their products land in outputs that are
  // never stored.
  uint32_t w_off[BG_CPW], x_off[BG_CPW];
#pragma unroll
  for (int i = 0; i < BG_CPW; ++i) {
    const int row = 16 * (wave + BG_WAVES * i) + (lane >> 2);
    const int piece = (lane & 3) ^ ((row >> 1) & 3);
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

  // direct load u of stage kt: chunk i = u / (1 + NPART) of the weights (part 0),
  // the activations (1) or their low halves (2)
  auto issue_one = [&](int kt, int u) {
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
    const int i = u / (1 + NPART), part = u % (1 + NPART);
    const int chunk = (wave + BG_WAVES * i) * 1024;
    // uniform base + 32-bit byte offset (below 4 GB: a 256-row weight slice and
    // an activation matrix of at most 2^31 elements), the scalar-base form
    if (part == 0)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(B + k) + (uint64_t)(w_off[i] * 2u),
                                       st + chunk, 16, 0, 0);
    else if (part == 1)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(A + k) + (uint64_t)(x_off[i] * 2u),
                                       st + BG_TILEB + chunk, 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(Alo + k) + (uint64_t)(x_off[i] * 2u),
                                       st + 2 * BG_TILEB + chunk, 16, 0, 0);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) issue_one(kt, u);
  };

  f32x4_t acc[8][BG_MB];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < BG_MB; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // a step's fragments: activation part 0, the weights, then part 1, so that part
  // 0's MFMAs can start while the rest arrive
  auto read_frags = [&](int kt, u32x4_t (&wf)[8], u32x4_t (&xf)[NPART][BG_MB]) {
    const uint8_t* base = smem + (kt % STAGES) * STAGEB;
#pragma unroll
    for (int b = 0; b < BG_MB; ++b)
      xf[0][b] = *reinterpret_cast<const u32x4_t*>(base + BG_TILEB + bg_off(wm * (BG_MB * 16) + b * 16 + r16, g));
#pragma unroll
    for (int a = 0; a < 8; ++a)
      wf[a] = *reinterpret_cast<const u32x4_t*>(base + bg_off(wn * 128 + a * 16 + r16, g));
    if constexpr (DUAL) {
#pragma unroll
      for (int b = 0; b < BG_MB; ++b)
        xf[1][b] = *reinterpret_cast<const u32x4_t*>(base + 2 * BG_TILEB +
                                                     bg_off(wm * (BG_MB * 16) + b * 16 + r16, g));
    }
  };
  auto mfmas = [&](const u32x4_t (&wf)[8], const u32x4_t (&xf)[NPART][BG_MB]) {
#pragma unroll
    for (int part = 0; part < NPART; ++part)
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < BG_MB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xf[part][b], acc[a][b]);
  };

  if constexpr (!DUAL && LMOE_BIG_PIPE) {
    // Next step's fragments are read while this step's MFMAs run: after step
    // kt + 1's barrier the wave reads that step's activation fragments into a
    // second set and, as soon as the 4 MFMAs of weight fragment a have issued,
    // reloads fragment a from step kt + 1.  With every wave released by one
    // barrier, reads issued at the barrier and waited for would otherwise leave the
    // MFMA pipes idle while 96 KB of fragments stream out of LDS.  A ring slot is
    // free once every wave holds its fragments in registers, so all STAGES slots
    // carry loads:
    //   before step kt's barrier: stages issued 0 .. min(kt - 1 + STAGES, KT - 1);
    //   stage kt + 1 must be complete: later stages outstanding min(STAGES - 2, KT - 2 - kt)
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < KT) issue(s);
    wait_vmcnt((min(STAGES, KT) - 1) * LOADS);
    asm volatile("s_barrier" ::: "memory");
    u32x4_t wf[8], xa[1][BG_MB], xb[1][BG_MB];
    read_frags(0, wf, xa);
    // a step with a next one; every such step has the same shape, so the compiler's
    // wait insertion sees the current set complete (the explicit wait) and the next
    // set's reads as the only ones outstanding.  The last step runs on its own.
    auto step = [&](int kt, const u32x4_t (&xc)[1][BG_MB], u32x4_t (&xn)[1][BG_MB]) {
      // this wave's reads of step kt are in registers; after the barrier no wave
      // reads slot kt % STAGES any more
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
      wait_vmcnt(min(STAGES - 2, KT - 2 - kt) * LOADS);
      asm volatile("s_barrier" ::: "memory");
      const uint8_t* base = smem + ((kt + 1) % STAGES) * STAGEB;
#pragma unroll
      for (int b = 0; b < BG_MB; ++b)
        xn[0][b] = *reinterpret_cast<const u32x4_t*>(base + BG_TILEB + bg_off(wm * (BG_MB * 16) + b * 16 + r16, g));
#pragma unroll
      for (int a = 0; a < 8; ++a) {
#pragma unroll
        for (int b = 0; b < BG_MB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xc[0][b], acc[a][b]);
        wf[a] = *reinterpret_cast<const u32x4_t*>(base + bg_off(wn * 128 + a * 16 + r16, g));
        // stage kt + STAGES (into the slot every wave finished reading before this
        // step's barrier), its loads spread over the step: issued together after
        // the barrier, all waves' loads queue at the memory unit at once and each
        // wave's MFMAs wait behind its own loads
#pragma unroll
        for (int u = a * LOADS / 8; u < (a + 1) * LOADS / 8; ++u)
          if (kt + STAGES < KT) issue_one(kt + STAGES, u);
      }
      // keep the interleave: the activation reads, then 4 MFMAs and one read per a
      __builtin_amdgcn_sched_group_barrier(0x100, BG_MB, 0);
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        __builtin_amdgcn_sched_group_barrier(0x008, BG_MB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {
      step(kt, xa, xb);
      step(kt + 1, xb, xa);
    }
    if (kt + 1 < KT) {  // two steps left: one more with a next step, ending in xb
      step(kt, xa, xb);
#pragma unroll
      for (int b = 0; b < BG_MB; ++b) xa[0][b] = xb[0][b];
    }
    mfmas(wf, xa);
  } else {
    // all of a step's fragments are read before its first MFMA (the scheduler would
    // otherwise reuse one register for the weight fragments and wait for each read
    // in turn)
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
      u32x4_t wf[8], xf[NPART][BG_MB];
      read_frags(kt, wf, xf);
      __builtin_amdgcn_sched_barrier(0);
      // stage kt + STAGES - 1 goes to the slot every wave finished reading before
      // this barrier; its loads are spread over the MFMAs (see the pipelined path)
      const bool more = kt + STAGES - 1 < KT;
#pragma unroll
      for (int part = 0; part < NPART; ++part)
#pragma unroll
        for (int a = 0; a < 8; ++a) {
#pragma unroll
          for (int b = 0; b < BG_MB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xf[part][b], acc[a][b]);
          const int grp = part * 8 + a;
#pragma unroll
          for (int u = grp * LOADS / (8 * NPART); u < (grp + 1) * LOADS / (8 * NPART); ++u)
            if (more) issue_one(kt + STAGES - 1, u);
        }
    }
  }

  big_epilogue<EPI>(p, smem, acc, expert, split, row0, rows, n0, wn, wm, r16, g, tid);
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
    case EPI_GATE_BF16: f(std::integral_constant<int, EPI_GATE_BF16>{}); break;
    default: break;
  }
}

int gemm_big_setup() {
  const int kinds[] = {EPI_PARTIAL, EPI_BF16_HILO, EPI_SQRELU_HILO, EPI_SQRELU_BF16,
                       EPI_F32, EPI_F32_ADD, EPI_GATE_F32, EPI_GATE_BF16};
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
         epi == EPI_SQRELU_BF16 || epi == EPI_F32 || epi == EPI_F32_ADD || epi == EPI_GATE_F32 ||
         epi == EPI_GATE_BF16;
}

void launch_gemm_big(const GemmParams& p, hipStream_t s) {
  const int NQ = (p.N + BG_BN - 1) / BG_BN;
  long long tiles = p.tile_expert ? p.max_tiles : (p.M + BG_BM - 1) / BG_BM;
#if LMOE_BIG_XCD
  if (p.splits == 1) tiles = (tiles + 7) / 8 * 8;  // whole groups of 8 tiles
#endif
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
