// Large-tile MFMA GEMM for many rows per tile (prefill-like shapes).
//
// Block tile: 256 weight rows (output columns n) x 256 activation rows, k step
// 32, eight waves in a 2 x 4 arrangement, each wave 128 x 64 = 8 x 4 MFMA
// 16x16x32 tiles (128 fp32 accumulators per lane), two waves per SIMD so that
// one wave's LDS reads and waits overlap the other's MFMAs (one wave per SIMD
// with 128 x 128 wave tiles ran 11 % slower at prefill).  Per k step a wave
// reads 12 (16 in dual mode) 16-byte fragments for 32 (64) MFMAs.  A wave's 64
// activation rows are the 16-row groups wm, wm + 4, wm + 8, wm + 12 of the tile:
// in a partly filled expert tile the groups past its rows are skipped (no reads,
// no MFMAs), and the interleave spreads them evenly over the four SIMDs (at the
// Zipf-routed prefill this cut the expert GEMMs by 2-4 %).
//
// Operand tiles go from global memory straight into a ring of LDS buffers
// (global_load_lds, 16 bytes per lane, no staging registers), and a wave reads a
// step's fragments while the previous step's MFMAs run.
//
// Single mode (one activation part): a ring slot holds two k steps of one operand,
// rows of 128 bytes; three slots for the weights and two for the activations fill
// the 160 KB of LDS.  A direct load then covers 8 rows x 128 bytes, whole lines:
// with one k step per slot each load touched 16 half lines, and as the other half
// came a step later, after 64 KB of other lines, L1 fetched most lines twice
// (counters: 74 % of tag accesses missed; the loads are what the kernel waits on).
// Odd steps wait for the next pair (the weights of the pair after it may stay in
// flight), pass a barrier and refill the slots the last pair left: the weights,
// which come from HBM, are issued three pairs ahead, the activations two.  Even
// steps have no wait and no barrier.  The 16-byte piece p of row r sits at
// p ^ (r & 7), so the 8 rows a lane group reads at one piece fill all 32 banks.
// Prefill 3.78 -> 3.72 ms with paired steps in two shared slots, 3.73 -> 3.53 ms
// with the split ring (expert up and down 9 % faster each).

// Dual mode (hi + lo activation parts, 48 KB per k step): a ring of 3 one-step
// stages.  While step k computes, the loads of steps k+1 .. k+2 are in flight;
// each step waits for its own loads (vmcnt), then one barrier makes every wave's
// loads visible and frees the buffer the next issue overwrites.  LDS rows are 64
// bytes (32 bf16 of one k step); the 16-byte piece p of row r is stored at piece
// p ^ ((r >> 1) & 3).  A 16-byte LDS read is served four lanes at a time over 32
// four-byte banks, so the rows r .. r+7 that neighbouring lanes of a group read
// must fill the 128 bytes of banks without overlap: rows 2j and 2j+1 take the two
// 64-byte halves and bits 1..2 of r separate the four pairs.  (An XOR with bits
// 2..3 doubled up banks and read at 112 B/clk per CU against 198 B/clk
// conflict-free, measured.)
//
// A direct load writes lane l of a wave to slot l of a 1 KB chunk, so each lane
// fetches the global piece that belongs in its slot.
//
// k layout inside a 32-wide k step: lane group g = lane / 16 holds k = 8g .. 8g+7
// for both operands (in single mode step 2j + h is half h of pair j's rows).
// DUAL: the activation tile comes as two bf16 parts (hi + lo) and every weight
// fragment feeds both.
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

// single mode: rows of two k steps (128 bytes, 8 pieces), piece p of row r at
// p ^ (r & 7), so that any 8 consecutive rows read at one logical piece cover all
// 32 banks
constexpr int BG_PROWB = 2 * BG_ROWB;
constexpr int BG_PTILEB = 256 * BG_PROWB;  // 32 KB per operand and pair
__device__ __forceinline__ int bg_poff(int row, int piece) {
  return row * BG_PROWB + ((piece ^ (row & 7)) << 4);
}

// ring: 3 stages of one k step, 48 KB each (dual), or 5 slots of two k steps of one
// operand, 32 KB each (single: three for the weights, two for the activations)
template <bool DUAL>
constexpr int bg_stages() { return DUAL ? 3 : 5; }
template <bool DUAL>
constexpr int bg_stage_bytes() { return DUAL ? 3 * BG_TILEB : BG_PTILEB; }

// 8 waves of 128 x 64 (2 x 4), two waves per SIMD: one wave's LDS reads and waits
// overlap the other's MFMAs
constexpr int BG_WAVES = 8;
constexpr int BG_THREADS = 64 * BG_WAVES;
constexpr int BG_WM = BG_WAVES / 2;        // waves along the activation rows
constexpr int BG_MB = BG_BM / BG_WM / 16;  // 16-row activation tiles per wave
constexpr int BG_CPW = 16 / BG_WAVES;      // 1 KB chunks per wave per operand tile

// wait until at most n of this wave's vector-memory loads are outstanding
__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at max
#define VMCNT_WAIT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
  switch (n) {
    case 0: VMCNT_WAIT(0); break;
    case 4: VMCNT_WAIT(4); break;
    case 6: VMCNT_WAIT(6); break;
    case 8: VMCNT_WAIT(8); break;
    case 12: VMCNT_WAIT(12); break;
    case 16: VMCNT_WAIT(16); break;
    case 24: VMCNT_WAIT(24); break;
    default: VMCNT_WAIT(0); break;
  }
#undef VMCNT_WAIT
}

// the same with a compile-time count (one wait instruction, no selection)
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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
  const float ts = epi_tscale(p, expert);
  float rf[BG_MB];
#pragma unroll
  for (int b = 0; b < BG_MB; ++b) {
    const int m = (4 * b + wm) * 16 + r16;  // the wave's 16-row group b
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
    // group 4b + wm lies in half b / 2 (wm < 4): every wave stages in both halves
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int col = wn * 128 + a * 16 + 4 * g;
#pragma unroll
      for (int b = 2 * half; b < 2 * half + 2; ++b) {
        const int r = (4 * (b % 2) + wm) * 16 + r16;
        if constexpr (EB == 4) {
          *reinterpret_cast<f32x4_t*>(smem + r * RB + (((col >> 2) ^ (r & 7)) << 4)) = sf[a][b];
        } else {
          const int at = r * RB + (((col >> 3) ^ (r & 7)) << 4) + ((col >> 2) & 1) * 8;
          *reinterpret_cast<u32x2_t*>(smem + at) = sb[0][a][b];
          if constexpr (PL == 2) *reinterpret_cast<u32x2_t*>(smem + PLANEB + at) = sb[PL - 1][a][b];
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
        __builtin_nontemporal_store(v, dst);
      }
    }
    if (half == 0) __syncthreads();  // the copy has read the staged half
  }
}

// ONESEG: the reduction runs over one segment (every GEMM but the router's three
// weight pieces): a stage's load addresses are a base plus the stage's k offset,
// with no segment selection in the loop
template <bool DUAL, int EPI, bool ONESEG>
__global__ __launch_bounds__(BG_THREADS, 1) void gemm_big_kernel(GemmParams p) {
  constexpr int NPART = DUAL ? 2 : 1;
  constexpr int STAGES = bg_stages<DUAL>();
  constexpr int STAGEB = bg_stage_bytes<DUAL>();  // weights + activation part(s)
  // the epilogue stages half a tile (128 rows, every plane) in the ring's LDS
  static_assert(epi_planes<EPI>() * 128 * BG_BN * epi_bytes<EPI>() <= STAGES * STAGEB,
                "the staged half of the output tile must fit in the ring");
  constexpr int LOADS = BG_CPW * (1 + NPART);     // dual mode: direct loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS chunk bases stay scalar
  const int wn = wave & 1, wm = wave >> 1;  // 128 weight rows x the groups 4b + wm
  const int r16 = lane & 15, g = lane >> 4;

  const int NQ = (p.N + BG_BN - 1) / BG_BN;
  int item = blockIdx.x;
  bool mapped = false;
  int j = 0, q = 0;
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

  // This wave loads 1 KB chunks c = wave + BG_WAVES i of each operand tile: lane l
  // fills slot l of the chunk.  Dual: rows of one k step, row 16c + l/4, stored piece
  // l%4, which holds logical piece (l%4) ^ ((row >> 1) & 3).  Single: rows of two k
  // steps, row 8c + l/8, stored piece l%8 holding logical piece (l%8) ^ (row & 7).
  // Rows past the tile are clamped to a valid row: their products land in outputs
  // that are never stored.
  constexpr int CPW = DUAL ? BG_CPW : 2 * BG_CPW;  // chunks per wave and operand
  uint32_t w_off[CPW], x_off[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int row = DUAL ? 16 * (wave + BG_WAVES * i) + (lane >> 2) : 8 * (wave + BG_WAVES * i) + (lane >> 3);
    const int piece = DUAL ? (lane & 3) ^ ((row >> 1) & 3) : (lane & 7) ^ (row & 7);
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

  // dual mode: direct load u of stage kt: chunk i = u / (1 + NPART) of the weights
  // (part 0), the activations (1) or their low halves (2)
  auto issue_one = [&](int kt, int u) {
    int k = kbeg + kt * BG_BK;
    const uint16_t* A = A0;
    const uint16_t* B = B0;
    if constexpr (!ONESEG) {
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


  // Wave (wn, wm) multiplies the tile's 16-row activation groups 4b + wm: a partly
  // filled tile's empty groups fall evenly on the four SIMDs, and only the groups
  // that hold rows (the wave's first nb) are read and multiplied (wave-uniform).
  const int nb = min(BG_MB, max(0, (((rows + 15) >> 4) - wm + 3) >> 2));
  if constexpr (!DUAL) {
    // Paired steps: a ring slot holds two k steps (64 k) of one operand in rows of
    // 128 bytes, so a direct load of 8 rows x 128 bytes fetches whole lines (the
    // half-line loads of 32-k rows brought every line into L1 twice).  Three weight
    // slots and two activation slots (160 KB): step kt reads its fragments during
    // step kt - 1 (after that step's barrier, if any).  An odd step kt = 2j + 1
    // waits for pair j + 1 (the weights of pair j + 2 may stay in flight), passes
    // the barrier, and issues the activations of pair j + 2 and the weights of pair
    // j + 3 into the slots pair j left (every wave finished reading it in step 2j);
    // an even step needs no wait and no barrier.  The weights, which stream from
    // HBM, so get three steps more to land than the activations.
    const int KP = KT / 2;  // K is a multiple of 64 (the widths), so KT is even
    // slot bases: weight slot s at s * 32 KB (pair pr in slot pr % 3), activation
    // slot t at (3 + t) * 32 KB (pair pr in slot pr % 2)
    auto wslot = [&](int s) { return smem + s * BG_PTILEB; };
    auto aslot = [&](int t) { return smem + (3 + t) * BG_PTILEB; };
    // chunk i of pair pr's weights or activations (a wave's 4 of each operand) into
    // the slot at dst
    auto issue_w = [&](int pr, int i, uint8_t* dst) {
      int k = kbeg + pr * 2 * BG_BK;
      const uint16_t* B = B0;
      if constexpr (!ONESEG) {
        if (k >= K0 && p.nseg > 1) {
          k -= K0;
          B = B1;
          if (k >= K1 && p.nseg > 2) {
            k -= K1;
            B = B2;
          }
        }
      }
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(B + k) + (uint64_t)(w_off[i] * 2u),
                                       dst + (wave + BG_WAVES * i) * 1024, 16, 0, 0);
    };
    auto issue_a = [&](int pr, int i, uint8_t* dst) {
      int k = kbeg + pr * 2 * BG_BK;
      const uint16_t* A = A0;
      if constexpr (!ONESEG) {
        if (k >= K0 && p.nseg > 1) {
          k -= K0;
          A = A1;
          if (k >= K1 && p.nseg > 2) {
            k -= K1;
            A = A2;
          }
        }
      }
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(A + k) + (uint64_t)(x_off[i] * 2u),
                                       dst + (wave + BG_WAVES * i) * 1024, 16, 0, 0);
    };
    // fragment: row r of the slot at base, lane group g's 16 bytes of half h of the
    // 128-byte row (step 2j + h of the slot's pair j)
    auto frag = [&](const uint8_t* base, int h, int r) {
      return *reinterpret_cast<const u32x4_t*>(base + bg_poff(r, h * 4 + g));
    };
    // prologue: W0 A0 W1 A1 W2 in this order, so that pair 1 is complete when only
    // W2's loads are outstanding
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_w(0, i, wslot(0));
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_a(0, i, aslot(0));
    if (KP > 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) issue_w(1, i, wslot(1));
#pragma unroll
      for (int i = 0; i < 4; ++i) issue_a(1, i, aslot(1));
      if (KP > 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) issue_w(2, i, wslot(2));
        wait_vmcnt_c<12>();
      } else {
        wait_vmcnt_c<8>();
      }
    } else {
      wait_vmcnt_c<0>();
    }
    asm volatile("s_barrier" ::: "memory");
    auto single = [&](auto nbc) {
    constexpr int NB = decltype(nbc)::value;
    u32x4_t wf[8], xa[1][BG_MB], xb[1][BG_MB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xa[0][b] = frag(aslot(0), 0, (4 * b + wm) * 16 + r16);
#pragma unroll
    for (int a = 0; a < 8; ++a)
      if constexpr (NB > 0) wf[a] = frag(wslot(0), 0, wn * 128 + a * 16 + r16);
    // step kt with a next step, whose fragments sit in the slots wb and ab.  ODD
    // steps wait and pass the barrier: WAIT4, the weights of pair kt / 2 + 2 exist
    // (their 4 loads may stay in flight), which is also when the activations of
    // that pair are issued (into wa); ISSUEW: the weights of pair kt / 2 + 3 exist
    // and are issued (into ww).  The compiler's wait insertion sees the current
    // fragments complete and the next ones as the only reads outstanding.
    auto step = [&](int kt, const uint8_t* wb, const uint8_t* ab, uint8_t* ww, uint8_t* wa,
                    const u32x4_t (&xc)[1][BG_MB], u32x4_t (&xn)[1][BG_MB], auto odd, auto wait4, auto issuew) {
      constexpr bool ODD = decltype(odd)::value;
      constexpr bool WAIT4 = decltype(wait4)::value;
      constexpr bool ISSUEW = decltype(issuew)::value;
      constexpr int H = ODD ? 0 : 1;  // half of the next step's pair
      if constexpr (ODD) {
        // this wave's reads of step kt are in registers, and pair kt / 2 + 1 has landed
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
        if constexpr (WAIT4)
          wait_vmcnt_c<4>();
        else
          wait_vmcnt_c<0>();
        asm volatile("s_barrier" ::: "memory");
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) xn[0][b] = frag(ab, H, (4 * b + wm) * 16 + r16);
#pragma unroll
      for (int a = 0; a < 8; ++a) {
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xc[0][b], acc[a][b]);
        if constexpr (NB > 0) wf[a] = frag(wb, H, wn * 128 + a * 16 + r16);
        // the step's loads spread over its MFMAs (issued together after the
        // barrier, all waves' loads queue at the memory unit at once and each
        // wave's MFMAs wait behind its own loads): activations first, so that the
        // next odd step's wait leaves only the newest weights in flight
        if constexpr (ODD && WAIT4) {
          if (a < 4) issue_a(kt / 2 + 2, a, wa);
          else if (ISSUEW) issue_w(kt / 2 + 3, a - 4, ww);
        }
      }
      // keep the interleave: the activation reads, then NB MFMAs and one read per a
      if constexpr (NB > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    const std::true_type yes{};
    const std::false_type no{};
    int kt = 0;
    int ws = 0;  // weight slot of pair kt / 2
    // one pair: its even step reads the second half of pair j = kt / 2, its odd step
    // the first half of pair j + 1 and refills pair j's slots
    auto pair = [&](auto wait4, auto issuew) {
      const int ws1 = ws == 2 ? 0 : ws + 1;
      const int t = (kt >> 1) & 1;
      step(kt, wslot(ws), aslot(t), nullptr, nullptr, xa, xb, no, no, no);
      step(kt + 1, wslot(ws1), aslot(t ^ 1), wslot(ws), aslot(t), xb, xa, yes, wait4, issuew);
      ws = ws1;
      kt += 2;
    };
    while (kt + 6 < KT) pair(yes, yes);  // pair kt / 2 + 3 exists
    if (kt + 4 < KT) pair(yes, no);      // pair kt / 2 + 2 is the last
    if (kt + 2 < KT) pair(no, no);       // pair kt / 2 + 1 is the last: nothing to issue
    // the last pair: its second step has no next
    step(kt, wslot(ws), aslot((kt >> 1) & 1), nullptr, nullptr, xa, xb, no, no, no);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xb[0][b], acc[a][b]);
    };
    switch (nb) {
      case 4: single(std::integral_constant<int, 4>{}); break;
      case 3: single(std::integral_constant<int, 3>{}); break;
      case 2: single(std::integral_constant<int, 2>{}); break;
      case 1: single(std::integral_constant<int, 1>{}); break;
      default: single(std::integral_constant<int, 0>{}); break;
    }
  } else {
    // all of a step's fragments are read before its first MFMA (the scheduler would
    // otherwise reuse one register for the weight fragments and wait for each read
    // in turn)
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) issue(s);
    // FAST: a steady-state step (kt + STAGES - 1 < KT): STAGES - 2 later stages are in
    // flight (a compile-time wait) and stage kt + STAGES - 1 exists
    auto dual = [&](auto nbc) {
    constexpr int NB = decltype(nbc)::value;
    auto dstep = [&](int kt, auto fast) {
      constexpr bool FAST = decltype(fast)::value;
      // stages issued after step kt: min(STAGES - 2, KT - 1 - kt)
      if constexpr (FAST)
        wait_vmcnt_c<(STAGES - 2) * LOADS>();
      else
        wait_vmcnt(min(STAGES - 2, KT - 1 - kt) * LOADS);
      // a plain barrier: the step's own loads were waited for above; a fenced
      // __syncthreads would wait for every load in flight, draining the ring
      asm volatile("s_barrier" ::: "memory");
      // activation part 0, the weights, then part 1, so that part 0's MFMAs can
      // start while the rest arrive
      u32x4_t wf[8], xf[NPART][BG_MB];
      {
        const uint8_t* base = smem + (kt % STAGES) * STAGEB;
#pragma unroll
        for (int b = 0; b < NB; ++b)
          xf[0][b] = *reinterpret_cast<const u32x4_t*>(base + BG_TILEB + bg_off((4 * b + wm) * 16 + r16, g));
#pragma unroll
        for (int a = 0; a < 8; ++a)
          if constexpr (NB > 0) wf[a] = *reinterpret_cast<const u32x4_t*>(base + bg_off(wn * 128 + a * 16 + r16, g));
#pragma unroll
        for (int b = 0; b < NB; ++b)
          xf[1][b] = *reinterpret_cast<const u32x4_t*>(base + 2 * BG_TILEB + bg_off((4 * b + wm) * 16 + r16, g));
      }
      __builtin_amdgcn_sched_barrier(0);
      // stage kt + STAGES - 1 goes to the slot every wave finished reading before
      // this barrier; its loads are spread over the MFMAs (see the pipelined path)
      const bool more = FAST || kt + STAGES - 1 < KT;
#pragma unroll
      for (int part = 0; part < NPART; ++part)
#pragma unroll
        for (int a = 0; a < 8; ++a) {
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[a][b] = mfma_16x16x32(wf[a], xf[part][b], acc[a][b]);
          const int grp = part * 8 + a;
#pragma unroll
          for (int u = grp * LOADS / (8 * NPART); u < (grp + 1) * LOADS / (8 * NPART); ++u)
            if (more) issue_one(kt + STAGES - 1, u);
        }
    };
    int kt = 0;
    for (; kt + STAGES - 1 < KT; ++kt) dstep(kt, std::integral_constant<bool, true>{});
    for (; kt < KT; ++kt) dstep(kt, std::integral_constant<bool, false>{});
    };
    switch (nb) {
      case 4: dual(std::integral_constant<int, 4>{}); break;
      case 3: dual(std::integral_constant<int, 3>{}); break;
      case 2: dual(std::integral_constant<int, 2>{}); break;
      case 1: dual(std::integral_constant<int, 1>{}); break;
      default: dual(std::integral_constant<int, 0>{}); break;
    }
  }

  big_epilogue<EPI>(p, smem, acc, expert, split, row0, rows, n0, wn, wm, r16, g, tid);
}

template <bool DUAL>
constexpr int big_lds_bytes() { return bg_stages<DUAL>() * bg_stage_bytes<DUAL>(); }

template <bool DUAL, int EPI>
static hipError_t big_attr() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_big_kernel<DUAL, EPI, true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, big_lds_bytes<DUAL>());
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_big_kernel<DUAL, EPI, false>),
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
  if (p.splits == 1) tiles = (tiles + 7) / 8 * 8;  // whole groups of 8 tiles
  const long long blocks = tiles * NQ * p.splits;
  if (blocks <= 0) return;
  const bool one = p.nseg == 1;
  if (p.a_lo)
    big_for_each_epi(p.epi, [&](auto E) {
      constexpr int EPI = decltype(E)::value;
      if (one)
        gemm_big_kernel<true, EPI, true><<<(unsigned)blocks, BG_THREADS, big_lds_bytes<true>(), s>>>(p);
      else
        gemm_big_kernel<true, EPI, false><<<(unsigned)blocks, BG_THREADS, big_lds_bytes<true>(), s>>>(p);
    });
  else
    big_for_each_epi(p.epi, [&](auto E) {
      constexpr int EPI = decltype(E)::value;
      if (one)
        gemm_big_kernel<false, EPI, true><<<(unsigned)blocks, BG_THREADS, big_lds_bytes<false>(), s>>>(p);
      else
        gemm_big_kernel<false, EPI, false><<<(unsigned)blocks, BG_THREADS, big_lds_bytes<false>(), s>>>(p);
    });
}

}  // namespace lmoe
