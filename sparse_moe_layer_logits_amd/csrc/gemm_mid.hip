// Grouped MFMA GEMM for block-scaled FP4 expert weights and tiles of up to 64
// activation rows (experts that see tens of tokens); NP activation parts: bf16
// (1; the one launched: FP4 experts take bf16 activations) or a bf16 hi + lo
// pair (2).
//
// Block: W waves (W = 8 from N = 1024 on, else 8, 7 or 4 as they divide N into
// 32-row wave slabs; waves past N stage activations and skip their products);
// wave w owns two 16-row MFMA tiles of weight rows (n0 + 32w ..)
// against the tile's activation rows in 16-row groups (a tile of r rows runs
// ceil(r/16) groups, no more).  The k loop runs in stages of 128.  Stage s is
// loaded into register set s % NS, NS - 1 stages ahead: the activation stage
// (64 rows x 128 k per part, shared by all W waves) and the stage's E4M3
// block scales go through one of two LDS slots; each wave keeps its FP4 codes
// (64 contiguous bytes per weight row and stage) in registers.  The block
// scales are read from a stage-major copy made at initialisation, so one
// stage's scales for the block are one contiguous range.  Every weight byte
// crosses HBM once and is decoded once.
//
// Block-scaled FP4 ("Nemotron 3 Super", section 3.6; E2M1 elements and E4M3
// block scales per "Nemotron 3 Ultra") is decoded in registers with the exact
// decoder of fp4.hpp; the per-matrix fp32 scale multiplies the accumulator in
// the epilogue.
//
// MFMA roles follow the other kernels: weight tile = MFMA A operand (rows =
// output columns n), activations = B operand.  k order inside a 128-wide stage:
// lane group g holds k = 32g .. 32g+31 (16 code bytes, two scale blocks) and
// MFMA step j (0..3) uses k = 32g + 8j .. +7 from every lane group.
#include "common.hpp"
#include "epilogue.hpp"
#include "fp4.hpp"
#include "kernels.hpp"

#include <type_traits>


namespace lmoe {

constexpr int MD_ROWS = 64;                 // activation rows per tile
// 16-row weight tiles per wave: two (32 weight rows) keep a wave at 126 VGPRs, so
// two 7- or 8-wave blocks share a CU; four (the earlier form, ~230 VGPRs, one block
// per CU) ran 7 % slower, the activations re-read by half as many blocks
constexpr int MD_NT = 2;
constexpr int MD_KS = 128;                  // k per stage
constexpr int MD_ROWB = MD_KS * 2;          // bytes of one activation row per stage and part
constexpr int MD_PARTB = MD_ROWS * MD_ROWB; // 16 KB
constexpr int MD_PIECES = MD_PARTB / 16;    // 16-byte pieces per part and stage

// activation byte offset in a slot: 16 pieces of 16 bytes per row, XOR-swizzled
__device__ __forceinline__ int md_off(int part, int row, int piece) {
  return part * MD_PARTB + row * MD_ROWB + ((piece ^ (row & 15)) << 4);
}

// wait for this wave's LDS operations (its stores) before a barrier; vector
// memory loads stay in flight
__device__ __forceinline__ void md_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// one thread's share of one stage: XP 16-byte pieces of each activation part,
// the 8 scale bytes of one weight row, 16 code bytes per weight tile
template <int XP, int NP>
struct MdStage {
  u32x4_t x[NP][XP];     // [part][piece]
  u32x2_t sc;            // E4M3 scales of weight row n0 + thread
  u32x4_t codes[MD_NT];  // 32 E2M1 codes per weight tile
};

template <int W, int EPI, int MT, int NP>
__device__ __forceinline__ void mid_body(const GemmParams& p, uint8_t* smem, int expert, int row0,
                                         int rows, int n0, int nbase, bool active) {
  constexpr int NTH = 64 * W;
  constexpr int BN = 16 * MD_NT * W;  // weight rows per block
  constexpr int XP = (MD_PIECES + NTH - 1) / NTH;
  // two register sets (loads run one stage ahead): a third does not fit next to the
  // activation pieces in the 128 VGPRs of two blocks per CU
  constexpr int NS = 2;
  // activation parts + scales: every thread stages one weight row's 8 scale bytes
  // (rows past the block's BN are never read)
  constexpr int SLOTB = NP * MD_PARTB + NTH * 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int K = p.seg[0].K;
  const int P = K / MD_KS;

  // ---- activations: piece id = i * NTH + tid -> row id / 16, piece id % 16
  // (ids past the stage are clamped for the load and not stored) ----
  uint32_t x_off[XP], x_lds[XP];
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int id = min(i * NTH + tid, MD_PIECES - 1);
    const int row = id >> 4, piece = id & 15;
    const int xr = min(row, rows - 1);
    const int src = p.row_index ? p.row_index[row0 + xr] : row0 + xr;
    x_off[i] = ((uint32_t)src * (uint32_t)p.lda + piece * 8) * 2u;  // bytes
    x_lds[i] = md_off(0, row, piece);
  }
  const uint8_t* Xhi = reinterpret_cast<const uint8_t*>(p.seg[0].A);
  const uint8_t* Xlo = reinterpret_cast<const uint8_t*>(p.a_lo);

  // ---- codes: uniform expert base + 32-bit per-lane offsets (row n, bytes 16g ..);
  // waves past the end read a valid slab they never use (p.N is a multiple of 64)
  const int wrow0 = min(nbase, p.N - 16 * MD_NT);
  const uint8_t* Wb = reinterpret_cast<const uint8_t*>(p.seg[0].B) + (size_t)expert * (size_t)(p.b_stride / 2);
  uint32_t w_off[MD_NT];
  uint32_t s_lds[MD_NT];  // this lane's two scale bytes in a slot's scale part
#pragma unroll
  for (int nt = 0; nt < MD_NT; ++nt) {
    const uint32_t n = wrow0 + nt * 16 + r16;
    w_off[nt] = n * (uint32_t)(p.ldb / 2) + 16u * g;
    s_lds[nt] = NP * MD_PARTB + (n - n0) * 8 + 2 * g;
  }
  // scales, stage-major [expert][stage][N][8]: thread tid moves row n0 + tid
  // (the last row below N past the end)
  const uint8_t* Sb = p.b_scale_sm + ((size_t)expert * P * p.N + min(n0 + tid, p.N - 1)) * 8;
  const size_t s_stage = (size_t)p.N * 8;

  auto issue = [&](MdStage<XP, NP>& st, int ps) {
    const uint8_t* xh = Xhi + ps * (MD_KS * 2);
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      st.x[0][i] = *reinterpret_cast<const u32x4_t*>(xh + x_off[i]);
      if constexpr (NP == 2)
        st.x[NP - 1][i] = *reinterpret_cast<const u32x4_t*>(Xlo + ps * (MD_KS * 2) + x_off[i]);
    }
    st.sc = *reinterpret_cast<const u32x2_t*>(Sb + ps * s_stage);
    const uint8_t* wb = Wb + ps * (MD_KS / 2);
#pragma unroll
    for (int nt = 0; nt < MD_NT; ++nt) st.codes[nt] = *reinterpret_cast<const u32x4_t*>(wb + w_off[nt]);
  };
  auto stash = [&](const MdStage<XP, NP>& st, int s) {
    uint8_t* slot = smem + (s & 1) * SLOTB;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      if (XP * NTH == MD_PIECES || i * NTH + tid < MD_PIECES) {
#pragma unroll
        for (int part = 0; part < NP; ++part)
          *reinterpret_cast<u32x4_t*>(slot + part * MD_PARTB + x_lds[i]) = st.x[part][i];
      }
    }
    *reinterpret_cast<u32x2_t*>(slot + NP * MD_PARTB + tid * 8) = st.sc;
  };

  f32x4_t acc[MD_NT][MT];
#pragma unroll
  for (int a = 0; a < MD_NT; ++a)
#pragma unroll
    for (int b = 0; b < MT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const MdStage<XP, NP>& st, int s) {
    const uint8_t* slot = smem + (s & 1) * SLOTB;
    float sc[MD_NT][2];
#pragma unroll
    for (int nt = 0; nt < MD_NT; ++nt) {
      const uint32_t two = *reinterpret_cast<const uint16_t*>(slot + s_lds[nt]);
      const f32x2_t v = fp8x2_to_f32<false>(two);
      sc[nt][0] = v.x;
      sc[nt][1] = v.y;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t xf[NP][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int part = 0; part < NP; ++part)
          xf[part][mt] = *reinterpret_cast<const u32x4_t*>(slot + md_off(part, mt * 16 + r16, 4 * g + j));
      u32x4_t wf[MD_NT];
#pragma unroll
      for (int nt = 0; nt < MD_NT; ++nt) wf[nt] = fp4x8_to_bf16(st.codes[nt][j], sc[nt][j >> 1]);
#pragma unroll
      for (int nt = 0; nt < MD_NT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int part = 0; part < NP; ++part)
            acc[nt][mt] = mfma_16x16x32(wf[nt], xf[part][mt], acc[nt][mt]);
        }
      }
    }
  };

  // Stage s lives in register set s % NS; at step s, set (s - 1) % NS (emptied
  // at step s - 1) is refilled with stage s + NS - 1 first, then stage s's
  // activations and scales go to LDS slot s % 2 (last read at step s - 2,
  // before the previous barrier), then stage s is multiplied.  Every step
  // issues the same loads (past the last stage it re-reads the last one), so
  // the compiler's in-order wait counts are exact on every path;
  // sched_barrier keeps each stage's loads together and in stage order.  The
  // trip count is padded to a multiple of NS (one loop exit; a padding step
  // only moves data) so the register sets stay static.
  MdStage<XP, NP> st[NS];
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) {
    issue(st[i], min(i, P - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  const int PN = (P + NS - 1) / NS * NS;
  for (int s0 = 0; s0 < PN; s0 += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = s0 + i;
      issue(st[(i + NS - 1) % NS], min(s + NS - 1, P - 1));
      __builtin_amdgcn_sched_barrier(0);
      stash(st[i], s);
      md_wait_lgkm0();
      asm volatile("s_barrier" ::: "memory");
      if (active && s < P) compute(st[i], s);
    }
  }

  if (!active) return;
  epi_tile<EPI>(p, expert, 0, row0, rows, MT, [&](int nt) { return nbase + nt * 16 + 4 * g; },
                [&](int mt) { return mt * 16 + r16; }, acc);
}

// two slots of the activation parts and one 8-byte scale row per thread (SLOTB)
template <int W, int NP>
constexpr int mid_lds_bytes() {
  return 2 * (NP * MD_PARTB + 64 * W * 8);
}

template <int W, int EPI, int NP>
// 7- and 8-wave blocks: two per CU (four waves per SIMD, 128 VGPRs); 4-wave blocks
// (narrow N) keep 256 VGPRs
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 4) void gemm_mid_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int BN = 16 * MD_NT * W;
  const int NQ = (p.N + BN - 1) / BN;
  const int b = blockIdx.x;
  if (b >= p.n_tiles[0] * NQ) return;
  const int j = b / NQ;
  const int q = b % NQ;
  const int expert = p.tile_expert[j];
  const int row0 = p.tile_row0[j];
  const int rows = p.tile_rows[j];
  const int n0 = q * BN;
  const int nbase = n0 + (threadIdx.x >> 6) * 16 * MD_NT;
  const bool active = nbase < p.N;  // wave-uniform; inactive waves still stage activations
  switch ((rows + 15) >> 4) {
    case 1: mid_body<W, EPI, 1, NP>(p, smem, expert, row0, rows, n0, nbase, active); break;
    case 2: mid_body<W, EPI, 2, NP>(p, smem, expert, row0, rows, n0, nbase, active); break;
    case 3: mid_body<W, EPI, 3, NP>(p, smem, expert, row0, rows, n0, nbase, active); break;
    default: mid_body<W, EPI, 4, NP>(p, smem, expert, row0, rows, n0, nbase, active); break;
  }
}

template <int W, int EPI, int NP>
static void mid_launch(const GemmParams& p, hipStream_t s) {
  const long long blocks = (long long)p.max_tiles * ((p.N + 16 * MD_NT * W - 1) / (16 * MD_NT * W));
  if (blocks <= 0) return;
  gemm_mid_kernel<W, EPI, NP><<<(unsigned)blocks, 64 * W, mid_lds_bytes<W, NP>(), s>>>(p);
}

// waves per block: 8 from N = 1024 on (the idle waves of a partial last block cost
// less than the activation re-reads of more, narrower blocks: m = 2688 in 11 8-wave
// blocks ran expert up at 0.244 ms against 0.260 in 12 7-wave blocks), else the
// largest of 8, 7 that splits N into whole blocks, else 4
static int mid_waves(int N) { return N >= 1024 || N % 256 == 0 ? 8 : N % 224 == 0 ? 7 : 4; }

template <int EPI, int NP>
static void mid_launch_w(const GemmParams& p, hipStream_t s) {
  switch (mid_waves(p.N)) {
    case 8: mid_launch<8, EPI, NP>(p, s); break;
    case 7: mid_launch<7, EPI, NP>(p, s); break;
    default: mid_launch<4, EPI, NP>(p, s); break;
  }
}

// epilogues offered (FP4 experts take bf16 activations and give bf16 outputs):
// relu^2 to bf16 (expert up) and the gated rows as bf16 (expert down)
bool gemm_mid_supports(const GemmParams& p, bool fp4) {
  const bool epi_ok = !p.a_lo && (p.epi == EPI_SQRELU_BF16 || p.epi == EPI_GATE_BF16);
  return fp4 && p.tile_expert && p.rows_per_tile <= MD_ROWS && p.nseg == 1 && epi_ok &&
         p.b_scale_sm && p.N % 64 == 0 && p.seg[0].K % MD_KS == 0 && p.seg[0].K >= MD_KS;
}

template <int W, int EPI, int NP>
static hipError_t mid_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mid_kernel<W, EPI, NP>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, mid_lds_bytes<W, NP>());
}

template <int W>
static hipError_t mid_attr_w() {
  hipError_t e = mid_attr<W, EPI_SQRELU_BF16, 1>();
  if (e == hipSuccess) e = mid_attr<W, EPI_GATE_BF16, 1>();
  return e;
}

int gemm_mid_setup() {
  hipError_t e = mid_attr_w<8>();
  if (e == hipSuccess) e = mid_attr_w<7>();
  if (e == hipSuccess) e = mid_attr_w<4>();
  return (int)e;
}

void launch_gemm_mid(const GemmParams& p, bool fp4, hipStream_t s) {
  (void)fp4;
  if (p.epi == EPI_SQRELU_BF16)
    mid_launch_w<EPI_SQRELU_BF16, 1>(p, s);
  else
    mid_launch_w<EPI_GATE_BF16, 1>(p, s);
}

// [E][N][K/16] -> [E][K/128][N][8]: one thread per 8-byte group
__global__ void scale_stage_major_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                         long long groups, int N, int P) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // (e, n, s) row-major
  if (i >= groups) return;
  const int s = (int)(i % P);
  const long long en = i / P;
  const int n = (int)(en % N);
  const long long e = en / N;
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(src + 8 * i);
  *reinterpret_cast<u32x2_t*>(dst + (((e * P + s) * N) + n) * 8) = v;
}

void launch_scale_stage_major(const uint8_t* src, uint8_t* dst, long long E, int N, int K,
                              hipStream_t s) {
  const int P = K / MD_KS;
  const long long groups = E * N * P;
  if (groups <= 0) return;
  scale_stage_major_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(src, dst, groups, N, P);
}

}  // namespace lmoe
