// Host orchestration and C ABI of the LatentMoE layer forward.
//
// Step order per forward call ("Nemotron 3 Super", section 3.2; the gating
// network and the shared expert stay at width d, routing and expert compute
// happen in the latent width l):
//   router logits (x, width d)  -> top-K + softmax -> bucketing (counts,
//   offsets, permutation) -> z = W_down x -> grouped expert up (squared ReLU)
//   -> grouped expert down (times gate) -> combine in k order -> shared expert
//   (y = S2 relu(S1 x)^2) -> y += W_up y_lat.
// Everything is enqueued on the caller's stream; the forward allocates nothing
// and never waits on the host.
//
// Precision: products run on bf16 MFMA with fp32 accumulation.  Activations
// that feed a later product (z, the expert hidden h, the latent sum and the
// shared hidden) leave their producer as a bf16 pair (hi, lo = v - hi), and the
// consumer multiplies both parts with each weight fragment, so they carry about
// 16 significant bits; the weights are read once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/latentmoe.h"
#include "kernels.hpp"

using namespace lmoe;

namespace {

constexpr int STREAM_ROWS_BIG = 64;
constexpr int STREAM_ROWS_SMALL = 16;  // decode expert tiles
constexpr int STREAM_ROWS_MID = 32;
constexpr double ROWS16_MAX_AVG = 12.0;  // up to this many rows per expert on average: 16-row tiles
constexpr double ROWS32_MAX_AVG = 24.0;  // then up to this many: 32-row tiles, above: 64
constexpr int TILE_ROWS = 256;           // rows per tile of the large-tile kernel
// Large-tile path (prefill): a token's routed rows with the largest gates carry
// their activations (z, h, the gated output) as bf16 hi + lo pairs, the others as
// bf16 -- as many rows as it takes for the rows left as bf16 to hold at most
// PAIR_TAIL_FRAC of the token's gate energy sum_k g_k^2.  A row's bf16 rounding
// reaches the latent sum scaled by its gate; an fp64 emulation of the rounding
// points keeps the latent sum within 4e-3 of its rms with flat gates (K = 8 of
// 32, 22 of 512, 40 of 1024: 90-93 % of rows paired) and with skewed ones (one
// gate near 1: only that row paired), where a fixed gate threshold of 0.1
// reached 1.6-1.8e-2 with flat gates.
constexpr float PAIR_TAIL_FRAC = 1.0f / 32.0f;
// Activations of GEMMs whose weights are stored in FP4 or FP8 are single bf16
// values: weight-only quantisation with 16-bit activations, the W4A16 mode in
// which Hopper GPUs serve the NVFP4 checkpoint ("Nemotron 3.5 Super and
// Lightning", limitations; "Nemotron 3 Ultra", contributions).  bf16 weights keep
// the hi + lo pairs.  The bf16 rounding of an activation (2^-9 relative) is far
// below the weight formats' own step.
// smallest k range of a split for large-tile GEMMs with four or more row tiles
constexpr int BIG_KGRAN = 512;
constexpr int BUCKET_MIN_CHUNKS = 4;  // chunks of 16 mask blocks (256 tokens) from which the count is split
constexpr int TARGET_BLOCKS = 256;      // streaming kernel: 8-wave blocks, several per CU
// the two stacked GEMMs of the decode-sized path (one block per CU at 256 blocks: the
// blocks' load latency left HBM idle; 512 put two on each CU, -9 us per forward)
constexpr int TARGET_BLOCKS_STACKED = 512;
// mid-sized batches (65 .. STACK_X_ROWS tokens) with the stacked weights run the
// three GEMMs over x as one large-tile launch and one reduce (their own launches
// there are short split-K runs of a few row tiles, each with its own reduce)
constexpr int STACK_X_ROWS = 1024;
// the decode-sized up-projection alone (the shared expert's S2 ran with expert down)
constexpr int TARGET_BLOCKS_UP = 256;
constexpr int TARGET_BLOCKS_BIG = 256;  // large-tile kernel: one 8-wave block per CU

struct Plan {
  bool stream;  // weight-streaming kernel (true) or LDS-tiled kernel
  int splits;
  int k_split;
};

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// split-K plan for a dense GEMM of M rows, N columns, K reduction (target: blocks the
// streaming kernel aims at)
Plan plan_dense(int M, int N, int K, int target = TARGET_BLOCKS) {
  Plan p;
  p.stream = M <= STREAM_ROWS_BIG;
  const int per_split = p.stream ? ceil_div(N, 128) * ceil_div(M, STREAM_ROWS_BIG)
                                 : ceil_div(N, 256) * ceil_div(M, TILE_ROWS);
  // smallest k range of a split: with four or more row tiles the large-tile GEMMs
  // have blocks enough, and halving their splits halves the partial sums' traffic
  const int gran = !p.stream && M >= 4 * TILE_ROWS ? BIG_KGRAN : 256;
  int want = std::max(1, ceil_div(p.stream ? target : TARGET_BLOCKS_BIG, per_split));
  want = std::min(want, std::max(1, K / gran));
  int ks = ceil_div(ceil_div(K, want), gran) * gran;
  if (!p.stream) {
    // one block per CU: a last wave of blocks less than half full costs a whole block
    // time for a few blocks; fewer, longer splits that fill the whole waves instead
    // (S1 at 1024 tokens: 336 blocks -> 252, 87 -> 73 us; Ultra S1 94 -> 78 us)
    const int blocks = per_split * ceil_div(K, ks);
    const int full = blocks / TARGET_BLOCKS_BIG, rest = blocks % TARGET_BLOCKS_BIG;
    if (full > 0 && rest > 0 && 2 * rest < TARGET_BLOCKS_BIG) {
      const int fit = std::max(1, full * TARGET_BLOCKS_BIG / per_split);
      const int ks2 = ceil_div(ceil_div(K, fit), gran) * gran;
      if ((long long)per_split * ceil_div(K, ks2) <= (long long)full * TARGET_BLOCKS_BIG) ks = ks2;
    }
  }
  p.k_split = ks;
  p.splits = ceil_div(K, ks);
  return p;
}

struct Buffers {
  uint16_t* pieces = nullptr;
  float* logits = nullptr;
  float* partial = nullptr;
  float* partial2 = nullptr;  // split-K partials of the shared expert (side stream)
  float* partial3 = nullptr;  // split-K partials of W_down (side stream 2, without stacked copies)
  size_t partial_cap = 0;  // floats
  int* idx = nullptr;
  float* gates = nullptr;
  uint32_t* masks = nullptr;
  uint32_t* masks_hi = nullptr;  // rows carried as hi + lo pairs (large-tile path)
  uint8_t* paired = nullptr;     // [T*K]: 1 for those rows, 0 for the bf16 class
  int* block_prefix = nullptr;   // per (block, expert) prefix of the (hi-class) rows
  int* prefix_lo = nullptr;      // the same for the other rows
  int* chunk_hi = nullptr;       // per (chunk of mask blocks, expert) counts -> offsets (large T)
  int* chunk_lo = nullptr;
  int* counts_hi = nullptr;
  int* counts = nullptr;
  int* offsets = nullptr;
  int* tile_expert = nullptr;
  int* tile_row0 = nullptr;
  int* tile_rows = nullptr;
  int* n_tiles = nullptr;
  int max_tiles_cap = 0;
  int* row_src = nullptr;
  float* row_gate = nullptr;
  int* inv = nullptr;
  uint16_t* z = nullptr;
  uint16_t* z_lo = nullptr;
  uint16_t* h = nullptr;
  uint16_t* h_lo = nullptr;
  float* og = nullptr;
  uint16_t* og16 = nullptr;  // bf16-class expert-down rows (large-tile path, two row classes)
  uint16_t* y_lat = nullptr;
  uint16_t* y_lat_lo = nullptr;
  uint16_t* hs_hi = nullptr;
  uint16_t* hs_lo = nullptr;
  uint8_t* w1_scale_sm = nullptr;  // FP4: expert block scales in the mid kernel's stage-major order
  uint8_t* w2_scale_sm = nullptr;
  // exact bf16 values of FP4 / FP8 dense weights for the LDS-tiled kernel (T > 64)
  uint16_t* s1_bf16 = nullptr;
  uint16_t* s2_bf16 = nullptr;
  uint16_t* wd_bf16 = nullptr;
  uint16_t* wu_bf16 = nullptr;
  // decode-sized forwards with bf16 projections and shared expert (see `linear` below):
  uint16_t* wx = nullptr;     // stacked rows [router pieces 1-3; W_down; S1], [3N + l + m_s, d]
  uint16_t* wy = nullptr;     // [W_up | S2], [d, l + m_s]
  uint16_t* ay = nullptr;     // [min(T, 64), l + m_s]: y_lat then h_s, bf16 high parts
  uint16_t* ay_lo = nullptr;  // the remainders
};

struct Layout {
  size_t total = 0;
  std::vector<std::pair<void**, size_t>> items;
  void add(void** p, size_t bytes) {
    items.emplace_back(p, bytes);
    total += (bytes + 255) & ~size_t(255);
  }
};

int check_config(const latentmoe_config* c) {
  if (!c) return LATENTMOE_ERR_INVALID_ARG;
  if (c->d <= 0 || c->latent <= 0 || c->n_experts <= 0 || c->top_k <= 0 ||
      c->expert_hidden <= 0 || c->shared_hidden <= 0 || c->max_tokens <= 0)
    return LATENTMOE_ERR_INVALID_ARG;
  if (c->expert_format != LATENTMOE_FORMAT_BF16 &&
      c->expert_format != LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16)
    return LATENTMOE_ERR_UNSUPPORTED;
  if (c->shared_format != LATENTMOE_FORMAT_BF16 &&
      c->shared_format != LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16)
    return LATENTMOE_ERR_UNSUPPORTED;
  if (c->proj_format != LATENTMOE_FORMAT_BF16 && c->proj_format != LATENTMOE_FORMAT_FP8_E4M3)
    return LATENTMOE_ERR_UNSUPPORTED;
  // the FP4 block (16 elements along the input width) and the kernels' 16-row tiles;
  // widths that are not multiples of 64 run zero-padded to the next one
  if (c->d % 16 || c->latent % 16 || c->expert_hidden % 16 || c->shared_hidden % 16)
    return LATENTMOE_ERR_UNSUPPORTED;
  if (c->n_experts % 16 || c->n_experts > 4096) return LATENTMOE_ERR_UNSUPPORTED;
  if (c->top_k > c->n_experts || c->top_k > 64) return LATENTMOE_ERR_UNSUPPORTED;
  // the large-tile and FP4 kernels address activation rows with 32-bit byte offsets
  // (bf16 elements): h [T K, m], the gathered z [T, l], x [T, d], h_s [T, m_s] (at
  // the widths the kernels run: rounded up to multiples of 64)
  const long long lim = 1ll << 31;
  auto r64 = [](int v) { return (long long)(v + 63) / 64 * 64; };
  if ((long long)c->max_tokens * c->top_k * std::max(r64(c->latent), r64(c->expert_hidden)) >= lim ||
      (long long)c->max_tokens * std::max(r64(c->d), r64(c->shared_hidden)) >= lim)
    return LATENTMOE_ERR_UNSUPPORTED;
  return LATENTMOE_OK;
}

size_t max_partial_floats(const latentmoe_config& c, bool linear) {
  // every T a forward may see: the plans only change with the tile counts
  std::vector<int> Ts;
  for (int t = 1; t <= std::min(c.max_tokens, STREAM_ROWS_BIG); t = t < 16 ? t + 1 : t + 16) Ts.push_back(t);
  Ts.push_back(std::min(c.max_tokens, STREAM_ROWS_BIG));
  for (long long t = STREAM_ROWS_BIG + 1; t <= c.max_tokens; t += TILE_ROWS) Ts.push_back((int)t);
  for (long long t = TILE_ROWS; t <= c.max_tokens; t += TILE_ROWS) Ts.push_back((int)t);
  Ts.push_back(c.max_tokens);
  size_t best = 0;
  for (int T : Ts) {
    if (T < 1 || T > c.max_tokens) continue;
    struct G { int N, K; bool always; };
    const G gs[] = {{c.n_experts, 3 * c.d, false}, {c.latent, c.d, false},
                    {c.shared_hidden, c.d, false}, {c.d, c.shared_hidden, false},
                    {c.d, c.latent, false}};
    for (const G& g : gs) {
      Plan p = plan_dense(T, g.N, g.K);
      if (p.splits > 1 || g.always) best = std::max(best, (size_t)p.splits * T * g.N);
    }
    if (linear && T > STREAM_ROWS_BIG) {  // the stacked GEMM over x
      const int NX = 3 * c.n_experts + c.latent + (T <= STACK_X_ROWS ? c.shared_hidden : 0);
      best = std::max(best, (size_t)plan_dense(T, NX, c.d).splits * T * NX);
    }
    if (linear && T <= STREAM_ROWS_BIG) {  // the stacked GEMMs always leave partials
      const G lg[] = {{3 * c.n_experts + c.latent + c.shared_hidden, c.d, true},
                      {3 * c.n_experts + c.latent, c.d, true},
                      {c.d, c.latent + c.shared_hidden, true}};
      for (const G& g : lg)
        best = std::max(best, (size_t)plan_dense(T, g.N, g.K, TARGET_BLOCKS_STACKED).splits * T * g.N);
      best = std::max(best, (size_t)plan_dense(T, c.d, c.latent, TARGET_BLOCKS_UP).splits * T * c.d);
    }
  }
  return best;
}

// Decode-sized forwards (T <= 64) with bf16 projections and shared expert run on
// one stream with no events: every GEMM over x is one launch over the stacked
// rows [router pieces; W_down; S1] (one reduce splits logits, z and h_s), and
// y = W_up y_lat + S2 h_s is one dual GEMM over [W_up | S2] with y_lat and h_s side
// by side in one row.  On a multi-queue graph replay every cross-queue edge left
// the waiting queue idle for 6-12 us; this path has none.  With bf16 experts on the
// streaming kernel, S1 and S2 instead run inside the expert-up and expert-down
// launches, and the second stacked GEMM keeps W_up only (it adds onto the y S2 wrote).
bool linear_formats(const latentmoe_config& c) {
  return c.shared_format == LATENTMOE_FORMAT_BF16 && c.proj_format == LATENTMOE_FORMAT_BF16;
}

// ---- widths that are multiples of 16 but not of 64 ----
// The kernels take d, l, m, m_s in multiples of 64.  Other widths run at the widths
// rounded up to 64: init copies every weight into zero-padded matrices (the padded
// rows and columns add exact zeros to every product, so z, h, h_s, y_lat and the
// logits keep their values and the padded columns of each activation are zero);
// each forward copies x into a zero-padded [T, D] buffer and crops y out of a
// [T, D] one.
int round64(int v) { return (v + 63) / 64 * 64; }

bool needs_pad(const latentmoe_config& c) {
  return c.d % 64 || c.latent % 64 || c.expert_hidden % 64 || c.shared_hidden % 64;
}

latentmoe_config padded_config(const latentmoe_config& c) {
  latentmoe_config p = c;
  p.d = round64(c.d);
  p.latent = round64(c.latent);
  p.expert_hidden = round64(c.expert_hidden);
  p.shared_hidden = round64(c.shared_hidden);
  return p;
}

// One allocation: every weight matrix at the padded widths, then x_pad [max_tokens, D]
// bf16 and y_pad [max_tokens, D] fp32.  A matrix is `slices` slices of rows x cols
// elements of num/den bytes (FP4 codes 1/2, block scales 1/16) padded to prows x pcols.
struct PadPlan {
  struct Item {
    const void* src;
    size_t field;  // offset of the matrix's pointer in latentmoe_weights
    long long slices;
    int rows, prows;
    size_t row_bytes, prow_bytes;
  };
  std::vector<Item> items;
  size_t total = 0;
  size_t x_off = 0, y_off = 0;
  latentmoe_weights w{};  // the padded matrices (pointers set by place_pad_plan)

  void add(const void* src, size_t field, long long slices, int rows, int cols, int prows, int pcols,
           int num, int den) {
    Item it{src, field, slices, rows, prows, (size_t)cols * num / den, (size_t)pcols * num / den};
    items.push_back(it);
    total += (slices * (size_t)prows * it.prow_bytes + 255) & ~size_t(255);
  }
};

// the padded copies of cfg's weights (w may be null: sizes only)
PadPlan make_pad_plan(const latentmoe_config& c, const latentmoe_weights* w) {
  static const latentmoe_weights none{};
  const latentmoe_weights& s = w ? *w : none;
  const latentmoe_config p = padded_config(c);
  PadPlan P;
  P.w = s;
  const int N = c.n_experts;
  const int d = c.d, l = c.latent, m = c.expert_hidden, ms = c.shared_hidden;
  const int D = p.d, L = p.latent, M = p.expert_hidden, MS = p.shared_hidden;
  const bool fp4 = c.expert_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16;
  const bool sfp4 = c.shared_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16;
  const int pe = c.proj_format == LATENTMOE_FORMAT_FP8_E4M3 ? 1 : 2;  // projection bytes per element
#define LMOE_F(name) offsetof(latentmoe_weights, name)
  P.add(s.router_w, LMOE_F(router_w), 1, N, d, N, D, 4, 1);
  P.add(s.w_down, LMOE_F(w_down), 1, l, d, L, D, pe, 1);
  P.add(s.w_up, LMOE_F(w_up), 1, d, l, D, L, pe, 1);
  if (fp4) {  // codes (two per byte) and block scales (one per 16 input elements)
    P.add(s.expert_w1, LMOE_F(expert_w1), N, m, l, M, L, 1, 2);
    P.add(s.expert_w2, LMOE_F(expert_w2), N, l, m, L, M, 1, 2);
    P.add(s.expert_w1_scale, LMOE_F(expert_w1_scale), N, m, l, M, L, 1, 16);
    P.add(s.expert_w2_scale, LMOE_F(expert_w2_scale), N, l, m, L, M, 1, 16);
  } else {
    P.add(s.expert_w1, LMOE_F(expert_w1), N, m, l, M, L, 2, 1);
    P.add(s.expert_w2, LMOE_F(expert_w2), N, l, m, L, M, 2, 1);
  }
  if (sfp4) {
    P.add(s.shared_w1, LMOE_F(shared_w1), 1, ms, d, MS, D, 1, 2);
    P.add(s.shared_w2, LMOE_F(shared_w2), 1, d, ms, D, MS, 1, 2);
    P.add(s.shared_w1_scale, LMOE_F(shared_w1_scale), 1, ms, d, MS, D, 1, 16);
    P.add(s.shared_w2_scale, LMOE_F(shared_w2_scale), 1, d, ms, D, MS, 1, 16);
  } else {
    P.add(s.shared_w1, LMOE_F(shared_w1), 1, ms, d, MS, D, 2, 1);
    P.add(s.shared_w2, LMOE_F(shared_w2), 1, d, ms, D, MS, 2, 1);
  }
#undef LMOE_F
  P.x_off = P.total;
  P.total += ((size_t)c.max_tokens * p.d * 2 + 255) & ~size_t(255);
  P.y_off = P.total;
  P.total += ((size_t)c.max_tokens * p.d * 4 + 255) & ~size_t(255);
  return P;
}

// points the plan's matrices into buf and enqueues the padded copies on s
void place_pad_plan(PadPlan& P, char* buf, hipStream_t s) {
  size_t at = 0;
  for (const PadPlan::Item& it : P.items) {
    const void* q = buf + at;
    std::memcpy(reinterpret_cast<char*>(&P.w) + it.field, &q, sizeof(q));
    launch_pad_copy(it.src, it.row_bytes, it.rows, buf + at, it.prow_bytes, it.prows, it.slices, it.rows,
                    it.row_bytes, s);
    at += (it.slices * (size_t)it.prows * it.prow_bytes + 255) & ~size_t(255);
  }
}

// linear: lay out the stacked weights and rows of the decode-sized single-stream forward
Layout make_layout(const latentmoe_config& c, Buffers& b, bool linear) {
  Layout L;
  const size_t Tm = c.max_tokens, N = c.n_experts, K = c.top_k;
  const size_t TK = Tm * K;
  const size_t nblk = (Tm + 15) / 16;
  b.partial_cap = max_partial_floats(c, linear);
  // every expert may end in one partial tile per row class
  b.max_tiles_cap = (int)(ceil_div(TK, STREAM_ROWS_SMALL) + 2 * std::min(N, TK));
  if (linear) {  // the router pieces are the first 3N rows of the stacked x weights
    L.add((void**)&b.wx, (3 * N + c.latent + c.shared_hidden) * (size_t)c.d * 2);
    L.add((void**)&b.wy, (size_t)c.d * (c.latent + c.shared_hidden) * 2);
    const size_t Tl = std::min<size_t>(Tm, STREAM_ROWS_BIG);
    L.add((void**)&b.ay, Tl * (c.latent + c.shared_hidden) * 2);
    L.add((void**)&b.ay_lo, Tl * (c.latent + c.shared_hidden) * 2);
  } else {
    L.add((void**)&b.pieces, 3 * N * c.d * 2);
  }
  L.add((void**)&b.logits, Tm * N * 4);
  L.add((void**)&b.partial, b.partial_cap * 4);
  L.add((void**)&b.partial2, b.partial_cap * 4);
  L.add((void**)&b.partial3, b.partial_cap * 4);
  L.add((void**)&b.idx, TK * 4);
  L.add((void**)&b.gates, TK * 4);
  L.add((void**)&b.masks, nblk * N * 4);
  L.add((void**)&b.masks_hi, nblk * N * 4);
  L.add((void**)&b.block_prefix, nblk * N * 4);
  L.add((void**)&b.prefix_lo, nblk * N * 4);
  L.add((void**)&b.chunk_hi, (size_t)bucket_chunks((int)Tm) * N * 4);
  L.add((void**)&b.chunk_lo, (size_t)bucket_chunks((int)Tm) * N * 4);
  L.add((void**)&b.counts_hi, N * 4);
  L.add((void**)&b.counts, N * 4);
  L.add((void**)&b.offsets, (N + 1) * 4);
  L.add((void**)&b.tile_expert, (size_t)b.max_tiles_cap * 4);
  L.add((void**)&b.tile_row0, (size_t)b.max_tiles_cap * 4);
  L.add((void**)&b.tile_rows, (size_t)b.max_tiles_cap * 4);
  L.add((void**)&b.n_tiles, 2 * 4);
  L.add((void**)&b.row_src, TK * 4);
  L.add((void**)&b.row_gate, TK * 4);
  L.add((void**)&b.inv, TK * 4);
  L.add((void**)&b.paired, TK);
  L.add((void**)&b.z, Tm * c.latent * 2);
  L.add((void**)&b.z_lo, Tm * c.latent * 2);
  L.add((void**)&b.h, TK * c.expert_hidden * 2);
  L.add((void**)&b.h_lo, TK * c.expert_hidden * 2);
  L.add((void**)&b.og, TK * c.latent * 4);
  L.add((void**)&b.og16, TK * c.latent * 2 + 16);  // + the combine's 16-byte reads past the last row
  L.add((void**)&b.y_lat, Tm * c.latent * 2);
  L.add((void**)&b.y_lat_lo, Tm * c.latent * 2);
  L.add((void**)&b.hs_hi, Tm * c.shared_hidden * 2);
  L.add((void**)&b.hs_lo, Tm * c.shared_hidden * 2);
  if (c.expert_format == LATENTMOE_EXPERTS_FP4_E2M1_E4M3_B16) {  // the mid kernel's K is a multiple of 128
    const size_t sc_bytes = N * (size_t)c.expert_hidden * (c.latent / 16);  // either matrix
    if (c.latent % 128 == 0) L.add((void**)&b.w1_scale_sm, sc_bytes);
    if (c.expert_hidden % 128 == 0) L.add((void**)&b.w2_scale_sm, sc_bytes);
  }
  if (c.max_tokens > STREAM_ROWS_BIG) {  // some dense GEMMs run on the LDS-tiled kernel
    if (c.shared_format != LATENTMOE_FORMAT_BF16) {
      L.add((void**)&b.s1_bf16, (size_t)c.shared_hidden * c.d * 2);
      L.add((void**)&b.s2_bf16, (size_t)c.d * c.shared_hidden * 2);
    }
    if (c.proj_format != LATENTMOE_FORMAT_BF16) {
      L.add((void**)&b.wd_bf16, (size_t)c.latent * c.d * 2);
      L.add((void**)&b.wu_bf16, (size_t)c.d * c.latent * 2);
    }
  }
  return L;
}

}  // namespace

struct GraphKey {
  const void* x;
  int T;
  const void* y;
  const void* idx;
  const void* gate;
  bool operator==(const GraphKey& o) const {
    return x == o.x && T == o.T && y == o.y && idx == o.idx && gate == o.gate;
  }
};

struct latentmoe_handle_s {
  latentmoe_config cfg;  // the widths the kernels run (rounded up to multiples of 64)
  latentmoe_weights w;
  latentmoe_config ucfg;  // the caller's widths
  // widths that are not multiples of 64: the padded weights, x_pad and y_pad
  void* pad_buf = nullptr;
  uint16_t* x_pad = nullptr;
  float* y_pad = nullptr;
  Buffers b;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  int last_T = 0;
  // LATENTMOE_SERIAL=1 in the environment at init: every kernel on the caller's
  // stream in program order (no side streams), so a kernel trace shows each
  // kernel's own duration
  bool serial = false;
  bool linear = false;       // stacked weights present: decode-sized forwards run on one stream
  bool last_linear = false;  // the last forward took that path (y_lat, h_s in the stacked rows)
  // the shared expert runs on a side stream forked from the caller's stream
  hipStream_t side = nullptr;
  hipStream_t side2 = nullptr;  // W_down without stacked copies; the paired rows' expert down
  hipEvent_t ev_fork = nullptr, ev_fork2 = nullptr, ev_join = nullptr, ev_join2 = nullptr;
  hipEvent_t ev_hi = nullptr, ev_hi_done = nullptr;  // the hi class's expert down beside the bf16 class
  // graph replay of the whole forward (latentmoe_forward_graph)
  hipStream_t cap = nullptr;  // capture stream
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  GraphKey gkey{};
  uint32_t prof_mask = 0;
  // stage timing
  std::vector<hipEvent_t> events;
  int prof_max = 0;
  int prof_calls = 0;
  bool profiling = false;
};

namespace {

void drop_graph(latentmoe_handle_s* h);

struct StageTimer {
  latentmoe_handle_s* h;
  hipStream_t s;
  bool on;
  StageTimer(latentmoe_handle_s* h_, hipStream_t s_)
      : h(h_), s(s_), on(h_->profiling && h_->prof_calls < h_->prof_max) {}
  bool want(int stage) const { return on && ((h->prof_mask >> stage) & 1u); }
  hipEvent_t event(int stage, int end) const {
    return h->events[((size_t)h->prof_calls * LATENTMOE_NUM_STAGES + stage) * 2 + end];
  }
  void start(int stage, hipStream_t st = nullptr) {
    if (want(stage)) (void)hipEventRecord(event(stage, 0), st ? st : s);
  }
  void stop(int stage, hipStream_t st = nullptr) {
    if (want(stage)) (void)hipEventRecord(event(stage, 1), st ? st : s);
  }
  void done() {
    if (on) h->prof_calls++;
  }
};

GemmParams base_params() {
  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.splits = 1;
  return p;
}

// dense GEMM C[T, N] = sum_seg A_seg[T, K_seg] B_seg[N, K_seg]^T with a final epilogue;
// returns the number of k splits (with force_partial the caller reduces them).  fmt is
// seg[0].B's stored format; the LDS-tiled kernel reads bf16_B (its exact bf16 values)
// instead when fmt is not bf16.
int run_dense(latentmoe_handle_s* h, GemmParams p, int T, hipStream_t s, bool force_partial,
              float* partial = nullptr, int fmt = WF_BF16, const uint16_t* bf16_B = nullptr,
              int target = TARGET_BLOCKS) {
  int Ktot = 0;
  for (int i = 0; i < p.nseg; ++i) Ktot += p.seg[i].K;
  Plan pl = plan_dense(T, p.N, Ktot, target);
  // keep within the partial buffer (it is sized for every T at init)
  while (pl.splits > 1 && (size_t)pl.splits * T * p.N > h->b.partial_cap) {
    pl.k_split *= 2;
    pl.splits = ceil_div(Ktot, pl.k_split);
  }
  p.M = T;
  p.k_split = pl.k_split;
  p.splits = pl.splits;
  const int final_epi = p.epi;
  const bool use_partial = force_partial || pl.splits > 1;
  if (use_partial) {
    p.epi = EPI_PARTIAL;
    p.partial = partial ? partial : h->b.partial;
    p.partial_stride = (long long)T * p.N;
  }
  if (pl.stream) {
    launch_gemm_stream(p, fmt, s);
  } else {
    if (fmt != WF_BF16) {
      p.seg[0].B = bf16_B;
      p.b_scale = nullptr;
    }
    launch_gemm_big(p, s);
  }
  if (use_partial && !force_partial) {
    GemmParams r = p;
    r.epi = final_epi;
    launch_reduce(r, s);
  }
  return pl.splits;
}

}  // namespace

extern "C" {

const char* latentmoe_status_string(int status) {
  switch (status) {
    case LATENTMOE_OK: return "ok";
    case LATENTMOE_ERR_INVALID_ARG: return "invalid argument";
    case LATENTMOE_ERR_UNSUPPORTED: return "unsupported shape or format";
    case LATENTMOE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LATENTMOE_ERR_HIP: return "HIP runtime error";
    case LATENTMOE_ERR_SCRATCH: return "workspace exceeds the static scratch array";
    default: return "unknown status";
  }
}

int latentmoe_workspace_bytes(const latentmoe_config* cfg, size_t* bytes) {
  int st = check_config(cfg);
  if (st != LATENTMOE_OK) return st;
  if (!bytes) return LATENTMOE_ERR_INVALID_ARG;
  Buffers b;
  if (needs_pad(*cfg)) {
    const latentmoe_config p = padded_config(*cfg);
    *bytes = make_layout(p, b, linear_formats(p)).total + make_pad_plan(*cfg, nullptr).total;
  } else {
    *bytes = make_layout(*cfg, b, linear_formats(*cfg)).total;
  }
  return LATENTMOE_OK;
}

}  // extern "C"

namespace {

// the handle for widths that are multiples of 64 (cfg and w are what the kernels run)
int init_handle(const latentmoe_config* cfg, const latentmoe_weights* w, hipStream_t stream,
                latentmoe_handle_t* out) {
  int st = LATENTMOE_OK;
  if (!w || !w->router_w || !w->w_down || !w->w_up || !w->expert_w1 || !w->expert_w2 ||
      !w->shared_w1 || !w->shared_w2)
    return LATENTMOE_ERR_INVALID_ARG;
  const bool fp4 = cfg->expert_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16;
  if (fp4 && (!w->expert_w1_scale || !w->expert_w2_scale || !w->expert_w1_tscale ||
              !w->expert_w2_tscale))
    return LATENTMOE_ERR_INVALID_ARG;
  const bool shared_fp4 = cfg->shared_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16;
  if (shared_fp4 && (!w->shared_w1_scale || !w->shared_w2_scale || !w->shared_w1_tscale ||
                     !w->shared_w2_tscale))
    return LATENTMOE_ERR_INVALID_ARG;
  const bool proj_fp8 = cfg->proj_format == LATENTMOE_FORMAT_FP8_E4M3;
  if (proj_fp8 && (!w->w_down_tscale || !w->w_up_tscale)) return LATENTMOE_ERR_INVALID_ARG;

  latentmoe_handle_s* h = new (std::nothrow) latentmoe_handle_s();
  if (!h) return LATENTMOE_ERR_OUT_OF_MEMORY;
  h->cfg = *cfg;
  h->w = *w;
  {
    const char* ser = std::getenv("LATENTMOE_SERIAL");
    h->serial = ser && ser[0] == '1';
  }
  h->linear = linear_formats(*cfg);
  Layout L = make_layout(*cfg, h->b, h->linear);
  // LATENTMOE_FAIL_ALLOC=1 in the environment makes the workspace allocation fail
  // (tests of the out-of-memory path)
  const char* fail = std::getenv("LATENTMOE_FAIL_ALLOC");
  const bool force_fail = fail && fail[0] == '1';
  if (force_fail || hipMalloc(&h->workspace, L.total) != hipSuccess) {
    h->workspace = nullptr;
    (void)hipGetLastError();
    delete h;
    return LATENTMOE_ERR_OUT_OF_MEMORY;
  }
  h->workspace_bytes = L.total;
  if (gemm_big_setup() != 0 ||
      (cfg->expert_format == LATENTMOE_EXPERTS_FP4_E2M1_E4M3_B16 && gemm_mid_setup() != 0)) {
    (void)hipGetLastError();
    (void)hipFree(h->workspace);
    delete h;
    return LATENTMOE_ERR_HIP;
  }
  char* base = static_cast<char*>(h->workspace);
  for (auto& it : L.items) {
    *it.first = base;
    base += (it.second + 255) & ~size_t(255);
  }
  if (h->linear) h->b.pieces = h->b.wx;
  if (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
      hipStreamCreateWithFlags(&h->side2, hipStreamNonBlocking) != hipSuccess ||
      hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_fork2, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_join2, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_hi, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_hi_done, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    latentmoe_destroy(h);
    return LATENTMOE_ERR_HIP;
  }
  launch_router_split(w->router_w, h->b.pieces, (long long)cfg->n_experts * cfg->d, stream);
  if (h->linear) {
    // stacked copies: wx rows [3N, 3N + l) = W_down, then S1; wy = [W_up | S2] row by row
    const size_t N = cfg->n_experts, d = cfg->d, l = cfg->latent, ms = cfg->shared_hidden;
    uint16_t* wx = h->b.wx;
    if (hipMemcpyAsync(wx + 3 * N * d, w->w_down, l * d * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(wx + (3 * N + l) * d, w->shared_w1, ms * d * 2, hipMemcpyDeviceToDevice, stream) !=
            hipSuccess ||
        hipMemcpy2DAsync(h->b.wy, (l + ms) * 2, w->w_up, l * 2, l * 2, d, hipMemcpyDeviceToDevice, stream) !=
            hipSuccess ||
        hipMemcpy2DAsync(h->b.wy + l, (l + ms) * 2, w->shared_w2, ms * 2, ms * 2, d, hipMemcpyDeviceToDevice,
                         stream) != hipSuccess) {
      (void)hipGetLastError();
      latentmoe_destroy(h);
      return LATENTMOE_ERR_HIP;
    }
  }
  if (h->b.w1_scale_sm)
    launch_scale_stage_major(w->expert_w1_scale, h->b.w1_scale_sm, cfg->n_experts,
                             cfg->expert_hidden, cfg->latent, stream);
  if (h->b.w2_scale_sm)
    launch_scale_stage_major(w->expert_w2_scale, h->b.w2_scale_sm, cfg->n_experts, cfg->latent,
                             cfg->expert_hidden, stream);
  const long long n_shared = (long long)cfg->shared_hidden * cfg->d;  // elements per matrix
  const long long n_proj = (long long)cfg->latent * cfg->d;
  if (h->b.s1_bf16) {
    launch_fp4_dequant(static_cast<const uint8_t*>(w->shared_w1), w->shared_w1_scale,
                       n_shared / 16, h->b.s1_bf16, stream);
    launch_fp4_dequant(static_cast<const uint8_t*>(w->shared_w2), w->shared_w2_scale,
                       n_shared / 16, h->b.s2_bf16, stream);
  }
  if (h->b.wd_bf16) {
    launch_fp8_dequant(static_cast<const uint8_t*>(w->w_down), n_proj / 16, h->b.wd_bf16, stream);
    launch_fp8_dequant(static_cast<const uint8_t*>(w->w_up), n_proj / 16, h->b.wu_bf16, stream);
  }
  // the derived copies are complete before the handle is used on any stream
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    latentmoe_destroy(h);
    return LATENTMOE_ERR_HIP;
  }
  *out = h;
  return LATENTMOE_OK;
}

}  // namespace

extern "C" {

int latentmoe_init(const latentmoe_config* cfg, const latentmoe_weights* w, hipStream_t stream,
                   latentmoe_handle_t* out) {
  if (!out) return LATENTMOE_ERR_INVALID_ARG;
  *out = nullptr;
  int st = check_config(cfg);
  if (st != LATENTMOE_OK) return st;
  if (!w || !w->router_w || !w->w_down || !w->w_up || !w->expert_w1 || !w->expert_w2 ||
      !w->shared_w1 || !w->shared_w2)
    return LATENTMOE_ERR_INVALID_ARG;
  if (cfg->expert_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 &&
      (!w->expert_w1_scale || !w->expert_w2_scale || !w->expert_w1_tscale || !w->expert_w2_tscale))
    return LATENTMOE_ERR_INVALID_ARG;
  if (cfg->shared_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 &&
      (!w->shared_w1_scale || !w->shared_w2_scale || !w->shared_w1_tscale || !w->shared_w2_tscale))
    return LATENTMOE_ERR_INVALID_ARG;
  if (cfg->proj_format == LATENTMOE_FORMAT_FP8_E4M3 && (!w->w_down_tscale || !w->w_up_tscale))
    return LATENTMOE_ERR_INVALID_ARG;
  if (!needs_pad(*cfg)) {
    st = init_handle(cfg, w, stream, out);
    if (st == LATENTMOE_OK) (*out)->ucfg = *cfg;
    return st;
  }
  // zero-padded copies of the weights (enqueued on `stream`, which init_handle
  // synchronises before it returns), then the handle at the padded widths
  PadPlan P = make_pad_plan(*cfg, w);
  const char* fail = std::getenv("LATENTMOE_FAIL_ALLOC");
  void* buf = nullptr;
  if ((fail && fail[0] == '1') || hipMalloc(&buf, P.total) != hipSuccess) {
    (void)hipGetLastError();
    return LATENTMOE_ERR_OUT_OF_MEMORY;
  }
  place_pad_plan(P, static_cast<char*>(buf), stream);
  const latentmoe_config pc = padded_config(*cfg);
  st = init_handle(&pc, &P.w, stream, out);
  if (st != LATENTMOE_OK) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(buf);
    return st;
  }
  latentmoe_handle_s* h = *out;
  h->ucfg = *cfg;
  h->pad_buf = buf;
  h->x_pad = reinterpret_cast<uint16_t*>(static_cast<char*>(buf) + P.x_off);
  h->y_pad = reinterpret_cast<float*>(static_cast<char*>(buf) + P.y_off);
  return LATENTMOE_OK;
}

int latentmoe_destroy(latentmoe_handle_t h) {
  if (!h) return LATENTMOE_OK;
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_fork2) (void)hipEventDestroy(h->ev_fork2);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->ev_join2) (void)hipEventDestroy(h->ev_join2);
  if (h->ev_hi) (void)hipEventDestroy(h->ev_hi);
  if (h->ev_hi_done) (void)hipEventDestroy(h->ev_hi_done);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->side2) (void)hipStreamDestroy(h->side2);
  drop_graph(h);
  if (h->cap) (void)hipStreamDestroy(h->cap);
  hipError_t e = h->workspace ? hipFree(h->workspace) : hipSuccess;
  if (h->pad_buf && hipFree(h->pad_buf) != hipSuccess) e = hipErrorUnknown;
  delete h;
  return e == hipSuccess ? LATENTMOE_OK : LATENTMOE_ERR_HIP;
}

}  // extern "C"

namespace {

// enqueue one forward on stream s (eager, or into a stream capture)
void forward_impl(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y, int32_t* topk_idx,
                  float* topk_gate, hipStream_t s, bool timing) {

  const latentmoe_config& c = h->cfg;
  const latentmoe_weights& w = h->w;
  Buffers& b = h->b;
  const int N = c.n_experts, K = c.top_k, d = c.d, L = c.latent, m = c.expert_hidden,
            ms = c.shared_hidden;
  const bool fp4 = c.expert_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16;
  const int shared_fmt = c.shared_format == LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 ? WF_FP4 : WF_BF16;
  const int proj_fmt = c.proj_format == LATENTMOE_FORMAT_FP8_E4M3 ? WF_FP8 : WF_BF16;
  // single bf16 activations next to FP4 / FP8 weights (R17).  In a layer with FP4
  // experts the bf16 shared expert's h_s and W_up's input y_lat are single bf16 too
  // (on the multi-stream path, where the pairs cost a second MFMA pass): the layer's
  // output is held to the FP4 bound, and the expert path's own bf16 activations
  // already put ~7e-3 of rms(y) into it; a single h_s adds at most ~8e-3.
  const bool expert_a16 = fp4;                        // single bf16 z, h
  const bool shared_a16 = shared_fmt != WF_BF16 || fp4;  // single bf16 h_s
  const bool ylat_a16 = proj_fmt != WF_BF16 || fp4;      // W_up reads y_lat's high part
  const long long TK = (long long)T * K;
  StageTimer tm(h, s);
  if (!timing) tm.on = false;

  // The shared expert and W_down do not depend on routing.  Above 64 tokens the
  // shared expert (from 65 to STACK_X_ROWS tokens only S2) runs on a side stream
  // forked from the caller's stream (same priority) and joins before W_up, so its
  // GEMMs fill the latency-bound top-K / bucketing chain.  With the stacked weight
  // copies W_down shares the router's launch on the caller's stream; without them
  // (FP8 projections, an FP4 shared expert) it runs on a second side stream forked
  // at the start, and the shared expert forks after the router GEMM.
  // Stage-timed calls run in program order on the caller's stream as well, so
  // each stage's events bracket its own kernels with nothing beside them.
  const bool one_stream = h->serial || tm.on;
  hipStream_t side = h->side;
  hipStream_t side2 = h->side2;
  if (one_stream) side = side2 = s;
  // event edges between the streams (none on one stream)
  auto record = [&](hipEvent_t ev, hipStream_t on) {
    if (!one_stream) (void)hipEventRecord(ev, on);
  };
  auto wait = [&](hipStream_t on, hipEvent_t ev) {
    if (!one_stream) (void)hipStreamWaitEvent(on, ev, 0);
  };
  auto fork_to = [&](hipStream_t to, hipEvent_t ev) {
    record(ev, s);
    wait(to, ev);
  };
  auto shared_up = [&]() {
    // ---- shared expert (side stream): h_s = relu(S1 x)^2 as bf16 hi + lo, y = S2 h_s ----
    tm.start(LATENTMOE_STAGE_SHARED_UP, side);
    GemmParams ps = base_params();
    ps.seg[0] = GemmSeg{x, w.shared_w1, d};
    ps.nseg = 1;
    ps.lda = d;
    ps.ldb = d;
    ps.N = ms;
    if (shared_fmt == WF_FP4) {
      ps.b_scale = w.shared_w1_scale;
      ps.b_tscale = w.shared_w1_tscale;
    }
    ps.epi = shared_a16 ? EPI_SQRELU_BF16 : EPI_SQRELU_HILO;
    ps.C = b.hs_hi;
    ps.C2 = b.hs_lo;
    ps.ldc = ms;
    run_dense(h, ps, T, side, false, b.partial2, shared_fmt, b.s1_bf16);
    tm.stop(LATENTMOE_STAGE_SHARED_UP, side);
  };
  auto shared_down = [&]() {
    tm.start(LATENTMOE_STAGE_SHARED_DOWN, side);
    GemmParams p2 = base_params();
    p2.seg[0] = GemmSeg{b.hs_hi, w.shared_w2, ms};
    p2.a_lo = shared_a16 ? nullptr : b.hs_lo;
    p2.nseg = 1;
    p2.lda = ms;
    p2.ldb = ms;
    p2.N = d;
    if (shared_fmt == WF_FP4) {
      p2.b_scale = w.shared_w2_scale;
      p2.b_tscale = w.shared_w2_tscale;
    }
    p2.epi = EPI_F32;
    p2.C = y;
    p2.ldc = d;
    run_dense(h, p2, T, side, false, b.partial2, shared_fmt, b.s2_bf16);
    tm.stop(LATENTMOE_STAGE_SHARED_DOWN, side);

    record(h->ev_join, side);
  };
  auto down_proj = [&]() {
    // ---- z = W_down x (side stream 2, concurrent with routing) ----
    tm.start(LATENTMOE_STAGE_DOWN_PROJ, side2);
    GemmParams pd = base_params();
    pd.seg[0] = GemmSeg{x, w.w_down, d};
    pd.nseg = 1;
    pd.lda = d;
    pd.ldb = d;
    pd.N = L;
    if (proj_fmt == WF_FP8) pd.b_tscale = w.w_down_tscale;
    pd.epi = EPI_BF16_HILO;
    pd.C = b.z;
    pd.C2 = b.z_lo;
    pd.ldc = L;
    run_dense(h, pd, T, side2, false, b.partial3, proj_fmt, b.wd_bf16);
    tm.stop(LATENTMOE_STAGE_DOWN_PROJ, side2);
    record(h->ev_join2, side2);
  };
  // decode-sized forward on one stream (the stacked GEMMs); otherwise W_down and the
  // shared expert run on the side streams
  const bool linear = h->linear && T <= STREAM_ROWS_BIG;
  h->last_linear = linear;
  const bool stack_x = h->linear && !linear && T <= STACK_X_ROWS;
  // above that, the router pieces and W_down still share one launch and one reduce,
  // with the shared expert on the side stream
  const bool stack_rz = h->linear && !linear && !stack_x;
  const int LS = L + ms;  // row length of the stacked activations [y_lat | h_s]
  // bf16 experts on the streaming kernel: the shared expert's GEMMs run inside the
  // expert launches (S1 with expert up, S2 with expert down) instead of in the
  // stacked GEMMs, where a few tokens' dense GEMM is a latency-bound launch
  const bool shared_rides = linear && !fp4 && (double)TK / N <= 48.0;
  const int MSX = shared_rides ? 0 : ms;  // shared-hidden rows of the stacked x GEMM
  if (linear) {
    // ---- 1. router logits, z = W_down x (and the shared hidden) in one GEMM over x ----
    tm.start(LATENTMOE_STAGE_ROUTER);
    GemmParams px = base_params();
    px.seg[0] = GemmSeg{x, b.wx, d};
    px.nseg = 1;
    px.lda = d;
    px.ldb = d;
    px.N = 3 * N + L + MSX;
    px.ldc = px.N;
    const int splits = run_dense(h, px, T, s, true, b.partial, WF_BF16, nullptr, TARGET_BLOCKS_STACKED);
    launch_xreduce(b.partial, splits, (long long)T * px.N, T, N, L, MSX, b.logits, b.z, b.z_lo, b.ay + L,
                   b.ay_lo + L, LS, s);
    tm.stop(LATENTMOE_STAGE_ROUTER);
    // stages without a launch of their own here are recorded empty
    for (int st : {LATENTMOE_STAGE_DOWN_PROJ, LATENTMOE_STAGE_SHARED_UP, LATENTMOE_STAGE_SHARED_DOWN}) {
      tm.start(st);
      tm.stop(st);
    }
  } else if (stack_x || stack_rz) {
    // ---- 1. router logits, z = W_down x and (up to STACK_X_ROWS tokens) h_s =
    // relu(S1 x)^2 in one GEMM over x (partial sums, then one reduce that sums the
    // router pieces); the rest of the shared expert on the side stream ----
    const int MSX = stack_x ? ms : 0;
    if (stack_rz) {
      fork_to(side, h->ev_fork2);
      shared_up();
      shared_down();
    }
    tm.start(LATENTMOE_STAGE_ROUTER);
    GemmParams px = base_params();
    px.seg[0] = GemmSeg{x, b.wx, d};
    px.nseg = 1;
    px.lda = d;
    px.ldb = d;
    px.N = 3 * N + L + MSX;
    px.ldc = px.N;
    const int splits = run_dense(h, px, T, s, true, b.partial);
    launch_xreduce(b.partial, splits, (long long)T * px.N, T, N, L, MSX, b.logits, b.z, b.z_lo, b.hs_hi,
                   b.hs_lo, ms, s);
    tm.stop(LATENTMOE_STAGE_ROUTER);
    tm.start(LATENTMOE_STAGE_DOWN_PROJ);
    tm.stop(LATENTMOE_STAGE_DOWN_PROJ);
    if (stack_x) {
      tm.start(LATENTMOE_STAGE_SHARED_UP);
      tm.stop(LATENTMOE_STAGE_SHARED_UP);
      fork_to(side, h->ev_fork2);
      shared_down();
    }
  } else {
    fork_to(side2, h->ev_fork);
    down_proj();

    // ---- 1. router logits: x [T, d] times the three exact bf16 pieces of W_r ----
    tm.start(LATENTMOE_STAGE_ROUTER);
    GemmParams pr = base_params();
    for (int i = 0; i < 3; ++i) pr.seg[i] = GemmSeg{x, b.pieces + (size_t)i * N * d, d};
    pr.nseg = 3;
    pr.lda = d;
    pr.ldb = d;
    pr.N = N;
    pr.ldc = N;
    pr.epi = EPI_F32;
    pr.C = b.logits;
    run_dense(h, pr, T, s, false);
    tm.stop(LATENTMOE_STAGE_ROUTER);
    fork_to(side, h->ev_fork2);
    shared_up();
    shared_down();
  }

  // ---- 2. top-K + softmax over the logits (plus the bias, when given) ----
  tm.start(LATENTMOE_STAGE_TOPK);
  int* idx_buf = topk_idx ? topk_idx : b.idx;  // written in place when the caller asks
  float* gate_buf = topk_gate ? topk_gate : b.gates;
  const double avg_rows = (double)TK / N;
  const bool expert_stream = fp4 || avg_rows <= 48.0;
  // large-tile path: rows split by gate energy into a hi + lo class and a bf16 class
  const bool split_rows = !expert_stream;
  uint32_t* masks_hi = split_rows ? b.masks_hi : nullptr;
  launch_topk(b.logits, w.router_bias, T, N, K, idx_buf, gate_buf, b.masks, PAIR_TAIL_FRAC,
              masks_hi, b.paired, s);
  tm.stop(LATENTMOE_STAGE_TOPK);

  // ---- 3. bucketing ----
  const int rows_per_tile =
      !expert_stream                   ? TILE_ROWS
      : avg_rows <= ROWS16_MAX_AVG ? STREAM_ROWS_SMALL
      : avg_rows <= ROWS32_MAX_AVG ? STREAM_ROWS_MID
                                        : STREAM_ROWS_BIG;
  const int max_tiles =
      ceil_div(TK, rows_per_tile) + (split_rows ? 2 : 1) * (int)std::min<long long>(N, TK);
  tm.start(LATENTMOE_STAGE_BUCKET);
  const bool fuse_place = TK <= 8192;  // one workgroup places a few thousand rows quickly
  // many mask blocks: count them in chunks on many workgroups first
  const bool chunked = !fuse_place && bucket_chunks(T) >= BUCKET_MIN_CHUNKS;
  int* chunk_hi = chunked ? b.chunk_hi : nullptr;
  int* chunk_lo = chunked ? b.chunk_lo : nullptr;
  launch_bucket_scan(b.masks, masks_hi, T, N, rows_per_tile, b.counts, b.counts_hi, b.offsets,
                     b.block_prefix, b.prefix_lo, b.tile_expert, b.tile_row0, b.tile_rows,
                     b.n_tiles, max_tiles, fuse_place ? idx_buf : nullptr, gate_buf, K, b.row_src,
                     b.row_gate, b.inv, chunk_hi, chunk_lo, s);
  if (!fuse_place)
    launch_place(idx_buf, gate_buf, b.masks, masks_hi, b.offsets, b.counts_hi, b.block_prefix,
                 b.prefix_lo, T, N, K, b.row_src, b.row_gate, b.inv, chunk_hi, chunk_lo, s);
  tm.stop(LATENTMOE_STAGE_BUCKET);

  // ---- 4. wait for z = W_down x (side stream 2) ----
  if (!linear && !stack_x && !stack_rz) wait(s, h->ev_join2);

  // ---- 5/6. grouped expert GEMMs ----
  GemmParams pe = base_params();
  pe.nseg = 1;
  pe.tile_expert = b.tile_expert;
  pe.tile_row0 = b.tile_row0;
  pe.tile_rows = b.tile_rows;
  pe.n_tiles = b.n_tiles;
  pe.max_tiles = max_tiles;
  pe.rows_per_tile = rows_per_tile;
  pe.M = rows_per_tile;
  pe.splits = 1;

  // epi_lo, c_lo: the epilogue and output of the bf16-class launch (split rows)
  auto launch_expert = [&](const GemmParams& g, int epi_lo, void* c_lo) {
    if (split_rows) {
      launch_gemm_big(g, s);  // hi tiles: tiles [0, n_tiles[0])
      GemmParams gl = g;      // then tiles [n_tiles[0], n_tiles[0] + n_tiles[1]), one part
      gl.n_tiles = b.n_tiles + 1;
      gl.tile_first = b.n_tiles;
      gl.a_lo = nullptr;
      gl.epi = epi_lo;
      gl.C = c_lo;
      gl.C2 = nullptr;
      launch_gemm_big(gl, s);
    } else if (!expert_stream)
      launch_gemm_big(g, s);
    else if (rows_per_tile == STREAM_ROWS_BIG && gemm_mid_supports(g, fp4))
      launch_gemm_mid(g, fp4, s);
    else
      launch_gemm_stream(g, fp4 ? WF_FP4 : WF_BF16, s);
  };

  GemmParams pu = pe;
  pu.seg[0] = GemmSeg{b.z, w.expert_w1, L};
  pu.a_lo = expert_a16 ? nullptr : b.z_lo;
  pu.lda = L;
  pu.ldb = L;
  pu.N = m;
  pu.k_split = L;
  pu.row_index = b.row_src;
  pu.b_stride = (long long)m * L;
  pu.b_scale = fp4 ? w.expert_w1_scale : nullptr;
  pu.b_scale_sm = b.w1_scale_sm;
  pu.b_tscale = fp4 ? w.expert_w1_tscale : nullptr;
  pu.epi = expert_a16 ? EPI_SQRELU_BF16 : EPI_SQRELU_HILO;
  pu.C = b.h;
  pu.C2 = expert_a16 ? nullptr : b.h_lo;
  pu.ldc = m;

  GemmParams pw = pe;
  pw.seg[0] = GemmSeg{b.h, w.expert_w2, m};
  pw.a_lo = expert_a16 ? nullptr : b.h_lo;
  pw.lda = m;
  pw.ldb = m;
  pw.N = L;
  pw.k_split = m;
  pw.row_index = nullptr;
  pw.b_stride = (long long)L * m;
  pw.b_scale = fp4 ? w.expert_w2_scale : nullptr;
  pw.b_scale_sm = b.w2_scale_sm;
  pw.b_tscale = fp4 ? w.expert_w2_tscale : nullptr;
  pw.epi = EPI_GATE_F32;
  pw.row_scale = b.row_gate;
  pw.C = b.og;
  pw.ldc = L;

  // With split rows the hi class is a few tiles (often one expert's: the launches
  // fill part of the GPU); its expert down needs only its own expert up, so it runs
  // on side stream 2 beside the bf16 class's expert up, and the combine waits for
  // it.  Per-stage timing keeps the plain order, so each stage times whole launches.
  const bool hi_side = split_rows && !one_stream && !linear;
  // the bf16 class's expert-down rows go out as bf16: their rounding enters y_lat times
  // a gate below the class threshold, like that of their bf16 z and h; with FP4 experts
  // every gated row does (16-bit activations next to 4-bit weights, R17)
  const bool og_mix = split_rows;
  const bool og_bf16 = fp4 && !split_rows;
  if (hi_side) {
    launch_gemm_big(pu, s);  // expert up, hi tiles
    (void)hipEventRecord(h->ev_hi, s);
    (void)hipStreamWaitEvent(side2, h->ev_hi, 0);
    launch_gemm_big(pw, side2);  // expert down, hi tiles
    (void)hipEventRecord(h->ev_hi_done, side2);
    auto lo = [&](GemmParams g, int epi_lo, void* c_lo) {  // tiles [n_tiles[0], n_tiles[0] + n_tiles[1])
      g.n_tiles = b.n_tiles + 1;
      g.tile_first = b.n_tiles;
      g.a_lo = nullptr;
      g.epi = epi_lo;
      g.C = c_lo;
      g.C2 = nullptr;
      launch_gemm_big(g, s);
    };
    lo(pu, EPI_SQRELU_BF16, b.h);
    lo(pw, og_mix ? EPI_GATE_BF16 : EPI_GATE_F32, og_mix ? (void*)b.og16 : (void*)b.og);
    (void)hipStreamWaitEvent(s, h->ev_hi_done, 0);
  } else if (shared_rides) {
    // S1: h_s = relu(S1 x)^2 as bf16 hi + lo into the stacked rows [y_lat | h_s]
    GemmParams q1 = base_params();
    q1.seg[0] = GemmSeg{x, w.shared_w1, d};
    q1.nseg = 1;
    q1.lda = d;
    q1.ldb = d;
    q1.M = T;
    q1.N = ms;
    q1.splits = 1;
    q1.k_split = d;
    q1.epi = EPI_SQRELU_HILO;
    q1.C = b.ay + L;
    q1.C2 = b.ay_lo + L;
    q1.ldc = LS;
    // S2: y = S2 h_s (the up-projection adds onto it)
    GemmParams q2 = base_params();
    q2.seg[0] = GemmSeg{b.ay + L, w.shared_w2, ms};
    q2.a_lo = b.ay_lo + L;
    q2.nseg = 1;
    q2.lda = LS;
    q2.ldb = ms;
    q2.M = T;
    q2.N = d;
    q2.splits = 1;
    q2.k_split = ms;
    q2.epi = EPI_F32;
    q2.C = y;
    q2.ldc = d;
    tm.start(LATENTMOE_STAGE_EXPERT_UP);
    launch_gemm_stream_pair(pu, q1, s);
    tm.stop(LATENTMOE_STAGE_EXPERT_UP);
    tm.start(LATENTMOE_STAGE_EXPERT_DOWN);
    launch_gemm_stream_pair(pw, q2, s);
    tm.stop(LATENTMOE_STAGE_EXPERT_DOWN);
  } else {
    tm.start(LATENTMOE_STAGE_EXPERT_UP);
    launch_expert(pu, EPI_SQRELU_BF16, b.h);
    tm.stop(LATENTMOE_STAGE_EXPERT_UP);
    tm.start(LATENTMOE_STAGE_EXPERT_DOWN);
    if (og_bf16) {
      GemmParams g = pw;
      g.epi = EPI_GATE_BF16;
      g.C = b.og16;
      launch_expert(g, EPI_GATE_BF16, b.og16);
    } else {
      launch_expert(pw, og_mix ? EPI_GATE_BF16 : EPI_GATE_F32, og_mix ? (void*)b.og16 : (void*)b.og);
    }
    tm.stop(LATENTMOE_STAGE_EXPERT_DOWN);
  }

  // ---- 7. combine ----
  tm.start(LATENTMOE_STAGE_COMBINE);
  launch_combine(b.og, og_mix || og_bf16 ? b.og16 : nullptr, og_mix ? b.paired : nullptr, b.inv, T, K, L,
                 linear ? b.ay : b.y_lat, linear ? b.ay_lo : b.y_lat_lo, linear ? LS : L, s);
  tm.stop(LATENTMOE_STAGE_COMBINE);

  if (linear) {
    // ---- 8. y = [W_up | S2] [y_lat ; h_s], both as bf16 hi + lo; or, when S2 ran
    // with expert down, y += W_up y_lat (the first L columns of the stacked rows) ----
    tm.start(LATENTMOE_STAGE_UP_PROJ);
    GemmParams pq = base_params();
    pq.seg[0] = GemmSeg{b.ay, b.wy, shared_rides ? L : LS};
    pq.a_lo = b.ay_lo;
    pq.nseg = 1;
    pq.lda = LS;
    pq.ldb = LS;
    pq.N = d;
    pq.epi = shared_rides ? EPI_F32_ADD : EPI_F32;
    pq.C = y;
    pq.ldc = d;
    run_dense(h, pq, T, s, false, nullptr, WF_BF16, nullptr, shared_rides ? TARGET_BLOCKS_UP : TARGET_BLOCKS_STACKED);
    tm.stop(LATENTMOE_STAGE_UP_PROJ);
    tm.done();
    h->last_T = T;
    return;
  }

  // ---- 8. y += W_up y_lat (after the shared expert wrote y) ----
  wait(s, h->ev_join);
  tm.start(LATENTMOE_STAGE_UP_PROJ);
  GemmParams pp = base_params();
  pp.seg[0] = GemmSeg{b.y_lat, w.w_up, L};
  pp.a_lo = ylat_a16 ? nullptr : b.y_lat_lo;
  pp.nseg = 1;
  pp.lda = L;
  pp.ldb = L;
  pp.N = d;
  if (proj_fmt == WF_FP8) pp.b_tscale = w.w_up_tscale;
  pp.epi = EPI_F32_ADD;
  pp.C = y;
  pp.ldc = d;
  run_dense(h, pp, T, s, false, nullptr, proj_fmt, b.wu_bf16);
  tm.stop(LATENTMOE_STAGE_UP_PROJ);
  tm.done();
  h->last_T = T;
}

int check_forward_args(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y) {
  if (!h || T < 0) return LATENTMOE_ERR_INVALID_ARG;
  if (T == 0) return LATENTMOE_OK;
  if (!x || !y || T > h->cfg.max_tokens) return LATENTMOE_ERR_INVALID_ARG;
  return 1;  // proceed
}

// the forward at the caller's widths: padded widths copy x into x_pad (zeros past
// d) and crop y out of y_pad around the forward
void forward_outer(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y, int32_t* topk_idx,
                   float* topk_gate, hipStream_t s, bool eager) {
  if (!h->pad_buf) {
    forward_impl(h, x, T, y, topk_idx, topk_gate, s, eager);
    return;
  }
  const size_t d = h->ucfg.d, D = h->cfg.d;
  launch_pad_copy(x, d * 2, T, h->x_pad, D * 2, T, 1, T, d * 2, s);
  forward_impl(h, h->x_pad, T, h->y_pad, topk_idx, topk_gate, s, eager);
  launch_pad_copy(h->y_pad, D * 4, T, y, d * 4, T, 1, T, d * 4, s);
}

void drop_graph(latentmoe_handle_s* h) {
  if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  h->gexec = nullptr;
  h->graph = nullptr;
}

}  // namespace

extern "C" {

int latentmoe_forward(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y,
                      int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  const int st = check_forward_args(h, x, T, y);
  if (st != 1) return st;
  (void)hipGetLastError();
  forward_outer(h, x, T, y, topk_idx, topk_gate, s, true);
  return hipGetLastError() == hipSuccess ? LATENTMOE_OK : LATENTMOE_ERR_HIP;
}

int latentmoe_forward_graph(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y,
                            int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  const int st = check_forward_args(h, x, T, y);
  if (st != 1) return st;
  (void)hipGetLastError();
  const GraphKey key{x, T, y, topk_idx, topk_gate};
  if (!h->gexec || !(key == h->gkey)) {
    drop_graph(h);
    if (hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal) != hipSuccess)
      return LATENTMOE_ERR_HIP;
    forward_outer(h, x, T, y, topk_idx, topk_gate, h->cap, false);
    hipGraph_t g = nullptr;
    if (hipStreamEndCapture(h->cap, &g) != hipSuccess || !g) {
      (void)hipGetLastError();
      return LATENTMOE_ERR_HIP;
    }
    h->graph = g;
    if (hipGraphInstantiate(&h->gexec, g, nullptr, nullptr, 0) != hipSuccess) {
      (void)hipGetLastError();
      drop_graph(h);
      return LATENTMOE_ERR_HIP;
    }
    h->gkey = key;
  }
  if (hipGraphLaunch(h->gexec, s) != hipSuccess) return LATENTMOE_ERR_HIP;
  h->last_T = T;
  return hipGetLastError() == hipSuccess ? LATENTMOE_OK : LATENTMOE_ERR_HIP;
}

int latentmoe_debug_copy(latentmoe_handle_t h, int which, void* dst, size_t bytes,
                         hipStream_t s) {
  if (!h || !dst) return LATENTMOE_ERR_INVALID_ARG;
  const latentmoe_config& c = h->cfg;   // the widths the buffers have
  const latentmoe_config& u = h->ucfg;  // the caller's widths (the copies' rows)
  const size_t T = h->last_T, K = c.top_k;
  // rows of w bytes, `pitch` bytes apart in the buffer (decode-sized forwards keep
  // y_lat and h_s side by side in rows of l + m_s)
  const size_t LS = (size_t)(c.latent + c.shared_hidden) * 2;
  const bool lin = h->last_linear;
  const void* src = nullptr;
  size_t w = 0, pitch = 0, rows = 1;
  // rows of `width` bf16 values, `wbuf` apart in the buffer
  auto bf16_rows = [&](const void* p, int width, size_t wbuf, size_t n) {
    src = p;
    w = (size_t)width * 2;
    pitch = wbuf;
    rows = n;
  };
  // one flat run of `n` bytes
  auto flat = [&](const void* p, size_t n) {
    src = p;
    w = pitch = n;
  };
  const size_t L2 = (size_t)c.latent * 2, M2 = (size_t)c.expert_hidden * 2, MS2 = (size_t)c.shared_hidden * 2;
  switch (which) {
    case LATENTMOE_INTER_Z: bf16_rows(h->b.z, u.latent, L2, T); break;
    case LATENTMOE_INTER_Z_LO: bf16_rows(h->b.z_lo, u.latent, L2, T); break;
    case LATENTMOE_INTER_Y_LAT:
      if (lin) bf16_rows(h->b.ay, u.latent, LS, T);
      else bf16_rows(h->b.y_lat, u.latent, L2, T);
      break;
    case LATENTMOE_INTER_Y_LAT_LO:
      if (lin) bf16_rows(h->b.ay_lo, u.latent, LS, T);
      else bf16_rows(h->b.y_lat_lo, u.latent, L2, T);
      break;
    case LATENTMOE_INTER_HS_HI:
      if (lin) bf16_rows(h->b.ay + c.latent, u.shared_hidden, LS, T);
      else bf16_rows(h->b.hs_hi, u.shared_hidden, MS2, T);
      break;
    case LATENTMOE_INTER_HS_LO:
      if (lin) bf16_rows(h->b.ay_lo + c.latent, u.shared_hidden, LS, T);
      else bf16_rows(h->b.hs_lo, u.shared_hidden, MS2, T);
      break;
    case LATENTMOE_INTER_H: bf16_rows(h->b.h, u.expert_hidden, M2, T * K); break;
    case LATENTMOE_INTER_H_LO: bf16_rows(h->b.h_lo, u.expert_hidden, M2, T * K); break;
    case LATENTMOE_INTER_COUNTS: flat(h->b.counts, (size_t)c.n_experts * 4); break;
    case LATENTMOE_INTER_OFFSETS: flat(h->b.offsets, (size_t)(c.n_experts + 1) * 4); break;
    case LATENTMOE_INTER_ROW_SRC: flat(h->b.row_src, T * K * 4); break;
    case LATENTMOE_INTER_INV: flat(h->b.inv, T * K * 4); break;
    case LATENTMOE_INTER_PAIRED: flat(h->b.paired, T * K); break;
    default: return LATENTMOE_ERR_INVALID_ARG;
  }
  if (bytes > w * rows) return LATENTMOE_ERR_INVALID_ARG;
  if (bytes == 0) return LATENTMOE_OK;
  const size_t full = bytes / w, rest = bytes % w;
  if (full && hipMemcpy2DAsync(dst, w, src, pitch, w, full, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return LATENTMOE_ERR_HIP;
  if (rest && hipMemcpyAsync(static_cast<char*>(dst) + full * w, static_cast<const char*>(src) + full * pitch,
                             rest, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return LATENTMOE_ERR_HIP;
  return LATENTMOE_OK;
}

int latentmoe_profile_begin(latentmoe_handle_t h, int max_calls, uint32_t stage_mask) {
  if (!h || max_calls < 1) return LATENTMOE_ERR_INVALID_ARG;
  h->prof_mask = stage_mask;
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.assign((size_t)max_calls * LATENTMOE_NUM_STAGES * 2, nullptr);
  for (auto& e : h->events)
    if (hipEventCreate(&e) != hipSuccess) return LATENTMOE_ERR_HIP;
  h->prof_max = max_calls;
  h->prof_calls = 0;
  h->profiling = true;
  return LATENTMOE_OK;
}

int latentmoe_profile_end(latentmoe_handle_t h, float* stage_ms, int n_stages, int* calls) {
  if (!h || !stage_ms || !calls || n_stages < 0) return LATENTMOE_ERR_INVALID_ARG;
  h->profiling = false;
  std::vector<double> sum(LATENTMOE_NUM_STAGES, 0.0);
  for (int c = 0; c < h->prof_calls; ++c) {
    for (int st = 0; st < LATENTMOE_NUM_STAGES; ++st) {
      if (!((h->prof_mask >> st) & 1u)) continue;
      hipEvent_t a = h->events[((size_t)c * LATENTMOE_NUM_STAGES + st) * 2];
      hipEvent_t z = h->events[((size_t)c * LATENTMOE_NUM_STAGES + st) * 2 + 1];
      if (hipEventSynchronize(z) != hipSuccess) return LATENTMOE_ERR_HIP;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, a, z) != hipSuccess) return LATENTMOE_ERR_HIP;
      sum[st] += ms;
    }
  }
  for (int st = 0; st < n_stages; ++st) stage_ms[st] = st < LATENTMOE_NUM_STAGES ? (float)sum[st] : 0.f;
  *calls = h->prof_calls;
  return LATENTMOE_OK;
}

int latentmoe_fp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t n_blocks,
                         uint16_t* out, hipStream_t s) {
  if (!codes || !scales || !out || n_blocks < 0) return LATENTMOE_ERR_INVALID_ARG;
  (void)hipGetLastError();
  launch_fp4_dequant(codes, scales, n_blocks, out, s);
  return hipGetLastError() == hipSuccess ? LATENTMOE_OK : LATENTMOE_ERR_HIP;
}

int latentmoe_fp8_decode(const uint8_t* codes, int64_t n_groups, uint16_t* out, hipStream_t s) {
  if (!codes || !out || n_groups < 0) return LATENTMOE_ERR_INVALID_ARG;
  (void)hipGetLastError();
  launch_fp8_dequant(codes, n_groups, out, s);
  return hipGetLastError() == hipSuccess ? LATENTMOE_OK : LATENTMOE_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// latentmoe_forward_static: the forward without a handle, its workspace in a
// file-scope device array.  In host code `scratch` names a host-side stand-in,
// not device memory: the device address comes from hipGetSymbolAddress, once
// per device, and only that address is passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[LATENTMOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int STATIC_MAX_DEVICES = 64;
std::mutex g_static_mu;
void* g_static_ptr[STATIC_MAX_DEVICES];  // device address of `scratch` per device

// the array's address on the current device (looked up on the first call there,
// with the large-tile kernel's attributes set at the same time)
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LATENTMOE_ERR_HIP;
  if (dev < 0 || dev >= STATIC_MAX_DEVICES) return LATENTMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p || gemm_big_setup() != 0) {
      (void)hipGetLastError();
      return LATENTMOE_ERR_HIP;
    }
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return LATENTMOE_OK;
}

}  // namespace

extern "C" int latentmoe_forward_static(const latentmoe_config* cfg, const latentmoe_weights* w,
                                        const uint16_t* x, int32_t T, float* y, int32_t* topk_idx,
                                        float* topk_gate, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LATENTMOE_OK) return st;
  if (cfg->expert_format != LATENTMOE_FORMAT_BF16 || cfg->shared_format != LATENTMOE_FORMAT_BF16 ||
      cfg->proj_format != LATENTMOE_FORMAT_BF16 || needs_pad(*cfg))
    return LATENTMOE_ERR_UNSUPPORTED;
  if (!w || !w->router_w || !w->w_down || !w->w_up || !w->expert_w1 || !w->expert_w2 ||
      !w->shared_w1 || !w->shared_w2 || T < 0)
    return LATENTMOE_ERR_INVALID_ARG;
  if (T == 0) return LATENTMOE_OK;
  if (!x || !y || T > cfg->max_tokens) return LATENTMOE_ERR_INVALID_ARG;
  // the workspace laid out for this call's T
  latentmoe_handle_s h;
  h.cfg = *cfg;
  h.cfg.max_tokens = T;
  h.w = *w;
  h.serial = true;  // one stream, no events
  const Layout L = make_layout(h.cfg, h.b, false);
  if (L.total > (size_t)LATENTMOE_STATIC_SCRATCH_BYTES) return LATENTMOE_ERR_SCRATCH;
  void* base = nullptr;
  st = static_scratch(&base);
  if (st != LATENTMOE_OK) return st;
  char* at = static_cast<char*>(base);
  for (const auto& it : L.items) {
    *it.first = at;
    at += (it.second + 255) & ~size_t(255);
  }
  (void)hipGetLastError();
  // what the handle path derives once at init, here on every call: the router's
  // split weights
  launch_router_split(w->router_w, h.b.pieces, (long long)cfg->n_experts * cfg->d, stream);
  forward_impl(&h, x, T, y, topk_idx, topk_gate, stream, false);
  return hipGetLastError() == hipSuccess ? LATENTMOE_OK : LATENTMOE_ERR_HIP;
}
