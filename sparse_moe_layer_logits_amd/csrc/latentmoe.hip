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
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/latentmoe.h"
#include "kernels.hpp"

using namespace lmoe;

namespace {

#ifndef LMOE_SHARED_FORK_AT
#define LMOE_SHARED_FORK_AT 1  // 0: at the start, 1: after the router GEMM, 2: after bucketing
#endif

constexpr int STREAM_ROWS_BIG = 64;
constexpr int STREAM_ROWS_SMALL = 16;  // decode expert tiles
constexpr int STREAM_ROWS_MID = 32;
#ifndef LMOE_ROWS16_MAX_AVG
#define LMOE_ROWS16_MAX_AVG 12.0  // up to this many rows per expert on average: 16-row tiles
#endif
#ifndef LMOE_ROWS32_MAX_AVG
#define LMOE_ROWS32_MAX_AVG 24.0  // then up to this many: 32-row tiles, above: 64
#endif
constexpr int TILE_ROWS = 256;          // rows per tile of the large-tile kernel
#ifndef LMOE_HI_TAU
// Large-tile path (prefill): routed rows whose gate is at least this carry
// their activations as bf16 hi + lo; the others as bf16.  A row's rounding
// reaches the output multiplied by its gate, so the small-gate rows add little
// error (fp64 emulation of the rounding points: max |y - y_exact| rises from
// 1e-5 to 2.6e-3 rms with a uniform router, stays 1e-5 with the skewed one).
#define LMOE_HI_TAU 0.1
#endif
#ifndef LMOE_SERIAL
#define LMOE_SERIAL 0  // 1: no side streams
#endif
#ifndef LMOE_MID_FP4
#define LMOE_MID_FP4 1  // FP4 experts with 64-row tiles use the mid kernel
#endif
// Activations of GEMMs whose weights are stored in FP4 or FP8 are single bf16
// values: weight-only quantisation with 16-bit activations, the W4A16 mode in
// which Hopper GPUs serve the NVFP4 checkpoint ("Nemotron 3.5 Super and
// Lightning", limitations; "Nemotron 3 Ultra", contributions).  bf16 weights keep
// the hi + lo pairs.  The bf16 rounding of an activation (2^-9 relative) is far
// below the weight formats' own step.
#ifndef LMOE_LOWP_A16
#define LMOE_LOWP_A16 1
#endif

#ifndef LMOE_BIG_KGRAN
#define LMOE_BIG_KGRAN 512
#endif
#ifndef LMOE_OG16
#define LMOE_OG16 1  // bf16-class expert-down rows stored as bf16 (two row classes)
#endif
#ifndef LMOE_HI_DOWN_SIDE
#define LMOE_HI_DOWN_SIDE 1  // hi-class expert down on side stream 2 beside the bf16-class expert up
#endif
#ifndef LMOE_BUCKET_MIN_CHUNKS
#define LMOE_BUCKET_MIN_CHUNKS 4  // chunks of 16 mask blocks (256 tokens) from which the count is split
#endif
#ifndef LMOE_TARGET_BLOCKS
#define LMOE_TARGET_BLOCKS 256
#endif
constexpr int TARGET_BLOCKS = LMOE_TARGET_BLOCKS;  // streaming kernel: 8-wave blocks, several per CU
constexpr int TARGET_BLOCKS_BIG = 256;  // large-tile kernel: one 4-wave block per CU

struct Plan {
  bool stream;  // weight-streaming kernel (true) or LDS-tiled kernel
  int splits;
  int k_split;
};

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// split-K plan for a dense GEMM of M rows, N columns, K reduction
Plan plan_dense(int M, int N, int K) {
  Plan p;
  p.stream = M <= STREAM_ROWS_BIG;
  const int per_split = p.stream ? ceil_div(N, 128) * ceil_div(M, STREAM_ROWS_BIG)
                                 : ceil_div(N, 256) * ceil_div(M, TILE_ROWS);
  // smallest k range of a split: with four or more row tiles the large-tile GEMMs
  // have blocks enough, and halving their splits halves the partial sums' traffic
  const int gran = !p.stream && M >= 4 * TILE_ROWS ? LMOE_BIG_KGRAN : 256;
  int want = std::max(1, ceil_div(p.stream ? TARGET_BLOCKS : TARGET_BLOCKS_BIG, per_split));
  want = std::min(want, std::max(1, K / gran));
  int ks = ceil_div(ceil_div(K, want), gran) * gran;
  p.k_split = ks;
  p.splits = ceil_div(K, ks);
  return p;
}

struct Buffers {
  uint16_t* pieces = nullptr;
  float* logits = nullptr;
  float* partial = nullptr;
  float* partial2 = nullptr;  // split-K partials of the shared expert (side stream)
  float* partial3 = nullptr;  // split-K partials of W_down (side stream 2)
  size_t partial_cap = 0;  // floats
  int* idx = nullptr;
  float* gates = nullptr;
  uint32_t* masks = nullptr;
  uint32_t* masks_hi = nullptr;  // rows whose gate reaches LMOE_HI_TAU (large-tile path)
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
  float* zrow32 = nullptr;   // zero rows of `latent` elements (fp32, bf16) for the combine
  uint16_t* zrow16 = nullptr;
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
  if (c->d % 64 || c->latent % 64 || c->expert_hidden % 64 || c->shared_hidden % 64)
    return LATENTMOE_ERR_UNSUPPORTED;
  if (c->n_experts % 16 || c->n_experts > 1024) return LATENTMOE_ERR_UNSUPPORTED;
  if (c->top_k > c->n_experts || c->top_k > 64) return LATENTMOE_ERR_UNSUPPORTED;
  return LATENTMOE_OK;
}

size_t max_partial_floats(const latentmoe_config& c) {
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
  }
  return best;
}

Layout make_layout(const latentmoe_config& c, Buffers& b) {
  Layout L;
  const size_t Tm = c.max_tokens, N = c.n_experts, K = c.top_k;
  const size_t TK = Tm * K;
  const size_t nblk = (Tm + 15) / 16;
  b.partial_cap = max_partial_floats(c);
  // every expert may end in one partial tile per row class
  b.max_tiles_cap = (int)(ceil_div(TK, STREAM_ROWS_SMALL) + 2 * std::min(N, TK));
  L.add((void**)&b.pieces, 3 * N * c.d * 2);
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
  L.add((void**)&b.z, Tm * c.latent * 2);
  L.add((void**)&b.z_lo, Tm * c.latent * 2);
  L.add((void**)&b.h, TK * c.expert_hidden * 2);
  L.add((void**)&b.h_lo, TK * c.expert_hidden * 2);
  L.add((void**)&b.og, TK * c.latent * 4);
  L.add((void**)&b.og16, TK * c.latent * 2);
  L.add((void**)&b.zrow32, (size_t)c.latent * 4);
  L.add((void**)&b.zrow16, (size_t)c.latent * 2);
  L.add((void**)&b.y_lat, Tm * c.latent * 2);
  L.add((void**)&b.y_lat_lo, Tm * c.latent * 2);
  L.add((void**)&b.hs_hi, Tm * c.shared_hidden * 2);
  L.add((void**)&b.hs_lo, Tm * c.shared_hidden * 2);
  if (c.expert_format == LATENTMOE_EXPERTS_FP4_E2M1_E4M3_B16 && c.latent % 128 == 0 &&
      c.expert_hidden % 128 == 0) {
    const size_t sc_bytes = N * (size_t)c.expert_hidden * (c.latent / 16);  // same for both
    L.add((void**)&b.w1_scale_sm, sc_bytes);
    L.add((void**)&b.w2_scale_sm, sc_bytes);
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
  latentmoe_config cfg;
  latentmoe_weights w;
  Buffers b;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  int last_T = 0;
  // the shared expert runs on a side stream forked from the caller's stream
  hipStream_t side = nullptr;
  hipStream_t side2 = nullptr;  // W_down, concurrent with routing
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
  void start(int stage, hipStream_t st = nullptr) {
    if (want(stage)) (void)hipEventRecord(h->events[((size_t)h->prof_calls * LATENTMOE_NUM_STAGES + stage) * 2], st ? st : s);
  }
  void stop(int stage, hipStream_t st = nullptr) {
    if (want(stage)) (void)hipEventRecord(h->events[((size_t)h->prof_calls * LATENTMOE_NUM_STAGES + stage) * 2 + 1], st ? st : s);
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
              float* partial = nullptr, int fmt = WF_BF16, const uint16_t* bf16_B = nullptr) {
  int Ktot = 0;
  for (int i = 0; i < p.nseg; ++i) Ktot += p.seg[i].K;
  Plan pl = plan_dense(T, p.N, Ktot);
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
    default: return "unknown status";
  }
}

int latentmoe_workspace_bytes(const latentmoe_config* cfg, size_t* bytes) {
  int st = check_config(cfg);
  if (st != LATENTMOE_OK) return st;
  if (!bytes) return LATENTMOE_ERR_INVALID_ARG;
  Buffers b;
  *bytes = make_layout(*cfg, b).total;
  return LATENTMOE_OK;
}

int latentmoe_init(const latentmoe_config* cfg, const latentmoe_weights* w, hipStream_t stream,
                   latentmoe_handle_t* out) {
  if (!out) return LATENTMOE_ERR_INVALID_ARG;
  *out = nullptr;
  int st = check_config(cfg);
  if (st != LATENTMOE_OK) return st;
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
  Layout L = make_layout(*cfg, h->b);
  if (hipMalloc(&h->workspace, L.total) != hipSuccess) {
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
  if (hipMemsetAsync(h->b.zrow32, 0, (size_t)cfg->latent * 4, stream) != hipSuccess ||
      hipMemsetAsync(h->b.zrow16, 0, (size_t)cfg->latent * 2, stream) != hipSuccess) {
    (void)hipGetLastError();
    latentmoe_destroy(h);
    return LATENTMOE_ERR_HIP;
  }
  if (h->b.w1_scale_sm) {
    launch_scale_stage_major(w->expert_w1_scale, h->b.w1_scale_sm, cfg->n_experts,
                             cfg->expert_hidden, cfg->latent, stream);
    launch_scale_stage_major(w->expert_w2_scale, h->b.w2_scale_sm, cfg->n_experts, cfg->latent,
                             cfg->expert_hidden, stream);
  }
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
  if (hipGetLastError() != hipSuccess) {
    latentmoe_destroy(h);
    return LATENTMOE_ERR_HIP;
  }
  *out = h;
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
  const bool shared_a16 = shared_fmt != WF_BF16 && LMOE_LOWP_A16;  // single bf16 h_s
  const bool expert_a16 = fp4 && LMOE_LOWP_A16;                   // single bf16 z, h
  const long long TK = (long long)T * K;
  StageTimer tm(h, s);
  if (!timing) tm.on = false;

  // The shared expert and W_down do not depend on routing: each runs on a side
  // stream forked from the caller's stream (same priority) and joins before
  // its consumer.  W_down is forked at the start; the shared expert after the
  // router GEMM, so the router runs at full speed and the shared expert's
  // weight stream fills the latency-bound top-K / bucketing chain.
  hipStream_t side = h->side;
  hipStream_t side2 = h->side2;
#if LMOE_SERIAL
  side = side2 = s;  // everything in one stream, in program order (per-stage profiling)
#endif
  auto fork_to = [&](hipStream_t to, hipEvent_t ev) {
    (void)hipEventRecord(ev, s);
    (void)hipStreamWaitEvent(to, ev, 0);
  };
  auto shared_expert = [&]() {
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

    (void)hipEventRecord(h->ev_join, side);
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
    (void)hipEventRecord(h->ev_join2, side2);
  };
  fork_to(side2, h->ev_fork);
  down_proj();
#if LMOE_SHARED_FORK_AT == 0
  fork_to(side, h->ev_fork2);
  shared_expert();
#endif

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
#if LMOE_SHARED_FORK_AT == 1
  fork_to(side, h->ev_fork2);
  shared_expert();
#endif

  // ---- 2. top-K + softmax (sums the router's split partials, adds the bias) ----
  tm.start(LATENTMOE_STAGE_TOPK);
  int* idx_buf = topk_idx ? topk_idx : b.idx;  // written in place when the caller asks
  float* gate_buf = topk_gate ? topk_gate : b.gates;
  const double avg_rows = (double)TK / N;
  const bool expert_stream = fp4 || avg_rows <= 48.0;
  // large-tile path: rows split by gate into a hi + lo class and a bf16 class
  const bool split_rows = !expert_stream && LMOE_HI_TAU > 0;
  uint32_t* masks_hi = split_rows ? b.masks_hi : nullptr;
  launch_topk(b.logits, w.router_bias, T, N, K, idx_buf, gate_buf, b.masks, (float)LMOE_HI_TAU,
              masks_hi, s);
  tm.stop(LATENTMOE_STAGE_TOPK);

  // ---- 3. bucketing ----
  const int rows_per_tile =
      !expert_stream                   ? TILE_ROWS
      : avg_rows <= LMOE_ROWS16_MAX_AVG ? STREAM_ROWS_SMALL
      : avg_rows <= LMOE_ROWS32_MAX_AVG ? STREAM_ROWS_MID
                                        : STREAM_ROWS_BIG;
  const int max_tiles =
      ceil_div(TK, rows_per_tile) + (split_rows ? 2 : 1) * (int)std::min<long long>(N, TK);
  tm.start(LATENTMOE_STAGE_BUCKET);
  const bool fuse_place = TK <= 8192;  // one workgroup places a few thousand rows quickly
  // many mask blocks: count them in chunks on many workgroups first
  const bool chunked = !fuse_place && bucket_chunks(T) >= LMOE_BUCKET_MIN_CHUNKS;
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
#if LMOE_SHARED_FORK_AT == 2
  fork_to(side, h->ev_fork2);
  shared_expert();
#endif

  // ---- 4. wait for z = W_down x (side stream 2) ----
  (void)hipStreamWaitEvent(s, h->ev_join2, 0);

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
    else if (rows_per_tile == STREAM_ROWS_BIG && LMOE_MID_FP4 && gemm_mid_supports(g, fp4))
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
  const bool hi_side = split_rows && LMOE_HI_DOWN_SIDE && !tm.on;
  // the bf16 class's expert-down rows go out as bf16: their rounding enters y_lat times
  // a gate below the class threshold, like that of their bf16 z and h
  const bool og_mix = split_rows && LMOE_OG16;
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
  } else {
    tm.start(LATENTMOE_STAGE_EXPERT_UP);
    launch_expert(pu, EPI_SQRELU_BF16, b.h);
    tm.stop(LATENTMOE_STAGE_EXPERT_UP);
    tm.start(LATENTMOE_STAGE_EXPERT_DOWN);
    launch_expert(pw, og_mix ? EPI_GATE_BF16 : EPI_GATE_F32, og_mix ? (void*)b.og16 : (void*)b.og);
    tm.stop(LATENTMOE_STAGE_EXPERT_DOWN);
  }

  // ---- 7. combine ----
  tm.start(LATENTMOE_STAGE_COMBINE);
  launch_combine(b.og, og_mix ? b.og16 : nullptr, b.row_gate, (float)LMOE_HI_TAU, b.zrow32, b.zrow16, b.inv,
                 T, K, L, b.y_lat, b.y_lat_lo, s);
  tm.stop(LATENTMOE_STAGE_COMBINE);

  // ---- 8. y += W_up y_lat (after the shared expert wrote y) ----
  (void)hipStreamWaitEvent(s, h->ev_join, 0);
  tm.start(LATENTMOE_STAGE_UP_PROJ);
  GemmParams pp = base_params();
  pp.seg[0] = GemmSeg{b.y_lat, w.w_up, L};
  pp.a_lo = proj_fmt != WF_BF16 && LMOE_LOWP_A16 ? nullptr : b.y_lat_lo;
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
  forward_impl(h, x, T, y, topk_idx, topk_gate, s, true);
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
    forward_impl(h, x, T, y, topk_idx, topk_gate, h->cap, false);
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
  const latentmoe_config& c = h->cfg;
  const size_t T = h->last_T, K = c.top_k;
  const void* src = nullptr;
  size_t have = 0;
  switch (which) {
    case LATENTMOE_INTER_Z: src = h->b.z; have = T * c.latent * 2; break;
    case LATENTMOE_INTER_Y_LAT: src = h->b.y_lat; have = T * c.latent * 2; break;
    case LATENTMOE_INTER_COUNTS: src = h->b.counts; have = (size_t)c.n_experts * 4; break;
    case LATENTMOE_INTER_OFFSETS: src = h->b.offsets; have = (size_t)(c.n_experts + 1) * 4; break;
    case LATENTMOE_INTER_ROW_SRC: src = h->b.row_src; have = T * K * 4; break;
    case LATENTMOE_INTER_INV: src = h->b.inv; have = T * K * 4; break;
    case LATENTMOE_INTER_H: src = h->b.h; have = T * K * c.expert_hidden * 2; break;
    case LATENTMOE_INTER_HS_HI: src = h->b.hs_hi; have = T * c.shared_hidden * 2; break;
    case LATENTMOE_INTER_HS_LO: src = h->b.hs_lo; have = T * c.shared_hidden * 2; break;
    case LATENTMOE_INTER_Y_LAT_LO: src = h->b.y_lat_lo; have = T * c.latent * 2; break;
    case LATENTMOE_INTER_Z_LO: src = h->b.z_lo; have = T * c.latent * 2; break;
    case LATENTMOE_INTER_H_LO: src = h->b.h_lo; have = T * K * c.expert_hidden * 2; break;
    default: return LATENTMOE_ERR_INVALID_ARG;
  }
  if (bytes > have) return LATENTMOE_ERR_INVALID_ARG;
  if (bytes == 0) return LATENTMOE_OK;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) == hipSuccess
             ? LATENTMOE_OK
             : LATENTMOE_ERR_HIP;
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
