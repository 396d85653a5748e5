/*
 * latentmoe.h -- C ABI of the LatentMoE layer forward for AMD Instinct MI355X (gfx950).
 *
 * The layer ("Nemotron 3 Super: Open, Efficient Mixture-of-Experts Hybrid
 * Mamba-Transformer Model for Agentic Reasoning", section 3.2 LatentMoE): every
 * token x in R^d gets router logits over N experts at the full width d and a
 * top-K selection; it is projected by W_down (l x d) into the latent space,
 * run through its K selected experts in latent width (each expert l -> m -> l),
 * the gated sum is projected back by W_up (d x l) and added to a full-width
 * shared expert (d -> m_s -> d).  Shapes of the Super model are in the same
 * page's section 3.1 table; expert weights may be stored in the block-scaled
 * 4-bit format of section 3.6 (per-tensor and per-block scales) with E2M1
 * elements and E4M3 block scales ("Nemotron 3 Ultra", NVFP4 description).
 *
 * Readings of points the pages leave open (fixed by this library):
 *   - router: fp32 logits l = W_r x (+ b), the K largest logits with ties going
 *     to the lower expert index, gates = softmax over the K selected logits;
 *   - experts: two matrices per expert with a squared-ReLU activation,
 *     o = W2 relu(W1 z)^2; the shared expert has the same form at width d and
 *     is added without a gate; no biases or norms inside the layer;
 *   - FP4 weights: one E4M3FN scale per 16 consecutive input-dim elements and
 *     one fp32 scale per matrix; element 2j in the low nibble of byte j;
 *   - FP8 weights: E4M3FN elements and one fp32 scale per matrix.
 *
 * Conventions: all matrices are row-major; a weight [out, in] computes
 * y = x * W^T.  bf16 tensors are passed as raw 16-bit patterns.  Every pointer
 * argument named "device" is HIP device memory of the current device; "host"
 * pointers are ordinary host memory.  No function throws or aborts; each
 * returns a status code (LATENTMOE_OK == 0 on success).
 */
#ifndef LATENTMOE_H_
#define LATENTMOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define LATENTMOE_OK 0
#define LATENTMOE_ERR_INVALID_ARG (-1)  /* null pointer, bad size, T > max_tokens, ... */
#define LATENTMOE_ERR_UNSUPPORTED (-2)  /* shape outside what the kernels handle      */
#define LATENTMOE_ERR_OUT_OF_MEMORY (-3) /* workspace allocation failed               */
#define LATENTMOE_ERR_HIP (-4)          /* a HIP runtime call or kernel launch failed */
#define LATENTMOE_ERR_SCRATCH (-5)      /* workspace larger than the static scratch array */

/* ---- weight storage formats ----
 * BF16: raw bf16 patterns.
 * FP4_E2M1_E4M3_B16: block-scaled 4-bit ("Nemotron 3 Super", section 3.6: a
 *   per-tensor and a per-block scale; "Nemotron 3 Ultra": E2M1 elements, E4M3
 *   block scales): w = e2m1(code) * e4m3fn(block scale) * tensor scale, one
 *   block scale per 16 consecutive input-dim elements, element 2j in the low
 *   nibble of byte j.
 * FP8_E4M3: one E4M3FN byte per element times one fp32 tensor scale.
 * Which matrices may use which format follows the released precision mix
 * ("Nemotron 3.5 Super and Lightning", section on keeping accuracy under
 * 4-bit quantisation: experts and shared expert in NVFP4, other projections in
 * FP8); FP8 for the latent projections W_down / W_up is this library's reading,
 * the pages do not name their precision. */
#define LATENTMOE_FORMAT_BF16 0
#define LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 1
#define LATENTMOE_FORMAT_FP8_E4M3 2
#define LATENTMOE_EXPERTS_BF16 LATENTMOE_FORMAT_BF16
#define LATENTMOE_EXPERTS_FP4_E2M1_E4M3_B16 LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16

typedef struct latentmoe_handle_s* latentmoe_handle_t;

/* Layer shape (host struct).  Requirements, checked by latentmoe_init:
 * d, latent, expert_hidden, shared_hidden multiples of 16 (the FP4 block; the
 * kernels run widths in multiples of 64, and other widths run zero-padded to
 * the next multiple of 64, see latentmoe_init); n_experts a multiple of 16 and
 * at most 4096; 1 <= top_k <= min(n_experts, 64); max_tokens >= 1; the
 * activation matrices the kernels address with 32-bit offsets stay below 2^31
 * elements at the widths the kernels run: max_tokens * top_k * max(latent,
 * expert_hidden) and max_tokens * max(d, shared_hidden) (at the Super shapes,
 * d = 4096, l = 1024, m = 2688, m_s = 5376, K = 22: max_tokens <= 36314). */
typedef struct {
  int32_t d;             /* model width                                   */
  int32_t latent;        /* latent width l                                */
  int32_t n_experts;     /* N                                             */
  int32_t top_k;         /* K                                             */
  int32_t expert_hidden; /* m (each expert l -> m -> l)                   */
  int32_t shared_hidden; /* m_s (shared expert d -> m_s -> d)             */
  int32_t max_tokens;    /* largest T a forward call may pass             */
  int32_t expert_format; /* experts W1, W2: FORMAT_BF16 | FORMAT_FP4_...  */
  int32_t shared_format; /* shared S1, S2: FORMAT_BF16 | FORMAT_FP4_...   */
  int32_t proj_format;   /* W_down, W_up: FORMAT_BF16 | FORMAT_FP8_E4M3   */
} latentmoe_config;

/* Weights (host struct holding device pointers).  The library BORROWS every
 * buffer: it must stay allocated and unchanged until latentmoe_destroy (with a
 * width that is not a multiple of 64, init copies the matrices and reads the
 * caller's matrices only during the call; the bias and the per-tensor scales
 * stay borrowed).
 * Alignment: every pointer 16-byte aligned. */
typedef struct {
  const float* router_w;          /* [N, d] fp32                                  */
  const float* router_bias;       /* [N] fp32, or NULL for no bias                */
  const void* w_down;             /* bf16 [l, d]     | FP8 codes u8 [l, d]        */
  const void* w_up;               /* bf16 [d, l]     | FP8 codes u8 [d, l]        */
  const void* expert_w1;          /* bf16 [N, m, l]  | FP4 codes u8 [N, m, l/2]   */
  const void* expert_w2;          /* bf16 [N, l, m]  | FP4 codes u8 [N, l, m/2]   */
  const uint8_t* expert_w1_scale; /* FP4 only: E4M3FN [N, m, l/16], else NULL     */
  const uint8_t* expert_w2_scale; /* FP4 only: E4M3FN [N, l, m/16], else NULL     */
  const float* expert_w1_tscale;  /* FP4 only: fp32 [N], else NULL                */
  const float* expert_w2_tscale;  /* FP4 only: fp32 [N], else NULL                */
  const void* shared_w1;          /* bf16 [m_s, d]   | FP4 codes u8 [m_s, d/2]    */
  const void* shared_w2;          /* bf16 [d, m_s]   | FP4 codes u8 [d, m_s/2]    */
  const uint8_t* shared_w1_scale; /* FP4 shared only: E4M3FN [m_s, d/16]          */
  const uint8_t* shared_w2_scale; /* FP4 shared only: E4M3FN [d, m_s/16]          */
  const float* shared_w1_tscale;  /* FP4 shared only: fp32 [1]                    */
  const float* shared_w2_tscale;  /* FP4 shared only: fp32 [1]                    */
  const float* w_down_tscale;     /* FP8 projections only: fp32 [1]               */
  const float* w_up_tscale;       /* FP8 projections only: fp32 [1]               */
} latentmoe_weights;

/* Create a layer handle.  Validates the shape and pointers, allocates the
 * workspace for cfg->max_tokens tokens (device memory owned by the handle) and
 * derives the router's split weights on `stream`.  With max_tokens above 64
 * and an FP4 shared expert or FP8 projections, it also writes the exact bf16
 * values of those matrices (block scale applied, tensor scale not) into the
 * workspace on `stream`: dense GEMMs of more than 64 tokens run on the
 * LDS-tiled kernel, which reads bf16 weights; up to 64 tokens the stored
 * format is streamed and decoded in registers.  No other work is enqueued.
 * The call waits for that work to finish (it synchronises `stream`) before it
 * returns, so the handle may be used on any stream afterwards.
 * cfg, w: host pointers, read during the call only.  out: host pointer that
 * receives the handle (set to NULL on failure).
 * Errors: INVALID_ARG (null pointer, including a scale pointer that the
 * chosen format needs), UNSUPPORTED (shape requirements above, a format not
 * offered for that matrix), OUT_OF_MEMORY (the workspace allocation failed;
 * LATENTMOE_FAIL_ALLOC=1 in the environment forces this, for tests), HIP.
 * With bf16 projections and shared expert the workspace also holds stacked
 * copies of [router pieces; W_down; S1] and [W_up | S2] for forwards of at most
 * 64 tokens, which run on `stream` alone.  Larger forwards fork two side
 * streams of the default priority from `stream` (W_down; the shared expert);
 * LATENTMOE_SERIAL=1 in the environment at init keeps every stage of this
 * handle on `stream` in program order (per-kernel profiling).
 * Widths that are not multiples of 64 (d, latent, expert_hidden or
 * shared_hidden): init allocates zero-padded copies of every weight matrix at
 * the widths rounded up to 64 (D, L, M, M_s; device memory owned by the handle,
 * about the weights' size again; the padded rows and columns add exact zeros,
 * so the layer's results are those of the caller's widths) and a [max_tokens, D]
 * bf16 and a [max_tokens, D] fp32 buffer, and makes the copies on `stream`;
 * each forward then also copies x into the first buffer and crops y out of the
 * second (two kernels on the forward's stream). */
int latentmoe_init(const latentmoe_config* cfg, const latentmoe_weights* w, hipStream_t stream,
                   latentmoe_handle_t* out);

/* LatentMoE forward for T tokens, enqueued on `stream`, asynchronous: no host
 * synchronisation and no allocation happen inside.
 *   x         device, [T, d] bf16 tokens
 *   y         device, [T, d] fp32 output (fully overwritten)
 *   topk_idx  device, [T, K] int32 selected experts, largest logit first (ties
 *             to the lower index), or NULL
 *   topk_gate device, [T, K] fp32 gates in the same order, or NULL
 * T == 0 returns OK and enqueues nothing.  Errors (returned before anything is
 * enqueued): INVALID_ARG for a null handle/x/y, T < 0 or T > max_tokens;
 * HIP if a launch fails.  Calls that share a handle must not overlap: the
 * workspace is per handle (use one handle per concurrent stream). */
int latentmoe_forward(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y,
                      int32_t* topk_idx, float* topk_gate, hipStream_t stream);

/* Same contract and results as latentmoe_forward, replayed as a HIP graph.
 * The first call for a given (x, T, y, topk_idx, topk_gate) captures the whole
 * forward (all its streams) into a graph and instantiates it; that call
 * allocates graph resources.  Later calls with the same arguments only
 * enqueue hipGraphLaunch on `stream`, which removes the per-kernel launch
 * gaps of a serving loop; the buffers' contents may change between calls.
 * Different arguments replace the cached graph.  Errors as latentmoe_forward,
 * plus HIP when capture or instantiation fails.  Stage timing does not apply
 * to graph replays. */
int latentmoe_forward_graph(latentmoe_handle_t h, const uint16_t* x, int32_t T, float* y,
                            int32_t* topk_idx, float* topk_gate, hipStream_t stream);

/* Entry point that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same layer as latentmoe_init + latentmoe_forward, all
 * of it on `stream` in program order, without a handle.  It keeps no stacked
 * weight copies, so the router, W_down and the shared expert run as their own
 * GEMMs (the handle runs the GEMMs over x as one launch): outputs agree with
 * latentmoe_forward to rounding (max difference ~1e-5 of rms(y)), top-K sets
 * equal and gates within ~1e-6 unless two logits tie to rounding.  The workspace
 * for T tokens is laid out in a file-scope device array of
 * LATENTMOE_STATIC_SCRATCH_BYTES bytes (64 MiB, enough for T = 64 at the Super
 * decode shapes), which each GPU the library runs on holds until the process
 * ends.  Each call derives the router's split weights into that array, clears
 * what must start at zero (with kernels, no memset nodes) and enqueues the
 * forward; it calls no hipMalloc, hipFree or other allocating routine.  The
 * first call on a device looks up that device's address of the array
 * (hipGetSymbolAddress, not a stream operation) and sets kernel attributes.
 *   cfg, w     host pointers, read during the call; every format must be
 *              FORMAT_BF16 and every width a multiple of 64 (the FP4 / FP8
 *              paths and the padded widths need derived copies larger than
 *              the array); cfg->max_tokens bounds T
 *   x, T, y, topk_idx, topk_gate, stream: as latentmoe_forward
 * All calls on one GPU share its array and the array keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two threads) race and
 * must not be made.  Errors (before anything is enqueued): INVALID_ARG (null
 * pointers, T < 0, T > cfg->max_tokens), UNSUPPORTED (shape checks of
 * latentmoe_init, a format other than bf16, a width that is not a multiple of
 * 64), SCRATCH (the workspace for T
 * tokens exceeds LATENTMOE_STATIC_SCRATCH_BYTES), HIP. */
#define LATENTMOE_STATIC_SCRATCH_BYTES (64u << 20)
int latentmoe_forward_static(const latentmoe_config* cfg, const latentmoe_weights* w,
                             const uint16_t* x, int32_t T, float* y, int32_t* topk_idx,
                             float* topk_gate, hipStream_t stream);

/* Free the handle and its workspace.  Work still queued on a stream that uses
 * the handle must have completed.  NULL is accepted (returns OK). */
int latentmoe_destroy(latentmoe_handle_t h);

/* Static description of a status code (never NULL). */
const char* latentmoe_status_string(int status);

/* Bytes of device workspace latentmoe_init would allocate for cfg (host
 * pointers), including the padded copies of widths that are not multiples of
 * 64.  Errors as latentmoe_init's shape checks. */
int latentmoe_workspace_bytes(const latentmoe_config* cfg, size_t* bytes);

/* Intermediates of the last forward on this handle, for tests and tools.
 * Copies `bytes` bytes of intermediate `which` into device buffer dst on
 * `stream` (asynchronous).  Layouts for the last call's T, at the caller's
 * widths (padded widths are cropped):
 *   LATENTMOE_INTER_Z        [T, l] bf16       latent tokens W_down x
 *   LATENTMOE_INTER_Y_LAT    [T, l] bf16       gated expert sum (latent), high part
 *   LATENTMOE_INTER_Y_LAT_LO [T, l] bf16       gated expert sum, remainder
 *   LATENTMOE_INTER_COUNTS   [N] int32         tokens routed to each expert
 *   LATENTMOE_INTER_OFFSETS  [N+1] int32       first permuted row of each expert
 *   LATENTMOE_INTER_ROW_SRC  [T*K] int32       token of each permuted row
 *   LATENTMOE_INTER_INV      [T*K] int32       permuted row of (t, k)
 *   LATENTMOE_INTER_H        [T*K, m] bf16     expert hidden activations (permuted)
 *   LATENTMOE_INTER_HS_HI    [T, m_s] bf16     shared hidden, high part
 *   LATENTMOE_INTER_HS_LO    [T, m_s] bf16     shared hidden, remainder
 *   LATENTMOE_INTER_Z_LO     [T, l] bf16       latent tokens, remainder
 *   LATENTMOE_INTER_H_LO     [T*K, m] bf16     expert hidden, remainder
 *   LATENTMOE_INTER_PAIRED   [T, K] uint8      large-tile path only: 1 where the
 *                                              routed row (t, k) carries hi + lo
 * Permuted order: the rows of expert e are [OFFSETS[e], OFFSETS[e+1]), sorted
 * by token.  When the layer runs its large-tile path (bf16 experts and more
 * than 48 routed rows per expert on average, T*K/N > 48), each token's rows
 * with the largest gates are "paired": in top-K order (largest gate first),
 * row k is paired unless sum_{j >= k} g_j^2 <= sum_j g_j^2 / 32 (fp32, sums over
 * the token's K rows).  The paired rows of each expert come first (sorted by
 * token), then the others (sorted by token): only the first group carries z,
 * h and the gated expert output as hi + lo pairs or fp32, the others as bf16
 * (H_LO is not written for them).  GEMMs with FP4 or
 * FP8 weights take single bf16 activations (weight-only quantisation, 16-bit
 * activations): with FP4 experts H_LO is not written, with an FP4 shared expert
 * HS_LO is not written, and FP8 projections read Y_LAT but not Y_LAT_LO.
 * Errors: INVALID_ARG for an unknown `which`, a null pointer or more bytes
 * than the intermediate holds. */
#define LATENTMOE_INTER_Z 0
#define LATENTMOE_INTER_Y_LAT 1
#define LATENTMOE_INTER_COUNTS 2
#define LATENTMOE_INTER_OFFSETS 3
#define LATENTMOE_INTER_ROW_SRC 4
#define LATENTMOE_INTER_INV 5
#define LATENTMOE_INTER_H 6
#define LATENTMOE_INTER_HS_HI 7
#define LATENTMOE_INTER_HS_LO 8
#define LATENTMOE_INTER_Y_LAT_LO 9
#define LATENTMOE_INTER_Z_LO 10
#define LATENTMOE_INTER_H_LO 11
#define LATENTMOE_INTER_PAIRED 12
int latentmoe_debug_copy(latentmoe_handle_t h, int which, void* dst, size_t bytes,
                         hipStream_t stream);

/* Stage timing with HIP events recorded on the stream each stage runs on.
 * latentmoe_profile_begin reserves events for up to max_calls forward calls
 * (host allocation of HIP events; call it outside any timed or captured
 * region); every later latentmoe_forward records one start/stop pair for each
 * stage whose bit (1 << LATENTMOE_STAGE_*) is set in stage_mask.  While
 * recording, a forward runs every stage in program order on the caller's
 * stream (no side streams), so a stage's time is that of its own kernels; its
 * outputs are the same as those of an untimed call.
 * latentmoe_profile_end synchronises those events, writes the summed
 * milliseconds of each stage to stage_ms (host, n_stages entries, order of
 * LATENTMOE_STAGE_*), the number of recorded calls to *calls (host), and
 * stops recording (stages outside the mask report 0).  Errors: INVALID_ARG
 * (null handle/pointers, max_calls < 1), HIP. */
#define LATENTMOE_STAGE_ROUTER 0      /* router logits GEMM                       */
#define LATENTMOE_STAGE_TOPK 1        /* top-K + softmax                          */
#define LATENTMOE_STAGE_BUCKET 2      /* counts, offsets, permutation             */
#define LATENTMOE_STAGE_DOWN_PROJ 3   /* z = W_down x                             */
#define LATENTMOE_STAGE_EXPERT_UP 4   /* h = relu(W1_e z)^2, grouped               */
#define LATENTMOE_STAGE_EXPERT_DOWN 5 /* g * W2_e h, grouped                       */
#define LATENTMOE_STAGE_COMBINE 6     /* y_lat = sum_k                            */
#define LATENTMOE_STAGE_SHARED_UP 7   /* h_s = relu(S1 x)^2                       */
#define LATENTMOE_STAGE_SHARED_DOWN 8 /* y = S2 h_s                               */
#define LATENTMOE_STAGE_UP_PROJ 9     /* y += W_up (y_lat hi + lo)                */
#define LATENTMOE_NUM_STAGES 10
int latentmoe_profile_begin(latentmoe_handle_t h, int max_calls, uint32_t stage_mask);
int latentmoe_profile_end(latentmoe_handle_t h, float* stage_ms, int n_stages, int* calls);

/* Decode n_blocks block-scaled FP4 blocks with the same in-register decoder
 * the expert GEMMs use: codes (device, n_blocks * 8 bytes, element 2j in the
 * low nibble of byte j), scales (device, n_blocks E4M3FN bytes) -> out (device,
 * n_blocks * 16 bf16).  The per-tensor scale is not applied.  Asynchronous on
 * `stream`.  Errors: INVALID_ARG (null pointers, n_blocks < 0), HIP. */
int latentmoe_fp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t n_blocks,
                         uint16_t* out, hipStream_t stream);

/* Decode n_groups groups of 16 E4M3FN bytes (device, n_groups * 16 bytes) to
 * bf16 (device, n_groups * 16 values, every finite E4M3 value is a bf16 number)
 * with the in-register decoder of the FP8 weight path; the tensor scale is not
 * applied.  Asynchronous on `stream`.  Errors: INVALID_ARG (null pointers,
 * n_groups < 0), HIP. */
int latentmoe_fp8_decode(const uint8_t* codes, int64_t n_groups, uint16_t* out,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LATENTMOE_H_ */
