/*
 * ssm_replay.h -- C ABI of the Mamba-2 checkpoint + replay verification step for
 * speculative decoding, on AMD Instinct MI355X (gfx950).
 *
 * The method ("Nemotron 3.5 Super and Lightning", serving section, on where the
 * throughput comes from): a Mamba layer keeps one fixed-size state per head and
 * every token updates it as  S <- a S + v k^T  (a decay, k a key, v a value); the
 * token's output is  y = S q  (q its query).  Verifying a speculative draft of T
 * tokens would write T candidate states to memory.  Instead one state is kept as
 * a checkpoint and each later token only appends its (k, v, a) record to a small
 * buffer; the output at buffer position p is the query times the checkpoint,
 * scaled by the product of the decays since the checkpoint, plus, for every record
 * j <= p, v_j times (q . k_j) times the product of the decays after record j.
 * After verification only the accepted tokens stay in the buffer (the count
 * advances by the number accepted; rejected drafts are overwritten by the next
 * append).  When the buffer is full the state is materialised once and written
 * back as the new checkpoint.  The state-writing scheme it replaces is also
 * offered (ssm_states_verify) so that both can be measured.
 *
 * Shapes ("Nemotron 3 Super", section 3.1 table): H heads of dimension P, state
 * dimension N, G groups; the heads h with h / (H / G) == g share group g's key and
 * query.  Readings of what the pages leave open:
 *   - the state of head h is a [P, N] matrix, S <- a S + v k^T with v the head's
 *     P-vector and k its group's N-vector; a token's output is taken after its own
 *     update;
 *   - states are stored as bf16 (the pages' 16-bit Mamba state), records as bf16
 *     keys and values with fp32 decays; all arithmetic is fp32;
 *   - the verified tokens are appended to the buffer by the verify call itself.
 *
 * Layouts (row-major; "device" = HIP device memory of the current device):
 *   ckpt / state  [R, H, P, N] bf16       one state per request and head
 *   buf_k         [R, cap, G, N] bf16     buffered keys
 *   buf_v         [R, cap, H, P] bf16     buffered values
 *   buf_a         [R, cap, H] fp32        buffered decays
 *   buf_len       [R] int32               records in each request's buffer
 *   q, k          [R, T, G, N] bf16       the verified tokens' queries and keys
 *   v             [R, T, H, P] bf16       their values
 *   a             [R, T, H] fp32          their decays
 *   y             [R, T, H, P] fp32       their outputs
 * bf16 tensors are passed as raw 16-bit patterns.  All calls are asynchronous on
 * `stream`, allocate nothing and return a status (0 = ok).  Errors (returned before
 * anything is enqueued): SSM_ERR_INVALID_ARG for a null pointer, R < 0, T < 1 or
 * T > capacity; SSM_ERR_UNSUPPORTED for a shape outside the one checked by
 * ssm_check_shape; SSM_ERR_HIP when a launch fails.
 */
#ifndef SSM_REPLAY_H_
#define SSM_REPLAY_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_OK 0
#define SSM_ERR_INVALID_ARG (-1)
#define SSM_ERR_UNSUPPORTED (-2)
#define SSM_ERR_HIP (-4)

typedef struct {
  int32_t heads;     /* H                                                   */
  int32_t groups;    /* G, divides H                                        */
  int32_t head_dim;  /* P: 64 or 128                                        */
  int32_t state_dim; /* N: 64 or 128                                        */
  int32_t capacity;  /* records per buffer between checkpoints, 1 .. 32     */
} ssm_shape;

/* OK if the kernels handle the shape (host pointer), else UNSUPPORTED (or
 * INVALID_ARG for a null pointer or non-positive sizes). */
int ssm_check_shape(const ssm_shape* shape);

/* Verify T tokens of each of R requests by checkpoint + replay: appends the
 * tokens' records (k, v, a) to each buffer at positions buf_len[r] .. + T - 1 and
 * writes their outputs y.  ckpt is read only.  A request whose buf_len[r] is
 * negative or leaves fewer than T free records gets NaN outputs and its buffer is
 * left unchanged.  buf_len is not changed (see ssm_replay_commit). */
int ssm_replay_verify(const ssm_shape* shape, int32_t R, int32_t T, const uint16_t* ckpt,
                      uint16_t* buf_k, uint16_t* buf_v, float* buf_a, const int32_t* buf_len,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* a,
                      float* y, hipStream_t stream);

/* buf_len[r] += accepted[r] for r < R (device int32 arrays): keeps the first
 * accepted[r] of the records the last verify appended; the caller guarantees
 * 0 <= accepted[r] <= T of that verify. */
int ssm_replay_commit(int32_t R, const int32_t* accepted, int32_t* buf_len, hipStream_t stream);

/* Materialise each request's state from its checkpoint and its buf_len[r]
 * buffered records, write it over ckpt (bf16, round to nearest even) and set
 * buf_len[r] = 0.  Requests with an empty buffer keep their checkpoint. */
int ssm_replay_flush(const ssm_shape* shape, int32_t R, uint16_t* ckpt, const uint16_t* buf_k,
                     const uint16_t* buf_v, const float* buf_a, int32_t* buf_len,
                     hipStream_t stream);

/* The scheme replay avoids: from the current state of each request, run the T
 * tokens through the recurrence, write every candidate state (states_out
 * [R, T, H, P, N] bf16, state after token t) and the outputs y (computed from the
 * fp32 running state).  state is read only. */
int ssm_states_verify(const ssm_shape* shape, int32_t R, int32_t T, const uint16_t* state,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* a,
                      uint16_t* states_out, float* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_REPLAY_H_ */
