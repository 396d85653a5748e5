// Mamba-2 checkpoint + replay verification for speculative decoding, and the
// state-writing verification it replaces ("Nemotron 3.5 Super and Lightning",
// serving section).  One 256-thread workgroup per (request, head).
//
// The state of a head is a [P, N] bf16 matrix, 2 P N bytes (16 KB at Super's
// P = 64, N = 128); a verify step reads it once with coalesced 16-byte loads
// (thread = one state row p and a contiguous range of NPT = N / TPR columns,
// TPR = 256 / P threads per row) and keeps it in fp32 registers.  The few records
// of the step (keys and queries of the head's group, its values and decays) are
// staged in LDS as fp32.  Every kernel is HBM-bound on the state: replay reads it,
// the flush reads and writes it once per buffer, the state-writing scheme reads it
// and writes T candidate states per step.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/ssm_replay.h"
#include "common.hpp"

namespace lmoe {

constexpr int SSM_THREADS = 256;
constexpr int SSM_T_MAX = 16;  // tokens per verify: draft plus the verified token
constexpr int SSM_CAP_MAX = 32;

struct SsmArgs {
  int R, T, H, G, cap;
  const uint16_t* ckpt;  // [R, H, P, N]
  uint16_t* ckpt_out;    // flush: [R, H, P, N] (may alias ckpt)
  uint16_t* buf_k;       // [R, cap, G, N]
  uint16_t* buf_v;       // [R, cap, H, P]
  float* buf_a;          // [R, cap, H]
  const int32_t* buf_len;
  const uint16_t* q;     // [R, T, G, N]
  const uint16_t* k;     // [R, T, G, N]
  const uint16_t* v;     // [R, T, H, P]
  const float* a;        // [R, T, H]
  uint16_t* states;      // [R, T, H, P, N]
  float* y;              // [R, T, H, P]
};

// this thread's NPT state values of row p, columns n0 .. n0 + NPT - 1 (fp32)
template <int NPT>
__device__ __forceinline__ void load_row(const uint16_t* src, float (&s)[NPT]) {
#pragma unroll
  for (int i = 0; i < NPT; i += 8) {
    const u32x4_t w = ld128(src + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[i + 2 * e] = __uint_as_float(w[e] << 16);
      s[i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

template <int NPT>
__device__ __forceinline__ void store_row(uint16_t* dst, const float (&s)[NPT]) {
#pragma unroll
  for (int i = 0; i < NPT; i += 8) {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[i + 2 * e], s[i + 2 * e + 1]);
    st128(dst + i, w);
  }
}

// eight bf16 (one 16-byte piece) -> eight fp32 in LDS
__device__ __forceinline__ void to_lds(float* dst, const u32x4_t& w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dst[2 * e] = __uint_as_float(w[e] << 16);
    dst[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

// sum over the TPR consecutive lanes that share a state row (TPR a power of two <= 64)
template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// ---- verify by checkpoint + replay ----
//
// Three small contractions per (request, head), all on the matrix cores:
//   U[p][t]  = sum_n S[p][n] q_t[n]          bf16 MFMA, S straight from HBM into the
//                                              A operand (exact bf16 products, fp32 sums)
//   C[t][j]  = q_t . k_j                      bf16 MFMA from LDS (one wave)
//   y[p][t]  = D[t] U[p][t] + sum_j V[j][p] C[t][j] w[t][j]
//                                              fp32 MFMA (16x16x4), seeded with D U
// where D[t] is the product of the decays from the checkpoint to token t and w[t][j]
// the product of the decays after record j up to token t (0 past token t).  U and y
// share the MFMA output layout (rows p, columns t), so U stays in registers.
// Columns t >= T and records j >= J are zero padding (T <= 16, J <= 32).
template <int P, int N>
__global__ __launch_bounds__(SSM_THREADS) void ssm_verify_kernel(SsmArgs A) {
  constexpr int N8 = N / 8, P8 = P / 8;
  constexpr int QS = N + 8;        // bf16 LDS row of a query / key (16-byte pad)
  constexpr int TILES = P / 16;    // 16-row tiles of the state
  constexpr int TPW = (TILES + 3) / 4;  // tiles per wave
  static_assert(N % 32 == 0 && P % 16 == 0, "MFMA tiles");
  const int r = blockIdx.x / A.H, h = blockIdx.x % A.H;
  const int g = h / (A.H / A.G);
  const bool key_writer = h % (A.H / A.G) == 0;  // one head per group appends the keys
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, gq = lane >> 4;

  const int T = A.T, cap = A.cap;
  // Loads that do not depend on the buffer's record count go first, so that their
  // latency overlaps the count's (a branch on the count would otherwise hold them).
  // ---- state rows of this wave's tiles: A operands of the U products, in flight
  // while the records are staged ----
  u32x4_t sa[TPW][N / 32];
#pragma unroll
  for (int w = 0; w < TPW; ++w) {
    const int tile = wave + 4 * w;
    if (tile < TILES) {
      const uint16_t* row = A.ckpt + (((long long)r * A.H + h) * P + tile * 16 + r16) * N;
#pragma unroll
      for (int st = 0; st < N / 32; ++st) sa[w][st] = ld128(row + 32 * st + 8 * gq);
    }
  }

  // ---- records (16-byte pieces, loads issued before use; the T tokens are appended
  // to the buffer on the way): the drafts first ----
  const long long rq = (long long)r * T;
  constexpr int KQ_IT = (SSM_T_MAX * N8 + SSM_THREADS - 1) / SSM_THREADS;
  constexpr int KB_IT = (SSM_CAP_MAX * N8 + SSM_THREADS - 1) / SSM_THREADS;
  constexpr int V_IT = (SSM_CAP_MAX * P8 + SSM_THREADS - 1) / SSM_THREADS;
  u32x4_t dq[KQ_IT], dk[KQ_IT], bk[KB_IT], vv[V_IT];
#pragma unroll
  for (int u = 0; u < KQ_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < T * N8) {
      const long long src = ((rq + i / N8) * A.G + g) * N + (i % N8) * 8;
      dq[u] = ld128(A.q + src);
      dk[u] = ld128(A.k + src);
    }
  }
  const int len = A.buf_len[r];
  const int J = len + T;  // records up to the last verified token

  if (len < 0 || J > cap) {  // no room: NaN outputs, buffer untouched
    for (int i = tid; i < T * P; i += SSM_THREADS) {
      const int t = i / P, p = i % P;
      A.y[(((long long)r * T + t) * A.H + h) * P + p] = __builtin_nanf("");
    }
    return;
  }

  extern __shared__ __attribute__((aligned(16))) float sm[];
  uint16_t* qb = reinterpret_cast<uint16_t*>(sm);  // [16][QS] bf16, rows >= T zero
  uint16_t* kb = qb + 16 * QS;                       // [32][QS] bf16, rows >= J zero
  float* vs = reinterpret_cast<float*>(kb + 32 * QS); // [32][P] fp32, rows >= J zero
  float* as = vs + 32 * P;                            // [32] decays
  float* coef = as + 32;                              // [16][33] C * w
  float* D = coef + 16 * 33;                          // [16]

#pragma unroll
  for (int u = 0; u < KB_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < len * N8) bk[u] = ld128(A.buf_k + (((long long)r * cap + i / N8) * A.G + g) * N + (i % N8) * 8);
  }
#pragma unroll
  for (int u = 0; u < V_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < J * P8) {
      const int j = i / P8, p = (i % P8) * 8;
      vv[u] = j < len ? ld128(A.buf_v + (((long long)r * cap + j) * A.H + h) * P + p)
                      : ld128(A.v + ((rq + j - len) * A.H + h) * P + p);
    }
  }
  float av = 0.f;
  if (tid < J)
    av = tid < len ? A.buf_a[((long long)r * cap + tid) * A.H + h] : A.a[(rq + tid - len) * A.H + h];

  // zero padding rows (queries t >= T, keys and values j >= J)
  for (int i = tid; i < (16 - T) * N8; i += SSM_THREADS)
    st128(qb + (T + i / N8) * QS + (i % N8) * 8, zero128());
  for (int i = tid; i < (32 - J) * N8; i += SSM_THREADS)
    st128(kb + (J + i / N8) * QS + (i % N8) * 8, zero128());
  for (int i = tid; i < (32 - J) * P; i += SSM_THREADS) vs[J * P + i] = 0.f;
#pragma unroll
  for (int u = 0; u < KQ_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < T * N8) {
      const int t = i / N8, n = (i % N8) * 8;
      if (key_writer) st128(A.buf_k + (((long long)r * cap + len + t) * A.G + g) * N + n, dk[u]);
      st128(kb + (len + t) * QS + n, dk[u]);
      st128(qb + t * QS + n, dq[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < KB_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < len * N8) st128(kb + (i / N8) * QS + (i % N8) * 8, bk[u]);
  }
#pragma unroll
  for (int u = 0; u < V_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < J * P8) {
      const int j = i / P8, p = (i % P8) * 8;
      if (j >= len) st128(A.buf_v + (((long long)r * cap + j) * A.H + h) * P + p, vv[u]);
      to_lds(vs + j * P + p, vv[u]);
    }
  }
  if (tid < J) {
    if (tid >= len) A.buf_a[((long long)r * cap + tid) * A.H + h] = av;
    as[tid] = av;
  }
  __syncthreads();

  // ---- C = Q K^T on wave 0 (two 16-column tiles of records), times the decay
  // weights; D on wave 1 ----
  if (wave == 0) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < N / 32; ++st) {
        const u32x4_t qa = *reinterpret_cast<const u32x4_t*>(qb + r16 * QS + 32 * st + 8 * gq);
        const u32x4_t kbv = *reinterpret_cast<const u32x4_t*>(kb + (16 * jt + r16) * QS + 32 * st + 8 * gq);
        c = mfma_16x16x32(qa, kbv, c);  // rows t, columns j
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * gq + i, j = 16 * jt + r16, pos = len + t;
        float w = 0.f;
        if (t < T && j <= pos) {
          w = 1.f;
          for (int m = j + 1; m <= pos; ++m) w *= as[m];
        }
        coef[t * 33 + j] = c[i] * w;
      }
    }
  } else if (wave == 1 && lane < 16) {
    float w = 1.f;
    if (lane < T)
      for (int m = 0; m <= len + lane; ++m) w *= as[m];
    D[lane] = lane < T ? w : 0.f;
  }

  // ---- U = S Q^T (rows p, columns t) for this wave's tiles ----
  f32x4_t acc[TPW];
#pragma unroll
  for (int w = 0; w < TPW; ++w) {
    acc[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (wave + 4 * w < TILES) {
#pragma unroll
      for (int st = 0; st < N / 32; ++st) {
        const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(qb + r16 * QS + 32 * st + 8 * gq);
        acc[w] = mfma_16x16x32(sa[w][st], qv, acc[w]);
      }
    }
  }
  __syncthreads();

  // ---- y = D U + V^T (C w)^T: fp32 MFMA over the 32 records, 4 per step ----
  const float dt = D[r16];
#pragma unroll
  for (int w = 0; w < TPW; ++w) {
    const int tile = wave + 4 * w;
    if (tile < TILES) {
      f32x4_t y = acc[w] * dt;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int j = 4 * st + gq;
        const float va = vs[j * P + tile * 16 + r16];  // A: row p, k = j
        const float cb = coef[r16 * 33 + j];           // B: k = j, column t
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(va, cb, y, 0, 0, 0);
      }
      // lane: rows p = tile*16 + 4 gq + i, column t = r16
      if (r16 < T) {
        float* dst = A.y + ((rq + r16) * A.H + h) * P + tile * 16 + 4 * gq;
        *reinterpret_cast<f32x4_t*>(dst) = y;
      }
    }
  }
}

// ---- flush: state after the checkpoint and the buffered records, written back ----
template <int P, int N>
__global__ __launch_bounds__(SSM_THREADS) void ssm_flush_kernel(SsmArgs A) {
  constexpr int TPR = SSM_THREADS / P;
  constexpr int NPT = N / TPR;
  constexpr int NS = N + 1;
  const int r = blockIdx.x / A.H, h = blockIdx.x % A.H;
  const int g = h / (A.H / A.G);
  const int tid = threadIdx.x;
  const int cap = A.cap;
  const int len = min(A.buf_len[r], cap);
  if (len <= 0) return;  // checkpoint unchanged

  extern __shared__ float sm[];
  float* ks = sm;              // [cap][NS]
  float* vs = ks + cap * NS;   // [cap][P]
  float* w = vs + cap * P;     // [cap]: decay product after record j
  float* dall = w + cap;       // [1]: decay product over all records
  // records as 16-byte pieces, every load issued before its use
  constexpr int N8 = N / 8, P8 = P / 8;
  constexpr int K_IT = (SSM_CAP_MAX * N8 + SSM_THREADS - 1) / SSM_THREADS;
  constexpr int V_IT = (SSM_CAP_MAX * P8 + SSM_THREADS - 1) / SSM_THREADS;
  u32x4_t kk[K_IT], vv[V_IT];
#pragma unroll
  for (int u = 0; u < K_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < len * N8)
      kk[u] = ld128(A.buf_k + (((long long)r * cap + i / N8) * A.G + g) * N + (i % N8) * 8);
  }
#pragma unroll
  for (int u = 0; u < V_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < len * P8)
      vv[u] = ld128(A.buf_v + (((long long)r * cap + i / P8) * A.H + h) * P + (i % P8) * 8);
  }
  const float aj = tid < len ? A.buf_a[((long long)r * cap + tid) * A.H + h] : 1.f;
  const int p = tid / TPR, n0 = (tid % TPR) * NPT;
  const long long off = (((long long)r * A.H + h) * P + p) * N + n0;
  float s[NPT];
  load_row<NPT>(A.ckpt + off, s);
#pragma unroll
  for (int u = 0; u < K_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < len * N8) to_lds(ks + (i / N8) * NS + (i % N8) * 8, kk[u]);
  }
#pragma unroll
  for (int u = 0; u < V_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < len * P8) to_lds(vs + (i / P8) * P + (i % P8) * 8, vv[u]);
  }
  if (tid < len) w[tid] = aj;  // decays first, turned into suffix products below
  __syncthreads();
  if (tid == 0) {  // w[j] = product of the decays after record j; dall = all of them
    float acc = 1.f;
    for (int j = len - 1; j >= 0; --j) {
      const float aj2 = w[j];
      w[j] = acc;
      acc *= aj2;
    }
    dall[0] = acc;
  }
  __syncthreads();
  const float d = dall[0];
#pragma unroll
  for (int i = 0; i < NPT; ++i) s[i] *= d;
  for (int j = 0; j < len; ++j) {
    const float c = w[j] * vs[j * P + p];
#pragma unroll
    for (int i = 0; i < NPT; ++i) s[i] += c * ks[j * NS + n0 + i];
  }
  store_row<NPT>(A.ckpt_out + off, s);
}

__global__ void ssm_reset_kernel(int R, int32_t* buf_len) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) buf_len[r] = 0;
}

__global__ void ssm_commit_kernel(int R, const int32_t* accepted, int32_t* buf_len) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) buf_len[r] += accepted[r];
}

// ---- the state-writing scheme: every candidate state goes to memory ----
template <int P, int N>
__global__ __launch_bounds__(SSM_THREADS) void ssm_states_kernel(SsmArgs A) {
  constexpr int TPR = SSM_THREADS / P;
  constexpr int NPT = N / TPR;
  constexpr int NS = N + 1;
  const int r = blockIdx.x / A.H, h = blockIdx.x % A.H;
  const int g = h / (A.H / A.G);
  const int tid = threadIdx.x;
  const int T = A.T;
  extern __shared__ float sm[];
  float* qs = sm;             // [T][NS]
  float* ks = qs + T * NS;    // [T][NS]
  float* vs = ks + T * NS;    // [T][P]
  float* as = vs + T * P;     // [T]
  const long long rq = (long long)r * T;
  constexpr int N8 = N / 8, P8 = P / 8;
  constexpr int KQ_IT = (SSM_T_MAX * N8 + SSM_THREADS - 1) / SSM_THREADS;
  constexpr int V_IT = (SSM_T_MAX * P8 + SSM_THREADS - 1) / SSM_THREADS;
  u32x4_t dq[KQ_IT], dk[KQ_IT], vv[V_IT];
#pragma unroll
  for (int u = 0; u < KQ_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < T * N8) {
      const long long src = ((rq + i / N8) * A.G + g) * N + (i % N8) * 8;
      dq[u] = ld128(A.q + src);
      dk[u] = ld128(A.k + src);
    }
  }
#pragma unroll
  for (int u = 0; u < V_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < T * P8) vv[u] = ld128(A.v + ((rq + i / P8) * A.H + h) * P + (i % P8) * 8);
  }
  const float at0 = tid < T ? A.a[(rq + tid) * A.H + h] : 0.f;
  const int p = tid / TPR, n0 = (tid % TPR) * NPT;
  float s[NPT];
  load_row<NPT>(A.ckpt + (((long long)r * A.H + h) * P + p) * N + n0, s);
#pragma unroll
  for (int u = 0; u < KQ_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < T * N8) {
      to_lds(ks + (i / N8) * NS + (i % N8) * 8, dk[u]);
      to_lds(qs + (i / N8) * NS + (i % N8) * 8, dq[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < V_IT; ++u) {
    const int i = tid + u * SSM_THREADS;
    if (i < T * P8) to_lds(vs + (i / P8) * P + (i % P8) * 8, vv[u]);
  }
  if (tid < T) as[tid] = at0;
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const float at = as[t], vt = vs[t * P + p];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      s[i] = at * s[i] + vt * ks[t * NS + n0 + i];
      acc += s[i] * qs[t * NS + n0 + i];
    }
    store_row<NPT>(A.states + ((((rq + t) * A.H + h) * P + p) * N + n0), s);
    acc = row_sum<TPR>(acc);
    if (n0 == 0) A.y[((rq + t) * A.H + h) * P + p] = acc;
  }
}

size_t verify_lds(int P, int N, int T, int cap) {
  (void)T;
  (void)cap;
  return (size_t)(16 + 32) * (N + 8) * 2 + sizeof(float) * ((size_t)32 * P + 32 + 16 * 33 + 16);
}
size_t flush_lds(int P, int N, int cap) {
  return sizeof(float) * ((size_t)cap * (N + 1) + (size_t)cap * P + cap + 1);
}
size_t states_lds(int P, int N, int T) {
  return sizeof(float) * (2 * (size_t)T * (N + 1) + (size_t)T * P + T);
}

// calls f(std::integral_constant<int, P>, std::integral_constant<int, N>) for the shape
template <class F>
bool ssm_dispatch(int P, int N, F&& f) {
  if (P == 64 && N == 64) return f(std::integral_constant<int, 64>{}, std::integral_constant<int, 64>{}), true;
  if (P == 64 && N == 128) return f(std::integral_constant<int, 64>{}, std::integral_constant<int, 128>{}), true;
  if (P == 128 && N == 64) return f(std::integral_constant<int, 128>{}, std::integral_constant<int, 64>{}), true;
  if (P == 128 && N == 128) return f(std::integral_constant<int, 128>{}, std::integral_constant<int, 128>{}), true;
  return false;
}

}  // namespace lmoe

using namespace lmoe;

extern "C" {

int ssm_check_shape(const ssm_shape* s) {
  if (!s) return SSM_ERR_INVALID_ARG;
  if (s->heads <= 0 || s->groups <= 0 || s->head_dim <= 0 || s->state_dim <= 0 || s->capacity <= 0)
    return SSM_ERR_INVALID_ARG;
  if (s->heads % s->groups) return SSM_ERR_UNSUPPORTED;
  if ((s->head_dim != 64 && s->head_dim != 128) || (s->state_dim != 64 && s->state_dim != 128))
    return SSM_ERR_UNSUPPORTED;
  if (s->capacity > SSM_CAP_MAX) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

static int ssm_check_t(const ssm_shape* s, int R, int T) {
  const int st = ssm_check_shape(s);
  if (st != SSM_OK) return st;
  if (R < 0 || T < 1 || T > s->capacity) return SSM_ERR_INVALID_ARG;
  if (T > SSM_T_MAX) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

static SsmArgs ssm_args(const ssm_shape* s, int R, int T) {
  SsmArgs A{};
  A.R = R;
  A.T = T;
  A.H = s->heads;
  A.G = s->groups;
  A.cap = s->capacity;
  return A;
}

int ssm_replay_verify(const ssm_shape* shape, int32_t R, int32_t T, const uint16_t* ckpt,
                      uint16_t* buf_k, uint16_t* buf_v, float* buf_a, const int32_t* buf_len,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* a,
                      float* y, hipStream_t stream) {
  const int st = ssm_check_t(shape, R, T);
  if (st != SSM_OK) return st;
  if (!ckpt || !buf_k || !buf_v || !buf_a || !buf_len || !q || !k || !v || !a || !y)
    return SSM_ERR_INVALID_ARG;
  if (R == 0) return SSM_OK;
  SsmArgs A = ssm_args(shape, R, T);
  A.ckpt = ckpt;
  A.buf_k = buf_k;
  A.buf_v = buf_v;
  A.buf_a = buf_a;
  A.buf_len = buf_len;
  A.q = q;
  A.k = k;
  A.v = v;
  A.a = a;
  A.y = y;
  (void)hipGetLastError();
  const size_t lds = verify_lds(shape->head_dim, shape->state_dim, T, shape->capacity);
  const unsigned grid = (unsigned)((long long)R * shape->heads);
  ssm_dispatch(shape->head_dim, shape->state_dim, [&](auto P, auto N) {
    ssm_verify_kernel<decltype(P)::value, decltype(N)::value><<<grid, SSM_THREADS, lds, stream>>>(A);
  });
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_replay_commit(int32_t R, const int32_t* accepted, int32_t* buf_len, hipStream_t stream) {
  if (R < 0 || !accepted || !buf_len) return SSM_ERR_INVALID_ARG;
  if (R == 0) return SSM_OK;
  (void)hipGetLastError();
  ssm_commit_kernel<<<(R + 255) / 256, 256, 0, stream>>>(R, accepted, buf_len);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_replay_flush(const ssm_shape* shape, int32_t R, uint16_t* ckpt, const uint16_t* buf_k,
                     const uint16_t* buf_v, const float* buf_a, int32_t* buf_len,
                     hipStream_t stream) {
  const int st = ssm_check_shape(shape);
  if (st != SSM_OK) return st;
  if (R < 0 || !ckpt || !buf_k || !buf_v || !buf_a || !buf_len) return SSM_ERR_INVALID_ARG;
  if (R == 0) return SSM_OK;
  SsmArgs A = ssm_args(shape, R, 1);
  A.ckpt = ckpt;
  A.ckpt_out = ckpt;
  A.buf_k = const_cast<uint16_t*>(buf_k);
  A.buf_v = const_cast<uint16_t*>(buf_v);
  A.buf_a = const_cast<float*>(buf_a);
  A.buf_len = buf_len;
  (void)hipGetLastError();
  const size_t lds = flush_lds(shape->head_dim, shape->state_dim, shape->capacity);
  const unsigned grid = (unsigned)((long long)R * shape->heads);
  ssm_dispatch(shape->head_dim, shape->state_dim, [&](auto P, auto N) {
    ssm_flush_kernel<decltype(P)::value, decltype(N)::value><<<grid, SSM_THREADS, lds, stream>>>(A);
  });
  // the counters are reset after every head of the request has read them
  ssm_reset_kernel<<<(R + 255) / 256, 256, 0, stream>>>(R, buf_len);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_states_verify(const ssm_shape* shape, int32_t R, int32_t T, const uint16_t* state,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* a,
                      uint16_t* states_out, float* y, hipStream_t stream) {
  const int st = ssm_check_t(shape, R, T);
  if (st != SSM_OK) return st;
  if (!state || !q || !k || !v || !a || !states_out || !y) return SSM_ERR_INVALID_ARG;
  if (R == 0) return SSM_OK;
  SsmArgs A = ssm_args(shape, R, T);
  A.ckpt = state;
  A.q = q;
  A.k = k;
  A.v = v;
  A.a = a;
  A.states = states_out;
  A.y = y;
  (void)hipGetLastError();
  const size_t lds = states_lds(shape->head_dim, shape->state_dim, T);
  const unsigned grid = (unsigned)((long long)R * shape->heads);
  ssm_dispatch(shape->head_dim, shape->state_dim, [&](auto P, auto N) {
    ssm_states_kernel<decltype(P)::value, decltype(N)::value><<<grid, SSM_THREADS, lds, stream>>>(A);
  });
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
