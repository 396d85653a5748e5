// Routing kernels: router weight split, top-K + softmax, expert bucketing.
//
// Gating runs at the full model width d and picks K of N experts per token
// ("Nemotron 3 Super", section 3.2: the gating network stays in dimension d;
// section 3.1 table: 512 experts, top-22).  Selection order is (-logit, index):
// equal logits go to the lower expert index.  Gates are a softmax over the K
// selected logits.
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {

// ---------------------------------------------------------------------------
// router weight split: w = hi + mid + lo exactly, each piece a bf16 (truncated
// 8-bit significands).  x (bf16) times each piece is exact in fp32, so the
// logits come from exact products accumulated in fp32.
// ---------------------------------------------------------------------------
__global__ void router_split_kernel(const float* __restrict__ w, uint16_t* __restrict__ pieces,
                                    long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = w[i];
  uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
  float r1 = v - __uint_as_float(hb);
  uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
  float r2 = r1 - __uint_as_float(mb);
  uint32_t lb = __float_as_uint(r2) & 0xFFFF0000u;  // r2 has <= 8 significant bits
  pieces[i] = (uint16_t)(hb >> 16);
  pieces[n + i] = (uint16_t)(mb >> 16);
  pieces[2 * n + i] = (uint16_t)(lb >> 16);
}

void launch_router_split(const float* w, uint16_t* pieces, long long n, hipStream_t s) {
  router_split_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w, pieces, n);
}

// ---------------------------------------------------------------------------
// top-K: one wavefront per token.  Logit e lives in lane e % 64, slot e / 64,
// as an order-preserving unsigned key.  The K-th largest key tau is found by a
// 32-step bisection whose counts are wave ballots; the experts above tau and
// the lowest-index experts equal to tau (ties go to the lower index) form the
// selection, which is then ranked by (-logit, index) for the output order.
// ---------------------------------------------------------------------------
constexpr int TOPK_TOKENS_PER_BLOCK = 16;  // one wave each; masks are 16 bits wide

__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal logits must tie
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// number of set bits of m in lanes below this one
__device__ __forceinline__ int bits_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int SLOTS>
__global__ __launch_bounds__(1024) void topk_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int N,
                                                    int K, int* __restrict__ idx_out,
                                                    float* __restrict__ gate_out,
                                                    uint32_t* __restrict__ masks) {
  __shared__ uint32_t smask[1024];
  __shared__ unsigned long long cand[TOPK_TOKENS_PER_BLOCK][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * TOPK_TOKENS_PER_BLOCK + w;
  for (int e = threadIdx.x; e < N; e += blockDim.x) smask[e] = 0u;
  __syncthreads();

  if (t < T) {
    uint32_t ok[SLOTS];  // orderable logit; 0 marks an empty slot
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int e = j * 64 + lane;
      ok[j] = 0u;
      if (e < N) ok[j] = orderable(logits[(long long)t * N + e] + (bias ? bias[e] : 0.0f));
    }
    // tau = the largest key with at least K keys >= it (the K-th largest key)
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = tau | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) cnt += __popcll(__ballot(ok[j] >= c));
      if (cnt >= K) tau = c;
    }
    int n_gt = 0;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) n_gt += __popcll(__ballot(ok[j] > tau));
    // selection in index order (slot-major, then lane): keys above tau, then
    // the first K - n_gt keys equal to tau
    const int need = K - n_gt;
    int eq_before = 0, base = 0;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const unsigned long long eqm = __ballot(ok[j] == tau);
      const bool take = ok[j] > tau || (ok[j] == tau && eq_before + bits_below(eqm) < need);
      eq_before += __popcll(eqm);
      const unsigned long long sm = __ballot(take);
      if (take)
        cand[w][base + bits_below(sm)] =
            ((unsigned long long)ok[j] << 32) | (uint32_t)(~(uint32_t)(j * 64 + lane));
      base += __popcll(sm);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // rank of each selected key: keys are unique (index in the low half)
    unsigned long long mine = 0ull, top = 0ull;
    int rank = 0;
    if (lane < K) mine = cand[w][lane];
    for (int c = 0; c < K; ++c) {
      const unsigned long long o = cand[w][c];
      rank += o > mine;
      top = o > top ? o : top;
    }
    const float v = from_orderable((uint32_t)(mine >> 32));
    const float vmax = from_orderable((uint32_t)(top >> 32));
    const float ex = lane < K ? expf(v - vmax) : 0.0f;
    const float tot = wave_sum(ex);
    if (lane < K) {
      const int e = (int)(~(uint32_t)mine);
      idx_out[(long long)t * K + rank] = e;
      gate_out[(long long)t * K + rank] = ex / tot;
      atomicOr(&smask[e], 1u << w);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) masks[(long long)blockIdx.x * N + e] = smask[e];
}

void launch_topk(const float* logits, const float* bias, int T, int N, int K, int* idx,
                 float* gates, uint32_t* masks, hipStream_t s) {
  const int blocks = (T + TOPK_TOKENS_PER_BLOCK - 1) / TOPK_TOKENS_PER_BLOCK;
  if (N <= 512)
    topk_kernel<8><<<blocks, 64 * TOPK_TOKENS_PER_BLOCK, 0, s>>>(logits, bias, T, N, K, idx, gates, masks);
  else
    topk_kernel<16><<<blocks, 64 * TOPK_TOKENS_PER_BLOCK, 0, s>>>(logits, bias, T, N, K, idx, gates, masks);
}

// ---------------------------------------------------------------------------
// bucketing.  Permuted order is (expert, token): rows of expert e occupy
// [offsets[e], offsets[e+1]) sorted by token.  The rank of token t inside
// expert e is a prefix over 16-token blocks plus a popcount inside the block,
// so the order is deterministic.  One workgroup, thread e owns expert e.
// ---------------------------------------------------------------------------
struct PlaceArgs {  // fused placement (small T): see place_kernel
  const int* idx;
  const float* gates;
  int T, K;
  int* row_src;
  float* row_gate;
  int* inv;
};

__device__ __forceinline__ void place_one(long long i, const int* __restrict__ idx,
                                          const float* __restrict__ gates,
                                          const uint32_t* __restrict__ masks,
                                          const int* __restrict__ offsets,
                                          const int* __restrict__ block_prefix, int N, int K,
                                          int* __restrict__ row_src, float* __restrict__ row_gate,
                                          int* __restrict__ inv) {
  const int t = (int)(i / K);
  const int e = idx[i];
  const int b = t / TOPK_TOKENS_PER_BLOCK;
  const int tl = t % TOPK_TOKENS_PER_BLOCK;
  const uint32_t m = masks[(long long)b * N + e];
  const int pos = offsets[e] + block_prefix[(long long)b * N + e] + __popc(m & ((1u << tl) - 1u));
  row_src[pos] = t;
  row_gate[pos] = gates[i];
  inv[i] = pos;
}

__global__ __launch_bounds__(1024) void bucket_scan_kernel(
    const uint32_t* __restrict__ masks, int nblk, int N, int tile_rows_max, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ block_prefix, int* __restrict__ tile_expert,
    int* __restrict__ tile_row0, int* __restrict__ tile_rows, int* __restrict__ n_tiles,
    int max_tiles, PlaceArgs pa) {
  __shared__ int scan_a[1024];
  __shared__ int scan_b[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N) {
    int b = 0;
    for (; b + 4 <= nblk; b += 4) {
      uint32_t m0 = masks[(long long)(b + 0) * N + e];
      uint32_t m1 = masks[(long long)(b + 1) * N + e];
      uint32_t m2 = masks[(long long)(b + 2) * N + e];
      uint32_t m3 = masks[(long long)(b + 3) * N + e];
      block_prefix[(long long)(b + 0) * N + e] = run; run += __popc(m0);
      block_prefix[(long long)(b + 1) * N + e] = run; run += __popc(m1);
      block_prefix[(long long)(b + 2) * N + e] = run; run += __popc(m2);
      block_prefix[(long long)(b + 3) * N + e] = run; run += __popc(m3);
    }
    for (; b < nblk; ++b) {
      uint32_t m = masks[(long long)b * N + e];
      block_prefix[(long long)b * N + e] = run;
      run += __popc(m);
    }
    counts[e] = run;
  }
  const int ntile_e = (e < N) ? (run + tile_rows_max - 1) / tile_rows_max : 0;
  // two inclusive scans at once (rows and tiles), Hillis-Steele over the block
  scan_a[e] = (e < N) ? run : 0;
  scan_b[e] = ntile_e;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int a = scan_a[e], bb = scan_b[e];
    if (e >= off) { a += scan_a[e - off]; bb += scan_b[e - off]; }
    __syncthreads();
    scan_a[e] = a;
    scan_b[e] = bb;
    __syncthreads();
  }
  const int row_start = scan_a[e] - ((e < N) ? run : 0);
  const int tile_start = scan_b[e] - ntile_e;
  if (e < N) {
    offsets[e] = row_start;
    for (int i = 0; i < ntile_e; ++i) {
      const int j = tile_start + i;
      if (j < max_tiles) {
        tile_expert[j] = e;
        tile_row0[j] = row_start + i * tile_rows_max;
        tile_rows[j] = min(tile_rows_max, run - i * tile_rows_max);
      }
    }
  }
  if (e == 0) {
    offsets[N] = scan_a[1023];
    n_tiles[0] = min(scan_b[1023], max_tiles);
  }
  if (pa.idx) {  // small T: the same workgroup places every (token, k)
    __syncthreads();
    const long long n = (long long)pa.T * pa.K;
    for (long long i = threadIdx.x; i < n; i += blockDim.x)
      place_one(i, pa.idx, pa.gates, masks, offsets, block_prefix, N, pa.K, pa.row_src, pa.row_gate,
                pa.inv);
  }
}

void launch_bucket_scan(const uint32_t* masks, int T, int N, int tile_rows_max, int* counts,
                        int* offsets, int* block_prefix, int* tile_expert, int* tile_row0,
                        int* tile_rows, int* n_tiles, int max_tiles, const int* place_idx,
                        const float* place_gates, int K, int* row_src, float* row_gate, int* inv,
                        hipStream_t s) {
  const int nblk = (T + TOPK_TOKENS_PER_BLOCK - 1) / TOPK_TOKENS_PER_BLOCK;
  PlaceArgs pa{place_idx, place_gates, T, K, row_src, row_gate, inv};
  bucket_scan_kernel<<<1, 1024, 0, s>>>(masks, nblk, N, tile_rows_max, counts, offsets,
                                        block_prefix, tile_expert, tile_row0, tile_rows, n_tiles,
                                        max_tiles, pa);
}

__global__ void place_kernel(const int* __restrict__ idx, const float* __restrict__ gates,
                             const uint32_t* __restrict__ masks, const int* __restrict__ offsets,
                             const int* __restrict__ block_prefix, int T, int N, int K,
                             int* __restrict__ row_src, float* __restrict__ row_gate,
                             int* __restrict__ inv) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * K) return;
  place_one(i, idx, gates, masks, offsets, block_prefix, N, K, row_src, row_gate, inv);
}

void launch_place(const int* idx, const float* gates, const uint32_t* masks, const int* offsets,
                  const int* block_prefix, int T, int N, int K, int* row_src, float* row_gate,
                  int* inv, hipStream_t s) {
  const long long n = (long long)T * K;
  place_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(idx, gates, masks, offsets,
                                                           block_prefix, T, N, K, row_src,
                                                           row_gate, inv);
}

}  // namespace lmoe
