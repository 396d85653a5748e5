// Routing kernels: router weight split, top-K + softmax, expert bucketing.
//
// Gating runs at the full model width d and picks K of N experts per token
// ("Nemotron 3 Super", section 3.2: the gating network stays in dimension d;
// section 3.1 table: 512 experts, top-22).  Selection order is (-logit, index):
// equal logits go to the lower expert index.  Gates are a softmax over the K
// selected logits.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

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
constexpr int TOPK_TOKENS_PER_BLOCK = 16;  // tokens per mask group: masks are 16 bits wide
// Top-K runs TOPK_WAVES tokens (one wave each) per workgroup, so a mask group is
// written by 16 / TOPK_WAVES workgroups on as many CUs: the bisection is a chain of
// scalar ballot counts, and a CU has one scalar unit for all its waves (16 tokens
// on one CU took ~16 us at 64 tokens).  Each workgroup owns one byte of the group's
// mask word for expert e: byte s holds tokens 4s .. 4s + 3 in its low 4 bits, and
// readers unpack the word with mask16().
constexpr int TOPK_WAVES = 4;
static_assert(TOPK_TOKENS_PER_BLOCK == 4 * TOPK_WAVES, "four workgroups of four tokens per mask group");

__device__ __forceinline__ uint32_t mask16(uint32_t w) {
  return (w & 0xFu) | ((w >> 4) & 0xF0u) | ((w >> 8) & 0xF00u) | ((w >> 12) & 0xF000u);
}

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
__global__ __launch_bounds__(64 * TOPK_WAVES) void topk_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int N,
                                                    int K, int* __restrict__ idx_out,
                                                    float* __restrict__ gate_out,
                                                    uint32_t* __restrict__ masks, float tail_frac,
                                                    uint32_t* __restrict__ masks_hi,
                                                    uint8_t* __restrict__ paired_out) {
  __shared__ uint32_t smask[SLOTS * 64];
  __shared__ uint32_t smask_hi[SLOTS * 64];
  __shared__ unsigned long long cand[TOPK_WAVES][64];
  __shared__ float esq[TOPK_WAVES][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * TOPK_WAVES + w;  // workgroups past T only write zero bytes
  for (int e = threadIdx.x; e < N; e += blockDim.x) smask[e] = smask_hi[e] = 0u;
  __syncthreads();

  if (t < T) {
    // every load is issued before the first use (clamped index, no per-slot branch):
    // guarded loads were each waited for on their own, a chain of global round trips
    const float* __restrict__ row = logits + (long long)t * N;
    float lv[SLOTS], bv[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) lv[j] = row[min(j * 64 + lane, N - 1)];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) bv[j] = 0.0f;
    if (bias) {
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) bv[j] = bias[min(j * 64 + lane, N - 1)];
    }
    uint32_t ok[SLOTS];  // orderable logit; 0 marks an empty slot
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) ok[j] = j * 64 + lane < N ? orderable(lv[j] + bv[j]) : 0u;
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
    const float gate = lane < K ? ex / tot : 0.0f;
    // Rows that carry a bf16 hi + lo pair on the large-tile path: the largest gates
    // of the token, until the rows left out hold at most tail_frac of its gate
    // energy sum_k g_k^2 (a row's bf16 rounding reaches the latent sum scaled by
    // its gate).  Row i is left out iff the energy of the rows ranked at or after
    // it is at most tail_frac times the total; both sums run over the candidates
    // in index order, so every lane sees the same total.
    bool paired = true;
    if (masks_hi) {
      esq[w][lane] = gate * gate;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float total = 0.0f, tail = 0.0f;
      for (int c = 0; c < K; ++c) {
        const float ec = esq[w][c];
        total += ec;
        tail += cand[w][c] <= mine ? ec : 0.0f;
      }
      paired = tail > tail_frac * total;
    }
    if (lane < K) {
      const int e = (int)(~(uint32_t)mine);
      idx_out[(long long)t * K + rank] = e;
      gate_out[(long long)t * K + rank] = gate;
      atomicOr(&smask[e], 1u << w);
      if (masks_hi) {
        if (paired) atomicOr(&smask_hi[e], 1u << w);
        paired_out[(long long)t * K + rank] = paired ? 1 : 0;
      }
    }
  }
  __syncthreads();
  // this workgroup's byte of each mask word of its group
  const long long grp = blockIdx.x / (TOPK_TOKENS_PER_BLOCK / TOPK_WAVES);
  const int byte = blockIdx.x % (TOPK_TOKENS_PER_BLOCK / TOPK_WAVES);
  uint8_t* m8 = reinterpret_cast<uint8_t*>(masks);
  uint8_t* mh8 = reinterpret_cast<uint8_t*>(masks_hi);
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    m8[(grp * N + e) * 4 + byte] = (uint8_t)smask[e];
    if (masks_hi) mh8[(grp * N + e) * 4 + byte] = (uint8_t)smask_hi[e];
  }
}

void launch_topk(const float* logits, const float* bias, int T, int N, int K, int* idx,
                 float* gates, uint32_t* masks, float tail_frac, uint32_t* masks_hi, uint8_t* paired,
                 hipStream_t s) {
  // whole mask groups: every byte of every group's words is written
  const int blocks = (T + TOPK_TOKENS_PER_BLOCK - 1) / TOPK_TOKENS_PER_BLOCK * (TOPK_TOKENS_PER_BLOCK / TOPK_WAVES);
  // each lane holds N / 64 keys (rounded up to 8, 16, 32 or 64)
  auto go = [&](auto slots) {
    topk_kernel<decltype(slots)::value><<<blocks, 64 * TOPK_WAVES, 0, s>>>(
        logits, bias, T, N, K, idx, gates, masks, tail_frac, masks_hi, paired);
  };
  if (N <= 512)
    go(std::integral_constant<int, 8>{});
  else if (N <= 1024)
    go(std::integral_constant<int, 16>{});
  else if (N <= 2048)
    go(std::integral_constant<int, 32>{});
  else
    go(std::integral_constant<int, 64>{});
}

// ---------------------------------------------------------------------------
// bucketing.  Permuted order is (expert, class, token): rows of expert e occupy
// [offsets[e], offsets[e+1]); with a second mask (rows whose gate reaches a
// threshold: the "hi" class) those rows come first, each class sorted by
// token, and every tile holds rows of one class; hi tiles of all experts come
// first in the tile list (n_tiles[0] of them), then the other tiles
// (n_tiles[1]).  Without the second mask every row is in the hi class.  The
// rank of token t inside its class is a prefix over 16-token blocks plus a
// popcount inside the block, so the order is deterministic.  One workgroup,
// thread e owns expert e.
// ---------------------------------------------------------------------------
struct PlaceArgs {  // fused placement (small T): see place_kernel
  const int* idx;
  const float* gates;
  int T, K;
  int* row_src;
  float* row_gate;
  int* inv;
};

// Large T splits the prefix over mask groups in chunks of BK_CHUNK groups: one
// workgroup per chunk counts it (prefixes inside the chunk), the scan turns the
// chunk counts into offsets, and a row's position adds its chunk's offset.  (One
// workgroup walking 512 groups per expert was a chain of 32 rounds of loads, ~55 us
// alone and ~220 us beside the shared expert's GEMMs at 8192 tokens.)
constexpr int BK_CHUNK = 16;

struct BucketMasks {
  const uint32_t* all;      // [nblk, N] rows of each expert per 16-token block
  const uint32_t* hi;       // [nblk, N] the hi-class subset, or null (all rows are hi)
  int* prefix_hi;           // [nblk, N] hi rows of expert e in blocks before b (of its chunk)
  int* prefix_lo;           // [nblk, N] the other rows likewise (used with hi)
  int* counts_hi;           // [N]
  const int* chunk_hi;      // [nchunk, N] hi rows of expert e in chunks before c, or null
  const int* chunk_lo;      // [nchunk, N] the other rows likewise
};

__device__ __forceinline__ void place_one(long long i, const int* __restrict__ idx,
                                          const float* __restrict__ gates, const BucketMasks& bm,
                                          const int* __restrict__ offsets, int N, int K,
                                          int* __restrict__ row_src, float* __restrict__ row_gate,
                                          int* __restrict__ inv) {
  const int t = (int)(i / K);
  const int e = idx[i];
  const int b = t / TOPK_TOKENS_PER_BLOCK;
  const int tl = t % TOPK_TOKENS_PER_BLOCK;
  const long long be = (long long)b * N + e;
  const uint32_t below = (1u << tl) - 1u;
  const uint32_t m = mask16(bm.all[be]);
  const long long ce = (long long)(b / BK_CHUNK) * N + e;
  int pos;
  if (!bm.hi) {
    pos = offsets[e] + bm.prefix_hi[be] + __popc(m & below);
    if (bm.chunk_hi) pos += bm.chunk_hi[ce];
  } else {
    const uint32_t mh = mask16(bm.hi[be]);
    if ((mh >> tl) & 1u) {
      pos = offsets[e] + bm.prefix_hi[be] + __popc(mh & below);
      if (bm.chunk_hi) pos += bm.chunk_hi[ce];
    } else {
      pos = offsets[e] + bm.counts_hi[e] + bm.prefix_lo[be] + __popc(m & ~mh & below);
      if (bm.chunk_hi) pos += bm.chunk_lo[ce];
    }
  }
  row_src[pos] = t;
  row_gate[pos] = gates[i];
  inv[i] = pos;
}

// chunk c = blockIdx.x: prefixes inside the chunk and the chunk's counts per expert
template <bool HI>
__global__ __launch_bounds__(256) void bucket_count_kernel(BucketMasks bm, int nblk, int N,
                                                           int* __restrict__ chunk_hi,
                                                           int* __restrict__ chunk_lo) {
  const int b0 = blockIdx.x * BK_CHUNK;
  const int nb = min(BK_CHUNK, nblk - b0);
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    uint32_t m[BK_CHUNK], mh[BK_CHUNK];
#pragma unroll
    for (int u = 0; u < BK_CHUNK; ++u) {
      m[u] = mh[u] = 0u;
      if (u < nb) {
        m[u] = mask16(bm.all[(long long)(b0 + u) * N + e]);
        if constexpr (HI) mh[u] = mask16(bm.hi[(long long)(b0 + u) * N + e]);
        else mh[u] = m[u];
      }
    }
    int run_hi = 0, run_lo = 0;
#pragma unroll
    for (int u = 0; u < BK_CHUNK; ++u) {
      if (u < nb) {
        const long long be = (long long)(b0 + u) * N + e;
        bm.prefix_hi[be] = run_hi;
        run_hi += __popc(mh[u]);
        if constexpr (HI) {
          bm.prefix_lo[be] = run_lo;
          run_lo += __popc(m[u] & ~mh[u]);
        }
      }
    }
    chunk_hi[(long long)blockIdx.x * N + e] = run_hi;
    if constexpr (HI) chunk_lo[(long long)blockIdx.x * N + e] = run_lo;
  }
}

// nchunk > 0: the prefixes inside chunks and the chunk counts are in place (from
// bucket_count_kernel); the counts become exclusive chunk offsets here.  Thread t
// owns the EPT experts t EPT .. t EPT + EPT - 1 (N <= 1024 EPT).
// LP (fused placement of a small batch, every (token, k) item by this workgroup):
// the per-(mask group, expert) words stay in LDS, (prefix << 16) | 16-bit mask of
// the hi class (all rows without classes), then (prefix_lo << 16) | mask of all rows
// with classes, beside the expert offsets and hi counts; each thread's items' expert
// and gate are loaded at the start, so placing costs no global round trip.
constexpr int LP_ITEMS = 8;  // items per thread: T * K <= 8192 on the fused path
template <bool HI>
constexpr int lp_words_per_entry() { return HI ? 2 : 1; }

template <bool HI, int EPT, bool LP>
__global__ __launch_bounds__(1024) void bucket_scan_kernel(
    BucketMasks bm, int nblk, int N, int tile_rows_max, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ tile_expert, int* __restrict__ tile_row0,
    int* __restrict__ tile_rows, int* __restrict__ n_tiles, int max_tiles, PlaceArgs pa,
    int nchunk, int* __restrict__ chunk_hi, int* __restrict__ chunk_lo) {
  __shared__ int scan_a[16];  // wave totals
  __shared__ int scan_b[16];
  __shared__ int scan_c[16];
  extern __shared__ uint32_t lp_words[];  // LP: [words per entry][nblk][N], offsets [N + 1], hi counts [N]
  int* const lp_off = reinterpret_cast<int*>(lp_words + lp_words_per_entry<HI>() * nblk * N);
  int* const lp_cnt = lp_off + N + 1;
  const int tid = threadIdx.x;
  const int n_items = pa.T * pa.K;
  int it_e[LP ? LP_ITEMS : 1];
  float it_g[LP ? LP_ITEMS : 1];
  if constexpr (LP) {  // clamped, unconditional: all in flight together
#pragma unroll
    for (int r = 0; r < LP_ITEMS; ++r) {
      const int i = min(tid + r * 1024, n_items - 1);
      it_e[r] = pa.idx[i];
      it_g[r] = pa.gates[i];
    }
  }
  // rows of each of this thread's experts in the two classes
  int rh[EPT], rl[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int e = tid * EPT + x;
    int run_hi = 0, run_lo = 0;
    if (e < N && nchunk > 0) {
      for (int c0 = 0; c0 < nchunk; c0 += 16) {  // 16 chunk counts in flight
        int ch[16], cl[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          ch[u] = cl[u] = 0;
          if (c0 + u < nchunk) {
            ch[u] = chunk_hi[(long long)(c0 + u) * N + e];
            if constexpr (HI) cl[u] = chunk_lo[(long long)(c0 + u) * N + e];
          }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (c0 + u < nchunk) {
            chunk_hi[(long long)(c0 + u) * N + e] = run_hi;
            run_hi += ch[u];
            if constexpr (HI) {
              chunk_lo[(long long)(c0 + u) * N + e] = run_lo;
              run_lo += cl[u];
            }
          }
        }
      }
    } else if (e < N) {
      // U blocks of masks in flight per step (16, then 4, then 1): the loads do
      // not wait on the prefix
      int b = 0;
      auto steps = [&](auto UC, int b_end) {
        constexpr int U = decltype(UC)::value;
        for (; b + U <= b_end; b += U) {
          uint32_t m[U], mh[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            m[u] = mask16(bm.all[(long long)(b + u) * N + e]);
            if constexpr (HI) mh[u] = mask16(bm.hi[(long long)(b + u) * N + e]);
            else mh[u] = m[u];
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const long long be = (long long)(b + u) * N + e;
            if constexpr (LP) {
              lp_words[be] = ((uint32_t)run_hi << 16) | mh[u];
              if constexpr (HI) lp_words[(long long)nblk * N + be] = ((uint32_t)run_lo << 16) | m[u];
            } else {
              bm.prefix_hi[be] = run_hi;
              if constexpr (HI) bm.prefix_lo[be] = run_lo;
            }
            run_hi += __popc(mh[u]);
            if constexpr (HI) run_lo += __popc(m[u] & ~mh[u]);
          }
        }
      };
      steps(std::integral_constant<int, 16>{}, nblk);
      steps(std::integral_constant<int, 4>{}, nblk);
      steps(std::integral_constant<int, 1>{}, nblk);
    }
    if (e < N) {
      if constexpr (HI) bm.counts_hi[e] = run_hi;
      if constexpr (LP && HI) lp_cnt[e] = run_hi;
      counts[e] = run_hi + run_lo;
    }
    rh[x] = run_hi;
    rl[x] = run_lo;
  }
  // this thread's totals: rows, hi tiles, other tiles
  int run = 0, nt_hi = 0, nt_lo = 0;
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    run += rh[x] + rl[x];
    nt_hi += (rh[x] + tile_rows_max - 1) / tile_rows_max;
    nt_lo += (rl[x] + tile_rows_max - 1) / tile_rows_max;
  }
  // inclusive scans at once (rows, hi tiles, other tiles): inside each wave by
  // cross-lane shifts, then the exclusive prefix of the 16 wave totals
  const int lane = tid & 63, wv = tid >> 6;
  int a = run, bb = nt_hi, cs = HI ? nt_lo : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ua = __shfl_up(a, off), ub = __shfl_up(bb, off);
    const int uc = HI ? __shfl_up(cs, off) : 0;
    if (lane >= off) {
      a += ua;
      bb += ub;
      cs += uc;
    }
  }
  if (lane == 63) {
    scan_a[wv] = a;
    scan_b[wv] = bb;
    scan_c[wv] = cs;
  }
  __syncthreads();
  int tot_a = 0, tot_b = 0, tot_c = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w == wv) {
      a += tot_a;
      bb += tot_b;
      cs += tot_c;
    }
    tot_a += scan_a[w];
    tot_b += scan_b[w];
    tot_c += scan_c[w];
  }
  const int total_hi = tot_b;
  const int total_lo = HI ? tot_c : 0;
  // this thread's first row, hi tile and other tile; then its experts in order
  int row_start = a - run;
  int hi_start = bb - nt_hi;
  int lo_start = HI ? total_hi + cs - nt_lo : 0;
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int e = tid * EPT + x;
    if (e >= N) break;
    const int run_hi = rh[x], run_lo = rl[x];
    const int eh = (run_hi + tile_rows_max - 1) / tile_rows_max;
    const int el = (run_lo + tile_rows_max - 1) / tile_rows_max;
    offsets[e] = row_start;
    if constexpr (LP) lp_off[e] = row_start;
    for (int i = 0; i < eh; ++i) {
      const int j = hi_start + i;
      if (j < max_tiles) {
        tile_expert[j] = e;
        tile_row0[j] = row_start + i * tile_rows_max;
        tile_rows[j] = min(tile_rows_max, run_hi - i * tile_rows_max);
      }
    }
    for (int i = 0; HI && i < el; ++i) {
      const int j = lo_start + i;
      if (j < max_tiles) {
        tile_expert[j] = e;
        tile_row0[j] = row_start + run_hi + i * tile_rows_max;
        tile_rows[j] = min(tile_rows_max, run_lo - i * tile_rows_max);
      }
    }
    row_start += run_hi + run_lo;
    hi_start += eh;
    lo_start += el;
  }
  if (tid == 0) {
    offsets[N] = tot_a;
    const int nh = min(total_hi, max_tiles);
    n_tiles[0] = nh;                                        // hi tiles: [0, n_tiles[0])
    n_tiles[1] = min(total_hi + total_lo, max_tiles) - nh;  // then n_tiles[1] others
  }
  if constexpr (LP) {  // the same workgroup places every (token, k), from LDS
    __syncthreads();
#pragma unroll
    for (int r = 0; r < LP_ITEMS; ++r) {
      const int i = tid + r * 1024;
      if (i >= n_items) break;
      const int t = i / pa.K, e = it_e[r];
      const int tl = t % TOPK_TOKENS_PER_BLOCK;
      const long long be = (long long)(t / TOPK_TOKENS_PER_BLOCK) * N + e;
      const uint32_t below = (1u << tl) - 1u;
      const uint32_t w = lp_words[be], mh = w & 0xFFFFu;
      int pos = lp_off[e];
      if (!HI || ((mh >> tl) & 1u)) {
        pos += (int)(w >> 16) + __popc(mh & below);
      } else {
        const uint32_t w1 = lp_words[(long long)nblk * N + be];
        pos += lp_cnt[e] + (int)(w1 >> 16) + __popc(w1 & ~mh & below & 0xFFFFu);
      }
      pa.row_src[pos] = t;
      pa.row_gate[pos] = it_g[r];
      pa.inv[i] = pos;
    }
  } else if (pa.idx) {  // small T: the same workgroup places every (token, k)
    __syncthreads();
    const long long n = (long long)pa.T * pa.K;
    for (long long i = threadIdx.x; i < n; i += blockDim.x)
      place_one(i, pa.idx, pa.gates, bm, offsets, N, pa.K, pa.row_src, pa.row_gate, pa.inv);
  }
}

int bucket_chunks(int T) {
  const int nblk = (T + TOPK_TOKENS_PER_BLOCK - 1) / TOPK_TOKENS_PER_BLOCK;
  return (nblk + BK_CHUNK - 1) / BK_CHUNK;
}

void launch_bucket_scan(const uint32_t* masks, const uint32_t* masks_hi, int T, int N,
                        int tile_rows_max, int* counts, int* counts_hi, int* offsets,
                        int* prefix_hi, int* prefix_lo, int* tile_expert, int* tile_row0,
                        int* tile_rows, int* n_tiles, int max_tiles, const int* place_idx,
                        const float* place_gates, int K, int* row_src, float* row_gate, int* inv,
                        int* chunk_hi, int* chunk_lo, hipStream_t s) {
  const int nblk = (T + TOPK_TOKENS_PER_BLOCK - 1) / TOPK_TOKENS_PER_BLOCK;
  const int nchunk = chunk_hi ? bucket_chunks(T) : 0;
  PlaceArgs pa{place_idx, place_gates, T, K, row_src, row_gate, inv};
  BucketMasks bm{masks, masks_hi, prefix_hi, prefix_lo, counts_hi, nullptr, nullptr};
  auto scan = [&](auto hi, auto ept) {
    constexpr bool HI = decltype(hi)::value;
    constexpr int EPT = decltype(ept)::value;
    if (nchunk) bucket_count_kernel<HI><<<nchunk, 256, 0, s>>>(bm, nblk, N, chunk_hi, chunk_lo);
    // placement from LDS when the batch's words, offsets and counts fit in 64 KB
    const long long lp_bytes = 4LL * ((long long)lp_words_per_entry<HI>() * nblk * N + 2 * N + 1);
    const bool lp = place_idx && !nchunk && (long long)T * K <= 1024LL * LP_ITEMS && T < 65536 &&
                    lp_bytes <= 65536;
    if (lp)
      bucket_scan_kernel<HI, EPT, true><<<1, 1024, (size_t)lp_bytes, s>>>(
          bm, nblk, N, tile_rows_max, counts, offsets, tile_expert, tile_row0, tile_rows, n_tiles, max_tiles,
          pa, nchunk, chunk_hi, chunk_lo);
    else
      bucket_scan_kernel<HI, EPT, false><<<1, 1024, 0, s>>>(
          bm, nblk, N, tile_rows_max, counts, offsets, tile_expert, tile_row0, tile_rows, n_tiles, max_tiles,
          pa, nchunk, chunk_hi, chunk_lo);
  };
  // experts per scan thread: N <= 1024, 2048, 4096
  auto by_n = [&](auto hi) {
    if (N <= 1024)
      scan(hi, std::integral_constant<int, 1>{});
    else if (N <= 2048)
      scan(hi, std::integral_constant<int, 2>{});
    else
      scan(hi, std::integral_constant<int, 4>{});
  };
  if (masks_hi)
    by_n(std::true_type{});
  else
    by_n(std::false_type{});
}

__global__ void place_kernel(const int* __restrict__ idx, const float* __restrict__ gates,
                             BucketMasks bm, const int* __restrict__ offsets, int T, int N, int K,
                             int* __restrict__ row_src, float* __restrict__ row_gate,
                             int* __restrict__ inv) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * K) return;
  place_one(i, idx, gates, bm, offsets, N, K, row_src, row_gate, inv);
}

void launch_place(const int* idx, const float* gates, const uint32_t* masks,
                  const uint32_t* masks_hi, const int* offsets, const int* counts_hi,
                  const int* prefix_hi, const int* prefix_lo, int T, int N, int K, int* row_src,
                  float* row_gate, int* inv, const int* chunk_hi, const int* chunk_lo, hipStream_t s) {
  const long long n = (long long)T * K;
  BucketMasks bm{masks, masks_hi, const_cast<int*>(prefix_hi), const_cast<int*>(prefix_lo),
                 const_cast<int*>(counts_hi), chunk_hi, chunk_lo};
  place_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(idx, gates, bm, offsets, T, N, K,
                                                           row_src, row_gate, inv);
}

}  // namespace lmoe
