// Split-K reduction, gated combine, FP4 / FP8 decoders (checks and bf16 expansion).
#include "common.hpp"
#include "epilogue.hpp"
#include "fp4.hpp"
#include "fp8.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace lmoe {

// out[row, n..n+3] = epilogue(sum over splits of partial[s, row, n..n+3])
__global__ void reduce_kernel(GemmParams p) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long groups = (long long)p.M * (p.N / 4);
  if (i >= groups) return;
  const int row = (int)(i / (p.N / 4));
  const int n = (int)(i % (p.N / 4)) * 4;
  const float* src = p.partial + (long long)row * p.N + n;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  // eight independent loads in flight per thread; the sum order is fixed
  for (; s + 8 <= p.splits; s += 8) {
    f32x4_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = *reinterpret_cast<const f32x4_t*>(src + (s + i) * p.partial_stride);
#pragma unroll
    for (int i = 0; i < 8; ++i) v += t[i];
  }
  for (; s < p.splits; ++s) v += *reinterpret_cast<const f32x4_t*>(src + s * p.partial_stride);
  epilogue4(p, 0, 0, row, n, v);
}

void launch_reduce(const GemmParams& p, hipStream_t s) {
  const long long groups = (long long)p.M * (p.N / 4);
  if (groups <= 0) return;
  reduce_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(p);
}

// Decode-sized forward: one GEMM over x with the stacked weight rows
// [router piece 1; piece 2; piece 3; W_down; S1] leaves split-K partials
// [splits][T][NS], NS = 3N + L + MS.  This sums them and splits the columns: the
// three piece columns of expert e add up to its fp32 logit (the pieces sum to the
// fp32 router weight exactly); then z = W_down x leaves as a bf16 pair; then
// h_s = relu(S1 x)^2 leaves as a bf16 pair into columns [L, L + MS) of the rows
// (stride ldh) that the final GEMM [W_up | S2] reads.  One thread per 4 columns
// of logits, z or h_s; splits are summed in order.
__global__ void xreduce_kernel(const float* __restrict__ partial, int splits, long long pstride, int T,
                               int N, int L, int MS, float* __restrict__ logits, uint16_t* __restrict__ z,
                               uint16_t* __restrict__ z_lo, uint16_t* __restrict__ hs,
                               uint16_t* __restrict__ hs_lo, int ldh) {
  const int G = (N + L + MS) / 4;  // output groups per row
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * G) return;
  const int t = (int)(i / G);
  const int c = (int)(i % G) * 4;  // output column in [0, N + L + MS)
  const int NS = 3 * N + L + MS;
  const float* row = partial + (long long)t * NS;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  if (c < N) {
    int s = 0;
    for (; s + 4 <= splits; s += 4) {  // twelve loads in flight; the sum order is fixed
      f32x4_t u[4][3];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) u[i][j] = *reinterpret_cast<const f32x4_t*>(row + (s + i) * pstride + c + j * N);
#pragma unroll
      for (int i = 0; i < 4; ++i) v += u[i][0] + u[i][1] + u[i][2];
    }
    for (; s < splits; ++s) {
      const float* q = row + s * pstride + c;
      v += *reinterpret_cast<const f32x4_t*>(q) + *reinterpret_cast<const f32x4_t*>(q + N) +
           *reinterpret_cast<const f32x4_t*>(q + 2 * N);
    }
    *reinterpret_cast<f32x4_t*>(logits + (long long)t * N + c) = v;
    return;
  }
  const int cc = c + 2 * N;  // partial column of z or h_s
  int s = 0;
  for (; s + 8 <= splits; s += 8) {  // eight loads in flight; the sum order is fixed
    f32x4_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = *reinterpret_cast<const f32x4_t*>(row + (s + i) * pstride + cc);
#pragma unroll
    for (int i = 0; i < 8; ++i) v += u[i];
  }
  for (; s < splits; ++s) v += *reinterpret_cast<const f32x4_t*>(row + s * pstride + cc);
  u32x2_t hi, lo;
  if (c < N + L) {
    epi_pack<EPI_BF16_HILO>(v, hi, lo);
    const long long off = (long long)t * L + (c - N);
    *reinterpret_cast<u32x2_t*>(z + off) = hi;
    *reinterpret_cast<u32x2_t*>(z_lo + off) = lo;
  } else {
    f32x4_t u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float r = fmaxf(v[j], 0.0f);
      u[j] = r * r;
    }
    epi_pack<EPI_SQRELU_HILO>(u, hi, lo);
    const long long off = (long long)t * ldh + (c - N - L);
    *reinterpret_cast<u32x2_t*>(hs + off) = hi;
    *reinterpret_cast<u32x2_t*>(hs_lo + off) = lo;
  }
}

void launch_xreduce(const float* partial, int splits, long long pstride, int T, int N, int L, int MS,
                    float* logits, uint16_t* z, uint16_t* z_lo, uint16_t* hs, uint16_t* hs_lo, int ldh,
                    hipStream_t s) {
  const long long n = (long long)T * ((N + L + MS) / 4);
  if (n <= 0) return;
  xreduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(partial, splits, pstride, T, N, L, MS, logits, z,
                                                             z_lo, hs, hs_lo, ldh);
}

// Gated sum over each token's K expert outputs, in the order of its top-K list
// ("Nemotron 3 Super", section 3.2: the experts' outputs are combined in the
// latent space before the up-projection).  og rows are already multiplied by
// their gate; the sum runs k = 0 .. K-1, so the result does not depend on
// scheduling.  The fp32 sum leaves as a bf16 pair (hi, lo = sum - hi) so the
// up-projection sees it to about 16 significant bits.
//
// MIX (large-tile path with two row classes): a row of the bf16 class (paired = 0)
// was written to og16 as bf16, the others to og as fp32; with no class flags
// (FP4 experts) every row is in og16.  A row costs one 16-byte
// load per thread from its own format's row (the first 8 bytes of a bf16 row's load
// are the thread's 4 values, widened exactly before the add; og16 has 16 bytes of
// slack past its last row): no branches, so the compiler keeps all loads in flight.
template <bool MIX>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ og,
                                                     const uint16_t* __restrict__ og16,
                                                     const uint8_t* __restrict__ paired,
                                                     const int* __restrict__ inv, int K, int L,
                                                     uint16_t* __restrict__ y_lat,
                                                     uint16_t* __restrict__ y_lat_lo, int ldy) {
  __shared__ int pos[64];
  __shared__ int wide[64];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int q = inv[(long long)t * K + threadIdx.x];
    pos[threadIdx.x] = q;
    // the class top-K assigned; MIX without class flags: every row is bf16
    wide[threadIdx.x] = !MIX || (paired && paired[(long long)t * K + threadIdx.x]);
  }
  __syncthreads();
  const int c = (blockIdx.y * 64 + threadIdx.x) * 4;
  if (c >= L) return;
  // row k as four fp32 values (bf16 rows: 4 bf16 in words 0-1, widened at the add)
  auto load = [&](int k) {
    const long long off = (long long)pos[k] * L + c;
    if (!MIX) return *reinterpret_cast<const u32x4_t*>(og + off);
    const uint8_t* src = wide[k] ? reinterpret_cast<const uint8_t*>(og + off)
                                 : reinterpret_cast<const uint8_t*>(og16 + off);
    return *reinterpret_cast<const u32x4_t*>(src);
  };
  auto value = [&](int k, const u32x4_t& v) {
    const f32x4_t bf = {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                        __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
    return !MIX || wide[k] ? __builtin_bit_cast(f32x4_t, v) : bf;
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 24 <= K; k += 24) {  // 24 rows in flight (every row of a top-22 token), summed in k order
    u32x4_t v[24];
#pragma unroll
    for (int i = 0; i < 24; ++i) v[i] = load(k + i);
#pragma unroll
    for (int i = 0; i < 24; ++i) acc += value(k + i, v[i]);
  }
  if (k + 8 <= K) {  // the rest: up to 23 rows, loads first, in k order
    u32x4_t v[23];
    const int r = K - k;
#pragma unroll
    for (int i = 0; i < 23; ++i)
      if (i < r) v[i] = load(k + i);
#pragma unroll
    for (int i = 0; i < 23; ++i)
      if (i < r) acc += value(k + i, v[i]);
    k = K;
  }
  for (; k < K; ++k) acc += value(k, load(k));
  float hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(acc[i]));
    lo[i] = acc[i] - hi[i];
  }
  store_bf16x4(y_lat, (long long)t * ldy + c, hi[0], hi[1], hi[2], hi[3]);
  store_bf16x4(y_lat_lo, (long long)t * ldy + c, lo[0], lo[1], lo[2], lo[3]);
}

void launch_combine(const float* og, const uint16_t* og16, const uint8_t* paired, const int* inv, int T,
                    int K, int L, uint16_t* y_lat, uint16_t* y_lat_lo, int ldy, hipStream_t s) {
  if (T <= 0) return;
  dim3 grid(T, (L / 4 + 63) / 64);
  if (og16)
    combine_kernel<true><<<grid, 64, 0, s>>>(og, og16, paired, inv, K, L, y_lat, y_lat_lo, ldy);
  else
    combine_kernel<false><<<grid, 64, 0, s>>>(og, nullptr, nullptr, inv, K, L, y_lat, y_lat_lo, ldy);
}

// zero n 32-bit words (a kernel rather than a memset node, so that a captured
// graph replays it as an ordinary kernel)
__global__ void zero_kernel(uint32_t* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

void launch_zero(void* p, size_t bytes, hipStream_t s) {
  const long long n = (long long)(bytes / 4);
  if (n <= 0) return;
  zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<uint32_t*>(p), n);
}

// decode n_blocks16 FP4 blocks (8 code bytes + 1 scale byte each) to bf16
__global__ void fp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                   const uint8_t* __restrict__ scales, long long nb,
                                   uint16_t* __restrict__ out) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const u32x2_t c = *reinterpret_cast<const u32x2_t*>(codes + 8 * b);
  const float sc = fp8x2_to_f32<false>(scales[b]).x;
  st128(out + 16 * b, fp4x8_to_bf16(c[0], sc));
  st128(out + 16 * b + 8, fp4x8_to_bf16(c[1], sc));
}

void launch_fp4_dequant(const uint8_t* codes, const uint8_t* scales, long long n_blocks16,
                        uint16_t* out, hipStream_t s) {
  if (n_blocks16 <= 0) return;
  fp4_dequant_kernel<<<(unsigned)((n_blocks16 + 255) / 256), 256, 0, s>>>(codes, scales,
                                                                          n_blocks16, out);
}

// decode n_groups16 groups of 16 E4M3 bytes to bf16
__global__ void fp8_dequant_kernel(const uint8_t* __restrict__ codes, long long ng,
                                   uint16_t* __restrict__ out) {
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ng) return;
  const u32x4_t c = ld128(codes + 16 * g);
  st128(out + 16 * g, fp8x8_to_bf16(c[0], c[1]));
  st128(out + 16 * g + 8, fp8x8_to_bf16(c[2], c[3]));
}

void launch_fp8_dequant(const uint8_t* codes, long long n_groups16, uint16_t* out, hipStream_t s) {
  if (n_groups16 <= 0) return;
  fp8_dequant_kernel<<<(unsigned)((n_groups16 + 255) / 256), 256, 0, s>>>(codes, n_groups16, out);
}

// Strided copy with zero fill, in units of U bytes: dst has `slices` slices of
// drows rows of dcols units; element (s, i, j) is src[(s srows + i) spitch + j] when
// i < rows and j < cols, else 0.  Widths that are not multiples of 64 run on
// zero-padded copies (weights once, tokens per call), and the output is cropped.
template <typename U>
__global__ void pad_copy_kernel(const U* __restrict__ src, long long spitch, int srows, U* __restrict__ dst,
                                long long dcols, int drows, int rows, long long cols, long long total) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long j = i % dcols;
    const long long r = i / dcols;
    const int row = (int)(r % drows);
    const long long sl = r / drows;
    dst[i] = row < rows && j < cols ? src[(sl * srows + row) * spitch + j] : U(0);
  }
}

void launch_pad_copy(const void* src, size_t spitch, int srows, void* dst, size_t dpitch, int drows,
                     long long slices, int rows, size_t cols, hipStream_t s) {
  const bool words = spitch % 4 == 0 && dpitch % 4 == 0 && cols % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(src) % 4 == 0 && reinterpret_cast<uintptr_t>(dst) % 4 == 0;
  const size_t u = words ? 4 : 1;
  const long long total = slices * (long long)drows * (long long)(dpitch / u);
  if (total <= 0) return;
  const unsigned blocks = (unsigned)std::min<long long>((total + 255) / 256, 65536);
  if (words)
    pad_copy_kernel<uint32_t><<<blocks, 256, 0, s>>>(static_cast<const uint32_t*>(src), (long long)(spitch / 4),
                                                     srows, static_cast<uint32_t*>(dst), (long long)(dpitch / 4),
                                                     drows, rows, (long long)(cols / 4), total);
  else
    pad_copy_kernel<uint8_t><<<blocks, 256, 0, s>>>(static_cast<const uint8_t*>(src), (long long)spitch, srows,
                                                    static_cast<uint8_t*>(dst), (long long)dpitch, drows, rows,
                                                    (long long)cols, total);
}

}  // namespace lmoe
