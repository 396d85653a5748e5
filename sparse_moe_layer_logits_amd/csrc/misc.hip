// Split-K reduction, gated combine, FP4 / FP8 decoders (checks and bf16 expansion).
#include "common.hpp"
#include "epilogue.hpp"
#include "fp4.hpp"
#include "fp8.hpp"
#include "kernels.hpp"

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

// Gated sum over each token's K expert outputs, in the order of its top-K list
// ("Nemotron 3 Super", section 3.2: the experts' outputs are combined in the
// latent space before the up-projection).  og rows are already multiplied by
// their gate; the sum runs k = 0 .. K-1, so the result does not depend on
// scheduling.  The fp32 sum leaves as a bf16 pair (hi, lo = sum - hi) so the
// up-projection sees it to about 16 significant bits.
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ og,
                                                     const int* __restrict__ inv, int K, int L,
                                                     uint16_t* __restrict__ y_lat,
                                                     uint16_t* __restrict__ y_lat_lo) {
  __shared__ int pos[64];
  const int t = blockIdx.x;
  if (threadIdx.x < K) pos[threadIdx.x] = inv[(long long)t * K + threadIdx.x];
  __syncthreads();
  const int c = (blockIdx.y * 64 + threadIdx.x) * 4;
  if (c >= L) return;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= K; k += 8) {  // eight loads in flight, summed in k order
    f32x4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4_t*>(og + (long long)pos[k + i] * L + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i];
  }
  for (; k < K; ++k) acc += *reinterpret_cast<const f32x4_t*>(og + (long long)pos[k] * L + c);
  float hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(acc[i]));
    lo[i] = acc[i] - hi[i];
  }
  store_bf16x4(y_lat, (long long)t * L + c, hi[0], hi[1], hi[2], hi[3]);
  store_bf16x4(y_lat_lo, (long long)t * L + c, lo[0], lo[1], lo[2], lo[3]);
}

void launch_combine(const float* og, const int* inv, int T, int K, int L, uint16_t* y_lat,
                    uint16_t* y_lat_lo, hipStream_t s) {
  if (T <= 0) return;
  dim3 grid(T, (L / 4 + 63) / 64);
  combine_kernel<<<grid, 64, 0, s>>>(og, inv, K, L, y_lat, y_lat_lo);
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

}  // namespace lmoe
