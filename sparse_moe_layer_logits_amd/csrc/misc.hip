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
//
// MIX (large-tile path with two row classes): a row whose gate is below tau (the
// bf16 class) was written to og16 as bf16, the others to og as fp32.  Every k
// loads one fp32 and one bf16 row, one of them the zero row z32 / z16, and adds
// both: the sum and its order are those of a single format, and a bf16-class row
// costs half the bytes from memory (the zero rows stay cached).
template <bool MIX>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ og,
                                                     const uint16_t* __restrict__ og16,
                                                     const float* __restrict__ row_gate, float tau,
                                                     const float* __restrict__ z32,
                                                     const uint16_t* __restrict__ z16,
                                                     const int* __restrict__ inv, int K, int L,
                                                     uint16_t* __restrict__ y_lat,
                                                     uint16_t* __restrict__ y_lat_lo) {
  __shared__ int pos[64];
  __shared__ int wide[64];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int q = inv[(long long)t * K + threadIdx.x];
    pos[threadIdx.x] = q;
    wide[threadIdx.x] = !MIX || row_gate[q] >= tau;  // the class top-K assigned (same fp32 test)
  }
  __syncthreads();
  const int c = (blockIdx.y * 64 + threadIdx.x) * 4;
  if (c >= L) return;
  // row k's two sources, formed from the global arguments (addresses kept in LDS
  // would be generic and turn the loads into flat ones)
  auto p32 = [&](int k) { return wide[k] ? og + (long long)pos[k] * L + c : z32 + c; };
  auto p16 = [&](int k) { return wide[k] ? z16 + c : og16 + (long long)pos[k] * L + c; };
  auto widen = [](const u32x2_t& w) {
    return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= K; k += 8) {  // eight rows in flight, summed in k order
    f32x4_t v[8];
    u32x2_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = *reinterpret_cast<const f32x4_t*>(MIX ? p32(k + i) : og + (long long)pos[k + i] * L + c);
      if constexpr (MIX) w[i] = *reinterpret_cast<const u32x2_t*>(p16(k + i));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (MIX) v[i] += widen(w[i]);
      acc += v[i];
    }
  }
  for (; k < K; ++k) {
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(MIX ? p32(k) : og + (long long)pos[k] * L + c);
    if constexpr (MIX) v += widen(*reinterpret_cast<const u32x2_t*>(p16(k)));
    acc += v;
  }
  float hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = bf16_bits_to_f32(f32_to_bf16_bits(acc[i]));
    lo[i] = acc[i] - hi[i];
  }
  store_bf16x4(y_lat, (long long)t * L + c, hi[0], hi[1], hi[2], hi[3]);
  store_bf16x4(y_lat_lo, (long long)t * L + c, lo[0], lo[1], lo[2], lo[3]);
}

void launch_combine(const float* og, const uint16_t* og16, const float* row_gate, float tau,
                    const float* z32, const uint16_t* z16, const int* inv, int T, int K, int L,
                    uint16_t* y_lat, uint16_t* y_lat_lo, hipStream_t s) {
  if (T <= 0) return;
  dim3 grid(T, (L / 4 + 63) / 64);
  if (og16)
    combine_kernel<true><<<grid, 64, 0, s>>>(og, og16, row_gate, tau, z32, z16, inv, K, L, y_lat, y_lat_lo);
  else
    combine_kernel<false><<<grid, 64, 0, s>>>(og, nullptr, nullptr, 0.f, nullptr, nullptr, inv, K, L, y_lat,
                                              y_lat_lo);
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
