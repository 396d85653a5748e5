// Kernel launch interface used by the host orchestration (latentmoe.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

// epilogue kinds; each applies to four consecutive output columns of one row
// (tscale = b_tscale, 1 when null; e = the tile's expert, 0 for dense GEMMs)
enum Epi : int {
  EPI_PARTIAL = 0,      // partial[split][row][n] = acc                         (split-K)
  EPI_BF16 = 1,         // C bf16 = acc
  EPI_SQRELU_BF16 = 2,  // C bf16 = relu(acc * tscale[e])^2
  EPI_SQRELU_HILO = 3,  // v = relu(acc * tscale[e])^2; C bf16 = hi(v), C2 bf16 = bf16(v - hi(v))
  EPI_F32 = 4,          // C f32 = acc * tscale[e] (+ bias[n])
  EPI_F32_ADD = 5,      // C f32 += acc * tscale[e]
  EPI_GATE_F32 = 6,     // C f32 = acc * tscale[e] * row_scale[row]
  EPI_GATE_BF16 = 7,    // C bf16 = acc * tscale[e] * row_scale[row]
  EPI_BF16_HILO = 8,    // v = acc * tscale[e]; C bf16 = hi(v), C2 bf16 = bf16(v - hi(v))
};

// stored weight formats of the B operand (same values as the C ABI's formats)
enum WFmt : int {
  WF_BF16 = 0,  // bf16
  WF_FP4 = 1,   // E2M1 codes, E4M3 scale per 16 k, fp32 scale per matrix
  WF_FP8 = 2,   // E4M3 bytes, fp32 scale per matrix
};

struct GemmSeg {
  const void* A;  // [rows, lda] bf16
  const void* B;  // [N, ldb] bf16, packed FP4 codes [N, ldb/2] bytes, or FP8 [N, ldb] bytes
  int K;          // multiple of 64
};

// With a_lo set ("dual" mode, one segment) the kernels compute
// (A + A_lo) * B^T: every weight fragment is loaded once and multiplied with
// both bf16 parts of the activation, which together carry about 16 bits.

// C[row, n] = sum over segments of sum_k A_seg[row, k] * B_seg[n, k]
struct GemmParams {
  GemmSeg seg[3];
  int nseg;
  const void* a_lo;  // [rows, lda] bf16 remainder of seg[0].A, or null
  int lda, ldb;      // row strides in elements (ldb counts FP4 elements for packed B)
  int M, N;          // dense rows, output columns
  // grouped (expert) mode: work tiles built on the device
  const int* tile_expert;   // null => dense
  const int* tile_row0;     // first (permuted) row of the tile
  const int* tile_rows;     // rows in the tile
  const int* n_tiles;       // number of valid tiles (device scalar)
  const int* tile_first;    // first tile of this launch in the tile list (device scalar) or null
  int max_tiles;            // launch bound on tiles
  int rows_per_tile;        // tile height the tile list was built for (grouped mode)
  const int* row_index;     // A row of permuted row p (null => A row = p)
  long long b_stride;       // elements between consecutive experts' B (FP4: elements, i.e. 2 per byte)
  // block-scaled FP4 B operand
  const uint8_t* b_scale;   // [E, N, ldb/16] E4M3FN
  const uint8_t* b_scale_sm; // the same scales stage-major, [E, ldb/128, N, 8] (or null)
  const float* b_tscale;    // [E] fp32 (FP4 / FP8 tensor scales) applied to the accumulator (null => 1)
  // split-K
  int splits;
  int k_split;              // k elements per split (multiple of 64)
  // epilogue
  int epi;
  void* C;
  void* C2;
  int ldc;
  const float* bias;        // [N] or null
  const float* row_scale;   // [rows] or null (gate per permuted row)
  float* partial;           // [splits, M, N]
  long long partial_stride; // elements between splits
};

// weight-streaming MFMA GEMM for <= 64 rows per tile (decode-like shapes); fmt is a
// WFmt (FP8 with 64-row tiles only)
void launch_gemm_stream(const GemmParams& p, int fmt, hipStream_t s);
// one launch of a grouped bf16 expert GEMM p (hi + lo activations) and a dense bf16
// GEMM q of at most 64 rows over its whole k range (q.splits == 1, q's blocks first)
void launch_gemm_stream_pair(const GemmParams& p, const GemmParams& q, hipStream_t s);
// grouped MFMA GEMM for 64-row expert tiles of block-scaled FP4 weights with dual
// activations (tens of rows per expert): activations staged in LDS, weights read once
void launch_gemm_mid(const GemmParams& p, bool fp4, hipStream_t s);
bool gemm_mid_supports(const GemmParams& p, bool fp4);
// one-time kernel attributes (dynamic LDS above 64 KB); returns a HIP error code
int gemm_mid_setup();
// FP4 block scales [E, N, K/16] -> stage-major [E, K/128, N, 8] (the mid kernel's order)
void launch_scale_stage_major(const uint8_t* src, uint8_t* dst, long long E, int N, int K,
                              hipStream_t s);
// large-tile MFMA GEMM, 256 x 256 tiles (prefill-sized problems)
void launch_gemm_big(const GemmParams& p, hipStream_t s);
bool gemm_big_supports(int epi);
// one-time kernel attributes (dynamic LDS above 64 KB); returns a HIP error code
int gemm_big_setup();
// sum split-K partials and apply the epilogue
void launch_reduce(const GemmParams& p, hipStream_t s);

// router weight fp32 [N, d] -> three bf16 pieces whose sum is exact
void launch_router_split(const float* w, uint16_t* pieces, long long n, hipStream_t s);

// per-token top-K + softmax over logits [T, N] (+ bias); builds per-16-token expert masks
// (masks_hi, if not null: the routed rows that carry a bf16 hi + lo pair -- each
// token's largest gates until the rows left out hold at most tail_frac of its
// sum_k g_k^2 -- and paired[t*K + k] = 1 for them, 0 for the others)
void launch_topk(const float* logits, const float* bias, int T, int N, int K, int* idx,
                 float* gates, uint32_t* masks, float tail_frac, uint32_t* masks_hi, uint8_t* paired,
                 hipStream_t s);
// counts, offsets, per-block prefixes and the expert tile list (tile_rows_max rows per tile);
// with masks_hi the rows of each expert are split into the hi class (first) and the rest,
// hi tiles first in the list: n_tiles[0] hi tiles, then n_tiles[1] others.  With place_idx
// set it also does launch_place's work in the same workgroup (small T)
// (chunk_hi, chunk_lo non-null: [bucket_chunks(T), N] scratch; the prefix is split
// over chunks of mask groups, and launch_place must get the same two pointers)
void launch_bucket_scan(const uint32_t* masks, const uint32_t* masks_hi, int T, int N,
                        int tile_rows_max, int* counts, int* counts_hi, int* offsets,
                        int* prefix_hi, int* prefix_lo, int* tile_expert, int* tile_row0,
                        int* tile_rows, int* n_tiles, int max_tiles, const int* place_idx,
                        const float* place_gates, int K, int* row_src, float* row_gate, int* inv,
                        int* chunk_hi, int* chunk_lo, hipStream_t s);
int bucket_chunks(int T);
// permuted positions: row_src[p] = token, row_gate[p] = gate, inv[t*K+k] = p
void launch_place(const int* idx, const float* gates, const uint32_t* masks,
                  const uint32_t* masks_hi, const int* offsets, const int* counts_hi,
                  const int* prefix_hi, const int* prefix_lo, int T, int N, int K, int* row_src,
                  float* row_gate, int* inv, const int* chunk_hi, const int* chunk_lo, hipStream_t s);
// y_lat[t] = sum_k og[inv[t*K+k]] (fixed k order) -> bf16 hi + bf16 lo (rows of stride
// ldy).  With og16, rows with paired[t*K+k] == 0 are read from og16 (bf16) instead.
void launch_combine(const float* og, const uint16_t* og16, const uint8_t* paired, const int* inv, int T,
                    int K, int L, uint16_t* y_lat, uint16_t* y_lat_lo, int ldy, hipStream_t s);
// split-K partials [splits][T][3N + L + MS] of the GEMM over x with the stacked rows
// [router pieces 1-3; W_down; S1] -> fp32 logits [T, N] (the three piece columns
// summed), z (bf16 hi + lo, [T, L]) and h_s = relu(.)^2 (bf16 hi + lo, rows of stride ldh)
void launch_xreduce(const float* partial, int splits, long long pstride, int T, int N, int L, int MS,
                    float* logits, uint16_t* z, uint16_t* z_lo, uint16_t* hs, uint16_t* hs_lo, int ldh,
                    hipStream_t s);
// FP4 blocks (8 code bytes + 1 scale byte each) -> exact bf16 with the in-register
// decoder (tensor scale not applied): decode check and the bf16 expansion at init
void launch_fp4_dequant(const uint8_t* codes, const uint8_t* scales, long long n_blocks16,
                        uint16_t* out, hipStream_t s);
// zero `bytes` bytes (a multiple of 4) at device address p with a kernel
void launch_zero(void* p, size_t bytes, hipStream_t s);
// dst[sl][i][j] = src[sl srows + i][j] for i < rows, j < cols, else 0 (bytes; dst rows of
// dpitch bytes, drows rows per slice; src rows of spitch bytes, srows rows per slice)
void launch_pad_copy(const void* src, size_t spitch, int srows, void* dst, size_t dpitch, int drows,
                     long long slices, int rows, size_t cols, hipStream_t s);
// groups of 16 E4M3 bytes -> exact bf16 with the in-register decoder (tensor scale not applied)
void launch_fp8_dequant(const uint8_t* codes, long long n_groups16, uint16_t* out, hipStream_t s);

}  // namespace lmoe
