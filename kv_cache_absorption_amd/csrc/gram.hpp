// K-contiguous ("NT") MFMA GEMM for the statistics, and 16-bit layout helpers.
#pragma once

#include "common.hpp"

namespace ispa {

enum {
  kNtAccum = 0,   // out[m][n] += acc (fp32), upper triangle for first-kind tiles if tri; with a K split the
                  // workgroups store partial sums to part[split][kind] (layout of out) for nt_split_reduce
  kNtStoreT = 1,  // out[m][n] = acc as 16-bit (mfma type) for n < n_valid, 0 for n_valid <= n < N;
                  // per-workgroup sum of squares of the stored values
  kNtStore = 2,   // out[m][n] = acc as out_dt (bf16, f16 or fp32)
  kNtStoreScaled = 3  // out[m][n] = acc * sx[m] * sy[n] as out_dt (the dequantising store of the fp8 product)
};

// Operand type of an NT GEMM with OCP FP8 E4M3 operands (1-byte elements, 64
// per K stage, v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).  Not
// an ispa_dtype: only the W8A8 projection uses it.
constexpr int kMtE4M3 = 0x38;

struct NtGemmParams {
  int64_t M, N, K;   // acc[m][n] = sum_k X[m][k] Y[n][k]; K a multiple of kNtBK
  const void* x;     // [M][ldx] 16-bit, k contiguous
  const void* y;     // [y_rows][ldy]
  const void* y2;    // second-kind tiles' y operand (same ldy)
  int64_t ldx, ldy;  // elements, multiples of 8
  int64_t y_rows;    // rows of y that exist (rows past it are not read)
  int32_t epi;
  void* out;
  void* out2;        // second-kind tiles' output
  int64_t ld_out;
  int64_t n_valid;   // kNtStoreT: columns at or past n_valid are written as 0
  int32_t tiles_m, tiles_n;  // tiles of kNtBM x bn
  int32_t bn;                 // tile width: 256, or 128 (no triangle)
  int32_t tri, two_kinds;
  int32_t ksplit;
  int64_t kchunk;
  double* sq_partials;
  float* part;        // kNtAccum with ksplit > 1: [ksplit][2][M][ld_out] partial sums
  int32_t out_dt;     // kNtStore, kNtStoreScaled
  const float* sx;    // kNtStoreScaled: per-row (m) and per-column (n) scales
  const float* sy;
};

// mfma_dt: ISPA_BF16, ISPA_F16 or kMtE4M3; x, y element size follows it (ldx,
// ldy in elements: multiples of 8, and of 16 for kMtE4M3); K a multiple of the
// K stage (32 elements, 64 for kMtE4M3)
ispa_status launch_nt_gemm(const NtGemmParams& p, int mfma_dt, hipStream_t stream, int* n_blocks_out);
// Symmetric per-row FP8 E4M3 quantisation: for each of `rows` rows of `cols`
// elements (in_dt fp32, bf16 or f16; cols a multiple of 4, ld_in of 4),
// scale = amax / 448 and code = E4M3(clamp(x / scale, -448, 448)) with both
// divisions correctly rounded in fp32, ties to even, and a zero magnitude as
// code 0; a zero row gets scale 0 and zero codes.  codes: rows x ld_codes bytes.
ispa_status launch_quant_rows_e4m3(const void* in, int in_dt, int64_t ld_in, int64_t rows, int64_t cols,
                                   uint8_t* codes, int64_t ld_codes, float* scales, hipStream_t stream);
// out (and out2) += sum over splits of the partial sums a kNtAccum launch left in p.part
// (nothing when p.ksplit == 1), and *r2 += the n_sq sums of squares in sq
ispa_status launch_nt_split_reduce(const NtGemmParams& p, const double* sq, int64_t n_sq, double* r2,
                                   hipStream_t stream);
// K split of the statistics GEMM over np tokens at width D (tiles of kNtBM)
int64_t nt_stats_split(int32_t D, int64_t np);
// out[c][r] = in[r][c] (r < rows), 0 for rows <= r < rows_pad; rows_pad multiple of 4, cols of 4;
// 16-bit elements converted from in_dt to out_dt when they differ
ispa_status launch_transpose16(const void* in, int64_t ld_in, int64_t rows, int64_t cols, void* out,
                               int64_t ld_out, int64_t rows_pad, int in_dt, int out_dt, hipStream_t stream);
// one or two such transposes in a single launch
struct Transpose16 {
  const void* in;
  void* out;
  int64_t ld_in, rows, cols, ld_out, rows_pad;
  int in_dt, out_dt;
};
ispa_status launch_transpose16(const Transpose16* jobs, int n_jobs, hipStream_t stream);

constexpr int kNtBM = 256, kNtBK = 32;

// Symmetric rank-k update of X = [A_loc | dA] into a per-layer statistics
// state: S copies (one per token split) of G = A_loc^T A_loc, M = A_loc^T dA
// and H = dA^T dA, each D x D fp32 (G and H: upper block triangle
// maintained), copy s at state + s * split_stride floats, G, M, H in order.
struct SyrkParams {
  const void* a;      // A_loc [n][lda] 16-bit
  const void* b;      // dA    [n][lda]
  int64_t n, lda;
  int32_t D, nbh;     // width (multiple of 64), 256-column blocks per half
  int32_t n_tiles;    // upper-triangle tiles of the 2 nbh x 2 nbh block grid
  int32_t ksplit;     // S
  int64_t kchunk;     // token rows per split, multiple of 32
  float* state;
  int64_t split_stride;  // 3 D^2
};
// Splits of the state for width D (fixed per D so that the state layout does
// not depend on the chunk size).
int gram_splits(int32_t D);
ispa_status launch_syrk(const SyrkParams& p, int mfma_dt, hipStream_t stream);
// The switch-time statistics of one layer from its state: G (upper triangle,
// entries below the diagonal untouched), C = M W and r2 = <H, W W^T>, all
// written (not accumulated).  w: bf16 [D][D].  Workspace: gram_finalize_ws_bytes.
size_t gram_finalize_ws_bytes(int32_t D);
ispa_status launch_gram_finalize(int32_t D, const float* state, int64_t split_stride, int S, const uint16_t* w,
                                 float* G, float* C, double* r2, void* ws, hipStream_t stream);

}  // namespace ispa
