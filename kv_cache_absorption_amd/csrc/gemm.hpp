// Tile GEMM on MFMA used by the statistics and the projection.
#pragma once

#include "common.hpp"

namespace ispa {

// Operand source: element (row, k) of an operand that the MFMA reads as
// [rows][k].  kDirect: memory holds [row][k] (k contiguous, leading dim ld).
// kTrans: memory holds [k][row] (rows contiguous, leading dim ld).
enum { kDirect = 0, kTrans = 1 };

// Epilogues.
enum {
  kStoreRt = 0,     // write acc as 16-bit (mfma type) to out[m][n] (ld_out) + sum of squares
  kAccum = 1,       // out[m][n] += acc (fp32, ld_out; atomic when K is split); upper triangle only if tri
  kStore = 2        // out[m][n] = acc as out_dt (fp32 / bf16 / f16)
};

struct GemmOperand {
  const void* p;
  int64_t ld;
  int32_t dt;      // element type in memory
  int32_t layout;  // kDirect / kTrans
};

struct GemmParams {
  int64_t M, N, K;
  GemmOperand x;   // rows = m
  GemmOperand y;   // rows = n
  GemmOperand y2;  // rows = n of the second kind of tiles (same layout and type as y)
  int32_t epi;
  int32_t out_dt;
  void* out;
  void* out2;      // output of the second kind of tiles
  int64_t ld_out;
  int32_t tiles_m, tiles_n;
  int32_t tri;     // first-kind tiles: upper triangle only (tm <= tn) and entries m <= n
  int32_t two_kinds;  // a full tiles_m x tiles_n grid of second-kind tiles follows
  int32_t ksplit;  // K split into ksplit ranges of kchunk (multiple of kGemmBK)
  int64_t kchunk;
  double* sq_partials;  // per-workgroup sum of squares (kStoreRt)
};

// mfma_dt: ISPA_BF16 or ISPA_F16 -- the type products are computed in.
ispa_status launch_gemm(const GemmParams& p, int mfma_dt, hipStream_t stream, int* n_blocks_out);

// fp32 paths (parity mode)
ispa_status launch_stats_f32(int64_t n, int32_t D, const float* a, const float* dl, const float* w,
                             float* G, float* C, double* r2, void* ws, hipStream_t stream);
ispa_status launch_proj_f32(int64_t n, int32_t D, const float* x, const float* w, void* y,
                            int32_t y_dt, hipStream_t stream);
// sum partials[0..n) into *r2 (one workgroup)
ispa_status launch_reduce_add(const double* partials, int64_t n, double* r2, hipStream_t stream);

constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 32;

}  // namespace ispa
