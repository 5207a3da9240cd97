// Ridge solve (G + lambda I) dW = C with eps, batched over layers, fp64.
//
// The closed form dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W
// (DE summary, Methodik) is evaluated as a blocked right-looking Cholesky
// factorisation G + lambda I = L L^T with 64 x 64 blocks, followed by block
// forward and backward substitution for all D right-hand sides.  Each step of
// the factorisation is three launches, all batched over layers:
//   potrf : factor the diagonal block in LDS and form its triangular inverse
//   trsm  : panel blocks L_ik = A_ik L_kk^-T  (block product with the inverse)
//   syrk  : trailing blocks A_ij -= L_ik L_jk^T
// and each substitution step is two launches (diagonal block, then update of
// the remaining block rows).  eps uses the identity that holds at the ridge
// optimum, eps = r2 - <dW, C> - lambda ||dW||^2 (from G dW = C - lambda dW),
// which is ||A_loc dW - R||^2 without the penalty (EN review, Key Design 2).
#include <cmath>

#include "common.hpp"

namespace ispa {

namespace {

constexpr int NB = 64;

struct SolveWs {
  double* A;     // [L][D][D]
  double* X;     // [L][D][D]
  double* Linv;  // [L][D][NB]
  double* lam;   // [L]
  double* part;  // [L][kEpsBlocks][2]
};
constexpr int kEpsBlocks = 64;

size_t ws_layout(int L, int D, SolveWs* w, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  double* A = (double*)take((size_t)L * D * D * 8);
  double* X = (double*)take((size_t)L * D * D * 8);
  double* Li = (double*)take((size_t)L * D * NB * 8);
  double* lam = (double*)take((size_t)L * 8);
  double* part = (double*)take((size_t)L * kEpsBlocks * 2 * 8);
  if (w) *w = SolveWs{A, X, Li, lam, part};
  return off;
}

__global__ void trace_kernel(int D, const float* G, int64_t ms, double la, double lr, double* lam,
                             int32_t* info) {
  __shared__ double red[256];
  const int l = blockIdx.x;
  const float* g = G + (int64_t)l * ms;
  double s = 0.0;
  for (int i = threadIdx.x; i < D; i += 256) s += (double)g[(int64_t)i * D + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    lam[l] = la + lr * red[0] / D;
    info[l] = 0;
  }
}

// A = sym(G upper) + lambda I, X = C  (fp64)
__global__ void fill_kernel(int D, const float* G, const float* C, int64_t ms, const double* lam,
                            double* A, double* X) {
  const int l = blockIdx.y;
  const int64_t DD = (int64_t)D * D;
  const float* g = G + (int64_t)l * ms;
  const float* c = C + (int64_t)l * ms;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < DD; e += (int64_t)gridDim.x * 256) {
    const int i = e / D, j = e % D;
    const int lo = i < j ? i : j, hi = i < j ? j : i;
    double a = (double)g[(int64_t)lo * D + hi];
    if (i == j) a += lam[l];
    A[l * DD + e] = a;
    X[l * DD + e] = (double)c[e];
  }
}

// Factor diagonal block kb of every layer and write its inverse.
__global__ __launch_bounds__(256) void potrf_kernel(int D, int kb, double* Aall, double* Liall,
                                                    int32_t* info) {
  __shared__ double a[NB][NB + 1];
  __shared__ int failed;
  const int l = blockIdx.x;
  const int tid = threadIdx.x;
  double* A = Aall + (int64_t)l * D * D;
  const int64_t base = (int64_t)kb * NB * D + (int64_t)kb * NB;
  for (int e = tid; e < NB * NB; e += 256) a[e / NB][e % NB] = A[base + (int64_t)(e / NB) * D + e % NB];
  if (tid == 0) failed = 0;
  __syncthreads();
  for (int j = 0; j < NB; ++j) {
    const double piv = a[j][j];
    if (!(piv > 0.0)) {
      if (tid == 0) {
        failed = 1;
        if (info[l] == 0) info[l] = kb * NB + j + 1;
      }
      break;
    }
    const double d = sqrt(piv);
    __syncthreads();
    if (tid == 0) a[j][j] = d;
    for (int i = j + 1 + tid; i < NB; i += 256) a[i][j] /= d;
    __syncthreads();
    const int m = NB - 1 - j;  // trailing size
    const int cnt = m * (m + 1) / 2;
    for (int idx = tid; idx < cnt; idx += 256) {
      // row r (0..m-1), col c (0..r) of the trailing lower triangle
      int r = (int)((sqrt(8.0 * idx + 1.0) - 1.0) * 0.5);
      while (r * (r + 1) / 2 > idx) --r;
      while ((r + 1) * (r + 2) / 2 <= idx) ++r;
      const int c = idx - r * (r + 1) / 2;
      const int i = j + 1 + r, k = j + 1 + c;
      a[i][k] -= a[i][j] * a[k][j];
    }
    __syncthreads();
  }
  __syncthreads();
  if (failed) {
    // leave NaN so every later product of this layer is NaN
    for (int e = tid; e < NB * NB; e += 256) A[base + (int64_t)(e / NB) * D + e % NB] = NAN;
    double* Li = Liall + (int64_t)l * D * NB + (int64_t)kb * NB * NB;
    for (int e = tid; e < NB * NB; e += 256) Li[e] = NAN;
    return;
  }
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, k = e % NB;
    A[base + (int64_t)i * D + k] = k <= i ? a[i][k] : 0.0;
  }
  if (tid < NB) {
    // column tid of L^-1 by forward substitution on e_tid
    double x[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      double s = (i == tid) ? 1.0 : 0.0;
#pragma unroll
      for (int t = 0; t < i; ++t) s -= a[i][t] * x[t];
      x[i] = s / a[i][i];
    }
    double* Li = Liall + (int64_t)l * D * NB + (int64_t)kb * NB * NB;
#pragma unroll
    for (int i = 0; i < NB; ++i) Li[i * NB + tid] = x[i];
  }
}

enum { kTrsm = 0, kSyrk = 1, kFwdDiag = 2, kFwdUpd = 3, kBwdDiag = 4, kBwdUpd = 5 };

struct BlockOp {
  const double* p;  // block top-left
  int64_t ld;
  int trans;        // operand element (i, k) = p[k*ld + i] if trans else p[i*ld + k]
};

// Out (64 x 64, ld) = [Out -] Aop Bop, K = 64.
__device__ void block_product(BlockOp A, BlockOp B, double* out, int64_t ld_out, bool subtract) {
  __shared__ double as[NB][33];
  __shared__ double bs[32][NB + 1];
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  double acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  for (int kh = 0; kh < 2; ++kh) {
    for (int e = tid; e < NB * 32; e += 256) {
      const int i = e >> 5, k = e & 31;
      const int kk = kh * 32 + k;
      as[i][k] = A.trans ? A.p[(int64_t)kk * A.ld + i] : A.p[(int64_t)i * A.ld + kk];
    }
    for (int e = tid; e < 32 * NB; e += 256) {
      const int k = e >> 6, j = e & 63;
      const int kk = kh * 32 + k;
      bs[k][j] = B.trans ? B.p[(int64_t)j * B.ld + kk] : B.p[(int64_t)kk * B.ld + j];
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = as[ty + 16 * r][k];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = bs[k][tx + 16 * c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      double* o = out + (int64_t)(ty + 16 * r) * ld_out + tx + 16 * c;
      *o = subtract ? *o - acc[r][c] : acc[r][c];
    }
}

__global__ __launch_bounds__(256) void block_step_kernel(int kind, int D, int kb, double* Aall,
                                                         double* Xall, const double* Liall) {
  const int l = blockIdx.y;
  const int nb = D / NB;
  double* A = Aall + (int64_t)l * D * D;
  double* X = Xall + (int64_t)l * D * D;
  const double* Li = Liall + (int64_t)l * D * NB + (int64_t)kb * NB * NB;
  auto blk = [&](double* M, int bi, int bj) { return M + (int64_t)bi * NB * D + (int64_t)bj * NB; };
  const int b = blockIdx.x;
  switch (kind) {
    case kTrsm: {  // A_ik = A_ik Li^T, i > kb
      const int i = kb + 1 + b;
      block_product(BlockOp{blk(A, i, kb), D, 0}, BlockOp{Li, NB, 1}, blk(A, i, kb), D, false);
      break;
    }
    case kSyrk: {  // A_ij -= A_ik A_jk^T, kb < j <= i
      int r = (int)((sqrt(8.0 * b + 1.0) - 1.0) * 0.5);
      while (r * (r + 1) / 2 > b) --r;
      while ((r + 1) * (r + 2) / 2 <= b) ++r;
      const int c = b - r * (r + 1) / 2;
      const int i = kb + 1 + r, j = kb + 1 + c;
      block_product(BlockOp{blk(A, i, kb), D, 0}, BlockOp{blk(A, j, kb), D, 1}, blk(A, i, j), D, true);
      break;
    }
    case kFwdDiag: {  // X_kb,j = Li X_kb,j
      block_product(BlockOp{Li, NB, 0}, BlockOp{blk(X, kb, b), D, 0}, blk(X, kb, b), D, false);
      break;
    }
    case kFwdUpd: {  // X_ij -= A_i,kb X_kb,j, i > kb
      const int i = kb + 1 + b / nb, j = b % nb;
      block_product(BlockOp{blk(A, i, kb), D, 0}, BlockOp{blk(X, kb, j), D, 0}, blk(X, i, j), D, true);
      break;
    }
    case kBwdDiag: {  // X_kb,j = Li^T X_kb,j
      block_product(BlockOp{Li, NB, 1}, BlockOp{blk(X, kb, b), D, 0}, blk(X, kb, b), D, false);
      break;
    }
    case kBwdUpd: {  // X_ij -= A_kb,i^T X_kb,j, i < kb
      const int i = b / nb, j = b % nb;
      block_product(BlockOp{blk(A, kb, i), D, 1}, BlockOp{blk(X, kb, j), D, 0}, blk(X, i, j), D, true);
      break;
    }
  }
}

// dW out, W_eff, and per-block partial sums <X, C>, ||X||^2
__global__ void finalize_kernel(int D, const double* Xall, const float* C, int64_t ms,
                                const int32_t* info, float* dW, const void* w, int w_dt, void* w_eff,
                                double* part) {
  __shared__ double r1[256], r2s[256];
  const int l = blockIdx.y;
  const int64_t DD = (int64_t)D * D;
  const double* X = Xall + l * DD;
  const bool bad = info[l] != 0;
  double s1 = 0.0, s2 = 0.0;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < DD; e += (int64_t)gridDim.x * 256) {
    const double x = X[e];
    s1 += x * (double)C[l * ms + e];
    s2 += x * x;
    const float xf = bad ? NAN : (float)x;
    dW[l * ms + e] = xf;
    if (w_eff) {
      const float we = load_as_f32(w, l * ms + e, w_dt) + xf;
      store_from_f32(w_eff, l * ms + e, we, w_dt);
    }
  }
  r1[threadIdx.x] = s1;
  r2s[threadIdx.x] = s2;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) {
      r1[threadIdx.x] += r1[threadIdx.x + off];
      r2s[threadIdx.x] += r2s[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[(l * kEpsBlocks + blockIdx.x) * 2 + 0] = r1[0];
    part[(l * kEpsBlocks + blockIdx.x) * 2 + 1] = r2s[0];
  }
}

__global__ void eps_kernel(int L, const double* r2, const double* lam, const int32_t* info,
                           const double* part, double* eps) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= L) return;
  double dot = 0.0, nrm = 0.0;
  for (int b = 0; b < kEpsBlocks; ++b) {
    dot += part[(l * kEpsBlocks + b) * 2 + 0];
    nrm += part[(l * kEpsBlocks + b) * 2 + 1];
  }
  eps[l] = info[l] ? NAN : r2[l] - dot - lam[l] * nrm;
}

}  // namespace

size_t solve_ws_bytes(int32_t n_layers, int32_t D) { return ws_layout(n_layers, D, nullptr, nullptr); }

ispa_status run_solve(int32_t L, int32_t D, const float* G, const float* C, const double* r2,
                      int64_t ms, double la, double lr, float* dW, double* eps, int32_t* info,
                      const void* w, int w_dt, void* w_eff, void* ws, hipStream_t stream) {
  SolveWs s;
  ws_layout(L, D, &s, (char*)ws);
  const int nb = D / NB;
  hipLaunchKernelGGL(trace_kernel, dim3(L), dim3(256), 0, stream, D, G, ms, la, lr, s.lam, info);
  const int64_t DD = (int64_t)D * D;
  const unsigned fill_blocks = (unsigned)std::min<int64_t>((DD + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_kernel, dim3(fill_blocks, L), dim3(256), 0, stream, D, G, C, ms, s.lam, s.A, s.X);
  for (int kb = 0; kb < nb; ++kb) {
    hipLaunchKernelGGL(potrf_kernel, dim3(L), dim3(256), 0, stream, D, kb, s.A, s.Linv, info);
    const int m = nb - 1 - kb;
    if (m > 0) {
      hipLaunchKernelGGL(block_step_kernel, dim3(m, L), dim3(256), 0, stream, (int)kTrsm, D, kb, s.A, s.X,
                         s.Linv);
      hipLaunchKernelGGL(block_step_kernel, dim3(m * (m + 1) / 2, L), dim3(256), 0, stream, (int)kSyrk, D,
                         kb, s.A, s.X, s.Linv);
    }
  }
  for (int kb = 0; kb < nb; ++kb) {
    hipLaunchKernelGGL(block_step_kernel, dim3(nb, L), dim3(256), 0, stream, (int)kFwdDiag, D, kb, s.A, s.X,
                       s.Linv);
    const int m = nb - 1 - kb;
    if (m > 0)
      hipLaunchKernelGGL(block_step_kernel, dim3(m * nb, L), dim3(256), 0, stream, (int)kFwdUpd, D, kb, s.A,
                         s.X, s.Linv);
  }
  for (int kb = nb - 1; kb >= 0; --kb) {
    hipLaunchKernelGGL(block_step_kernel, dim3(nb, L), dim3(256), 0, stream, (int)kBwdDiag, D, kb, s.A, s.X,
                       s.Linv);
    if (kb > 0)
      hipLaunchKernelGGL(block_step_kernel, dim3(kb * nb, L), dim3(256), 0, stream, (int)kBwdUpd, D, kb, s.A,
                         s.X, s.Linv);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(kEpsBlocks, L), dim3(256), 0, stream, D, s.X, C, ms, info, dW, w,
                     w_dt, w_eff, s.part);
  hipLaunchKernelGGL(eps_kernel, dim3((L + 63) / 64), dim3(64), 0, stream, L, r2, s.lam, info, s.part, eps);
  return check_launch("solve kernels");
}

}  // namespace ispa
