// Ridge solve (G + lambda I) dW = C with eps, batched over layers, fp64.
//
// The closed form dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W
// (DE summary, Methodik) is evaluated as a blocked right-looking Cholesky
// factorisation G + lambda I = L L^T with 64 x 64 blocks and block forward and
// backward substitution for all D right-hand sides, every launch batched over
// layers.  Per block column kb there are two launches: the panel (L_ik =
// A_ik inv(L_kk)^T, and the forward diagonal step on X's block row kb) and the
// update (trailing A_ij -= L_ik L_jk^T, forward X_ij -= L_ik X_kb,j, and the
// factorisation of the next diagonal block by the workgroup that updates it).
// The backward substitution is one launch per block row, whose workgroups of
// block row kb - 1 also apply inv(L)^T of that row right after its last
// update.  Block products are 64 x 64 x 64 fp64 MFMA tiles from LDS; a
// diagonal block is turned into inv(L_kk) by the workgroup (chol_inv64).  eps uses
// the identity that holds at the ridge optimum, eps = r2 - <dW, C> -
// lambda ||dW||^2 (from G dW = C - lambda dW), which is ||A_loc dW - R||^2
// without the penalty (EN review, Key Design 2).
#include <algorithm>
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
constexpr int kEpsBlocks = 1024;  // finalize workgroups per layer

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

// ---- 64 x 64 fp64 blocks in LDS (row pitch LDP doubles) and their MFMA product

constexpr int LDP = NB + 1;  // pitch: the 16 rows of an A fragment fall in distinct banks

struct BlockOp {
  const double* p;  // block top-left
  int64_t ld;
  int trans;        // element (r, c) = p[c*ld + r] if trans else p[r*ld + c]
};

// dst[r][c] = element (r, c) of o; global reads run along o's contiguous dimension
__device__ __forceinline__ void stage(double* dst, BlockOp o) {
  const int t = threadIdx.x;
  const int u = t & 63, v0 = t >> 6;
  double x[NB / 4];
#pragma unroll
  for (int it = 0; it < NB / 4; ++it) {
    const int v = v0 + 4 * it;
    x[it] = o.p[(int64_t)v * o.ld + u];
  }
#pragma unroll
  for (int it = 0; it < NB / 4; ++it) {
    const int v = v0 + 4 * it;
    if (o.trans)
      dst[u * LDP + v] = x[it];
    else
      dst[v * LDP + u] = x[it];
  }
}

// acc = As * Bs for this wave's 32 x 32 quadrant, as 2 x 2 tiles of
// v_mfma_f64_16x16x4 (A fragment: lane holds A[l % 16][l / 16]; B fragment:
// B[l / 16][l % 16]; result element e of lane l: row l / 16 + 4 e, column l % 16)
__device__ __forceinline__ void mma64(const double* As, const double* Bs, f64x4 (&acc)[2][2], bool accumulate = false) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32, li = lane & 15, lk = lane >> 4;
  if (!accumulate)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < NB / 4; ++ks) {
    const double a0 = As[(r0 + li) * LDP + 4 * ks + lk];
    const double a1 = As[(r0 + 16 + li) * LDP + 4 * ks + lk];
    const double b0 = Bs[(4 * ks + lk) * LDP + c0 + li];
    const double b1 = Bs[(4 * ks + lk) * LDP + c0 + 16 + li];
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
  }
}

// Visit this lane's product elements: f(row, col, value)
template <class F>
__device__ __forceinline__ void for_acc(const f64x4 (&acc)[2][2], F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32, li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int e = 0; e < 4; ++e) f(r0 + 16 * ti + lk + 4 * e, c0 + 16 * tj + li, acc[ti][tj][e]);
}

// out (global, ld) = acc, or out - acc
__device__ __forceinline__ void store_block(const f64x4 (&acc)[2][2], double* out, int64_t ld, bool subtract) {
  for_acc(acc, [&](int r, int c, double v) {
    double* o = out + (int64_t)r * ld + c;
    *o = subtract ? *o - v : v;
  });
}

// dst (LDS) = old (global) - acc
__device__ __forceinline__ void sub_to_lds(const f64x4 (&acc)[2][2], const double* old, int64_t ld, double* dst) {
  for_acc(acc, [&](int r, int c, double v) { dst[r * LDP + c] = old[(int64_t)r * ld + c] - v; });
}

// Inverse of the Cholesky factor of the SPD 64 x 64 block M (LDS, pitch LDP),
// by the workgroup's four waves.
//
// Lane a of every wave holds column a; wave w holds its rows 16w .. 16w+15.
// Elimination is right-looking, pivot by pivot, on symmetric Schur
// complements, so the multipliers of step j are row j.  The wave that holds
// row j publishes it to LDS twice: as is, for each lane's own multiplier, and
// with the entries at and above the diagonal zeroed, so that every wave
// updates all 16 of its rows without a branch.  One barrier per step makes
// each row visible.  When step j reaches its own column, lane j stops
// updating: its remaining entries are then column j of the inverse unit
// factor times -pivot_j, and the later steps update them with the same
// formula as the matrix columns.  Pivot j is the squared diagonal of the
// Cholesky factor, so inv(L)[i][a] = E[i][a] / sqrt(pivot_i) with E the
// inverse unit factor.
// M is overwritten (it holds the zeroed rows); rows: 64 x 64 doubles of LDS.
// Writes Li (row-major, 64 wide); returns the first non-positive pivot
// (1-based) or 0.  Every thread of the workgroup must call it.
__device__ __forceinline__ int chol_inv64(double* M, double* rows, double* Li) {
  const int a = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  double c[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = M[(16 * w + r) * LDP + a];
  __syncthreads();  // every row is in registers: M becomes the zeroed-row table
  double* mult = M;
  double* rowv = rows;
  auto publish = [&](int j, double v) {
    rowv[j * NB + a] = v;
    mult[j * NB + a] = a > j ? v : 0.0;
  };
  if (w == 0) publish(0, c[0]);
  int bad = 0;
#pragma unroll 1
  for (int j = 0; j < NB; ++j) {
    __syncthreads();  // row j is published
    const double piv = rowv[j * NB + j];
    if (!(piv > 0.0) && bad == 0) bad = j + 1;
    const double s = a == j ? 0.0 : rowv[j * NB + a] / piv;
    const double* mj = mult + j * NB + 16 * w;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = fma(-mj[r], s, c[r]);
    const int jn = j + 1;
    if (jn < NB && w == (jn >> 4)) {  // this wave holds row j + 1 (wave-uniform)
      const int rl = jn & 15;
      double v = c[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) v = rl == r ? c[r] : v;
      publish(jn, v);
    }
  }
  __syncthreads();  // the last row is published
  const double ea = -1.0 / rowv[a * NB + a];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 16 * w + r;
    const double isq = 1.0 / sqrt(rowv[i * NB + i]);
    const double v = i < a ? 0.0 : (i == a ? isq : c[r] * ea * isq);
    Li[i * NB + a] = bad ? NAN : v;
  }
  return bad;
}

// factor the block in As (all waves) and record the first failing pivot
__device__ __forceinline__ void factor_block(double* As, double* Bs, double* Li, int32_t* info, int base) {
  const int bad = chol_inv64(As, Bs, Li);
  if (bad && threadIdx.x == 0 && *info == 0) *info = base + bad;
}

enum { kPotrf0 = 0, kPanel = 1, kUpdate = 2, kBwd = 3 };

// Block ranges of one launch (block indices, half-open): the contraction range
// [k_lo, k_hi) and, for kUpdate, the A columns [j_lo, j_hi) (every block on or
// below the diagonal in them) and the X block rows [x_lo, x_hi); for kBwd the X
// block rows [x_lo, x_hi) and the row diag that is finished in the same launch.
struct StepArgs {
  int kind, kb;
  int k_lo, k_hi, j_lo, j_hi, x_lo, x_hi, diag;
};

// One launch of the blocked solve, batched over layers (blockIdx.y).
//   kPotrf0      : inv(L_00)
//   kPanel  (kb) : L_ik = A_ik inv(L_kk)^T for i > kb, and the forward diagonal
//                  step X_kb = inv(L_kk) X_kb (for the last kb also the backward
//                  one, X_kb = inv(L_kk)^T X_kb)
//   kUpdate      : A_ij -= sum_k L_ik L_jk^T for j in [j_lo, j_hi), i >= j, and
//                  X_ij -= sum_k L_ik X_kj for i in [x_lo, x_hi); the workgroup of
//                  the block (j_lo, j_lo) then factors it
//   kBwd         : X_ij -= sum_k L_ki^T X_kj for i in [x_lo, x_hi); for i = diag
//                  then also X_ij = inv(L_ii)^T X_ij
// Diagonal blocks keep only inv(L_kk) (in Li); the strictly lower blocks of A
// become L.  Every launch writes blocks that no other workgroup of it reads.
__global__ __launch_bounds__(256, 2) void solve_step_kernel(StepArgs g, int D, double* Aall, double* Xall,
                                                           double* Liall, int32_t* info) {
  __shared__ double As[NB * LDP], Bs[NB * LDP];
  const int l = blockIdx.y;
  const int nb = D / NB;
  const int b = blockIdx.x;
  double* A = Aall + (int64_t)l * D * D;
  double* X = Xall + (int64_t)l * D * D;
  double* Li = Liall + (int64_t)l * D * NB;
  auto blk = [&](double* M, int bi, int bj) { return M + (int64_t)bi * NB * D + (int64_t)bj * NB; };
  auto linv = [&](int k) { return Li + (int64_t)k * NB * NB; };
  f64x4 acc[2][2];
  double* fac_li = nullptr;  // set when this workgroup factors a diagonal block (in As)
  int fac_base = 0;
  auto product = [&](BlockOp x, BlockOp y, bool accumulate) {
    stage(As, x);
    stage(Bs, y);
    __syncthreads();
    mma64(As, Bs, acc, accumulate);
  };
  // acc = sum over the contraction range of x(k) y(k)
  auto sum_products = [&](auto x, auto y) {
    for (int k = g.k_lo; k < g.k_hi; ++k) {
      if (k > g.k_lo) __syncthreads();  // the previous product is done with As and Bs
      product(x(k), y(k), k > g.k_lo);
    }
  };
  switch (g.kind) {
    case kPotrf0: {
      stage(As, BlockOp{blk(A, 0, 0), D, 0});
      __syncthreads();
      fac_li = linv(0);
      break;
    }
    case kPanel: {
      const int kb = g.kb;
      const int m = nb - 1 - kb;
      if (b < m) {
        const int i = kb + 1 + b;
        product(BlockOp{blk(A, i, kb), D, 0}, BlockOp{linv(kb), NB, 1}, false);
        store_block(acc, blk(A, i, kb), D, false);
      } else {
        const int j = b - m;
        product(BlockOp{linv(kb), NB, 0}, BlockOp{blk(X, kb, j), D, 0}, false);
        if (m == 0) {
          __syncthreads();
          for_acc(acc, [&](int r, int c, double v) { Bs[r * LDP + c] = v; });
          stage(As, BlockOp{linv(kb), NB, 1});
          __syncthreads();
          mma64(As, Bs, acc);
        }
        store_block(acc, blk(X, kb, j), D, false);
      }
      break;
    }
    case kUpdate: {
      // A blocks: columns j_lo .. j_hi - 1, rows j .. nb - 1 each, column by column
      int q = b, j = g.j_lo;
      while (j < g.j_hi && q >= nb - j) {
        q -= nb - j;
        ++j;
      }
      if (j < g.j_hi) {
        const int i = j + q;
        sum_products([&](int k) { return BlockOp{blk(A, i, k), D, 0}; },
                     [&](int k) { return BlockOp{blk(A, j, k), D, 1}; });
        if (i == g.j_lo && j == g.j_lo) {  // the next diagonal block: finish it and factor it here
          __syncthreads();
          sub_to_lds(acc, blk(A, i, i), D, As);
          __syncthreads();
          fac_li = linv(i);
          fac_base = i * NB;
        } else {
          store_block(acc, blk(A, i, j), D, true);
        }
      } else {
        const int i = g.x_lo + q / nb, jx = q % nb;
        sum_products([&](int k) { return BlockOp{blk(A, i, k), D, 0}; },
                     [&](int k) { return BlockOp{blk(X, k, jx), D, 0}; });
        store_block(acc, blk(X, i, jx), D, true);
      }
      break;
    }
    case kBwd: {
      // rows diag (if in range) first, then downwards
      const int i = g.x_hi - 1 - b / nb, j = b % nb;
      sum_products([&](int k) { return BlockOp{blk(A, k, i), D, 1}; },
                   [&](int k) { return BlockOp{blk(X, k, j), D, 0}; });
      if (i == g.diag) {
        __syncthreads();
        sub_to_lds(acc, blk(X, i, j), D, Bs);
        stage(As, BlockOp{linv(i), NB, 1});
        __syncthreads();
        mma64(As, Bs, acc);
        store_block(acc, blk(X, i, j), D, false);
      } else {
        store_block(acc, blk(X, i, j), D, true);
      }
      break;
    }
  }
  if (fac_li) factor_block(As, Bs, fac_li, info + l, fac_base);
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

// one workgroup per layer: fixed-order sums of the finalize partials
__global__ __launch_bounds__(256) void eps_kernel(const double* r2, const double* lam, const int32_t* info,
                                                  const double* part, double* eps) {
  __shared__ double r1[256], r2s[256];
  const int l = blockIdx.x;
  double dot = 0.0, nrm = 0.0;
  for (int b = threadIdx.x; b < kEpsBlocks; b += 256) {
    dot += part[((int64_t)l * kEpsBlocks + b) * 2 + 0];
    nrm += part[((int64_t)l * kEpsBlocks + b) * 2 + 1];
  }
  r1[threadIdx.x] = dot;
  r2s[threadIdx.x] = nrm;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) {
      r1[threadIdx.x] += r1[threadIdx.x + off];
      r2s[threadIdx.x] += r2s[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) eps[l] = info[l] ? NAN : r2[l] - r1[0] - lam[l] * r2s[0];
}

}  // namespace

size_t solve_ws_bytes(int32_t n_layers, int32_t D) { return ws_layout(n_layers, D, nullptr, nullptr); }

// Block columns per trailing update: deeper updates cut the read-modify-write of
// the trailing blocks (which bounds large batched solves) but lengthen each
// workgroup, which a small solve feels as latency.
static int solve_group(int L, int D) {
  const double blocks = (double)L * (D / NB) * (D / NB);
  return blocks < 4096.0 ? 1 : D / NB >= 48 ? 8 : 4;
}

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
  // Block columns are taken in groups of P: inside a group the trailing update
  // covers only the group's own columns (and X block rows), and the blocks right
  // of (below) the group get the group's P columns in one update of depth P.
  const int P = solve_group(L, D);
  auto launch = [&](StepArgs g, int blocks) {
    if (blocks > 0)
      hipLaunchKernelGGL(solve_step_kernel, dim3((unsigned)blocks, (unsigned)L), dim3(256), 0, stream, g, D, s.A,
                         s.X, s.Linv, info);
  };
  auto strip = [&](int j_lo, int j_hi) {  // A blocks on or below the diagonal in columns [j_lo, j_hi)
    int n = 0;
    for (int j = j_lo; j < j_hi; ++j) n += nb - j;
    return n;
  };
  launch(StepArgs{kPotrf0, 0, 0, 0, 0, 0, 0, 0, -1}, 1);
  for (int g0 = 0; g0 < nb; g0 += P) {
    const int g1 = std::min(g0 + P, nb);
    for (int kb = g0; kb < g1; ++kb) {
      launch(StepArgs{kPanel, kb, 0, 0, 0, 0, 0, 0, -1}, (nb - 1 - kb) + nb);
      if (kb + 1 < g1)  // the rest of the group, by column kb
        launch(StepArgs{kUpdate, kb, kb, kb + 1, kb + 1, g1, kb + 1, g1, -1}, strip(kb + 1, g1) + (g1 - kb - 1) * nb);
      else if (g1 < nb)  // everything past the group, by the whole group
        launch(StepArgs{kUpdate, kb, g0, g1, g1, nb, g1, nb, -1}, strip(g1, nb) + (nb - g1) * nb);
    }
  }
  for (int g0 = (nb - 1) / P * P; g0 >= 0; g0 -= P) {
    const int g1 = std::min(g0 + P, nb);
    for (int kb = g1 - 1; kb > g0; --kb)  // rows of the group, by row kb
      launch(StepArgs{kBwd, kb, kb, kb + 1, 0, 0, g0, kb, kb - 1}, (kb - g0) * nb);
    if (g0 > 0)  // rows before the group, by the whole group
      launch(StepArgs{kBwd, g0, g0, g1, 0, 0, 0, g0, g0 - 1}, g0 * nb);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(kEpsBlocks, L), dim3(256), 0, stream, D, s.X, C, ms, info, dW, w,
                     w_dt, w_eff, s.part);
  hipLaunchKernelGGL(eps_kernel, dim3(L), dim3(256), 0, stream, r2, s.lam, info, s.part, eps);
  return check_launch("solve kernels");
}

}  // namespace ispa
