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
// update.  Small solves (one block column per update, where the launch chain's
// latency is what counts) use an explicit form instead: the forward sweep also
// carries Z = inv(L) (the identity as more right-hand sides) and adds each
// finished block row k of Y = inv(L) C to the solution as Z_k^T Y_k, so that
// dW = Z^T Y = (L L^T)^-1 C is complete when the sweep ends.  Block products are 64 x 64 x 64 fp64 MFMA tiles from LDS; a
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
  double* Z;     // [L][D][D], explicit form: inv(L) below the block diagonal
  double* XF;    // [L][D][D], explicit form: the solution inv(L)^T inv(L) C
};
constexpr int kEpsBlocks = 1024;  // finalize workgroups per layer

// Block columns per trailing update: deeper updates cut the read-modify-write of
// the trailing blocks (which bounds large batched solves) but lengthen each
// workgroup, which a small solve feels as latency.
int solve_group(int L, int D) {
  const double blocks = (double)L * (D / NB) * (D / NB);
  return blocks < 4096.0 ? 1 : D / NB >= 48 ? 8 : 4;
}

// Small solves (one block column per update) skip the backward substitution:
// the forward sweep also turns the identity into Z = inv(L) and adds each
// finished block row's share of inv(L)^T (inv(L) C) to the solution.
bool explicit_form(int L, int D) { return solve_group(L, D) == 1; }

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
  double* Z = nullptr;
  double* XF = nullptr;
  if (explicit_form(L, D)) {
    Z = (double*)take((size_t)L * D * D * 8);
    XF = (double*)take((size_t)L * D * D * 8);
  }
  if (w) *w = SolveWs{A, X, Li, lam, part, Z, XF};
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

// A block staged through registers: the loads of a thread (16 elements along
// o's contiguous dimension), then their LDS stores, so that the global loads of
// several blocks can be in flight together.
struct Staged {
  double x[NB / 4];
};
__device__ __forceinline__ Staged stage_load(BlockOp o) {
  const int t = threadIdx.x;
  const int u = t & 63, v0 = t >> 6;
  Staged r;
#pragma unroll
  for (int it = 0; it < NB / 4; ++it) r.x[it] = o.p[(int64_t)(v0 + 4 * it) * o.ld + u];
  return r;
}
// dst[r][c] = element (r, c) of o
__device__ __forceinline__ void stage_store(double* dst, const Staged& r, int trans) {
  const int t = threadIdx.x;
  const int u = t & 63, v0 = t >> 6;
#pragma unroll
  for (int it = 0; it < NB / 4; ++it) {
    const int v = v0 + 4 * it;
    if (trans)
      dst[u * LDP + v] = r.x[it];
    else
      dst[v * LDP + u] = r.x[it];
  }
}
__device__ __forceinline__ void stage(double* dst, BlockOp o) { stage_store(dst, stage_load(o), o.trans); }

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

// out (global, ld) = acc, out - acc, -acc or out + acc
enum { kStore = 0, kSub = 1, kStoreNeg = 2, kAdd = 3 };
__device__ __forceinline__ void store_block(const f64x4 (&acc)[2][2], double* out, int64_t ld, int mode) {
  for_acc(acc, [&](int r, int c, double v) {
    double* o = out + (int64_t)r * ld + c;
    *o = mode == kStore ? v : mode == kSub ? *o - v : mode == kStoreNeg ? -v : *o + v;
  });
}

// dst (LDS) = old (global) - acc
__device__ __forceinline__ void sub_to_lds(const f64x4 (&acc)[2][2], const double* old, int64_t ld, double* dst) {
  for_acc(acc, [&](int r, int c, double v) { dst[r * LDP + c] = old[(int64_t)r * ld + c] - v; });
}

// 16 x 16 x 16 product on the fp64 matrix core: acc (+)= A B for 16 x 16 blocks
// of LDS matrices with pitch LDP; A element (r, k) at a[r * LDP + k], B element
// (k, c) at b[k * bs_k + c * bs_c] (so B may be read transposed).  Lane l holds
// result rows l / 16 + 4 e, column l % 16.
__device__ __forceinline__ f64x4 prod16(const double* a, const double* b, int bs_k, int bs_c, f64x4 acc) {
  const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const double av = a[li * LDP + 4 * ks + lk];
    const double bv = b[(4 * ks + lk) * bs_k + li * bs_c];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
  }
  return acc;
}

// Workgroup barrier that orders LDS only: the global stores of the inverse
// blocks stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Lane l's value of x (any lane, active or not), as a wave-uniform value.
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Inverse of the Cholesky factor of the SPD 64 x 64 block M (LDS, pitch LDP),
// by the workgroup's four waves, blocked in 16 x 16 blocks (k = 0 .. 3):
//   * the first wave's lanes 0..15 factor the diagonal block M_kk and invert
//     its factor at once: lane a holds column a, and at step j every lane
//     publishes its entry of row j to LDS and reads the row back (the trailing
//     row is also the column of multipliers) while the pivot comes straight
//     from lane j (readlane), so the reciprocal does not wait for the LDS round
//     trip; lane j stops updating at its own pivot, after
//     which its entries are column j of the inverse unit factor times
//     -pivot_j, updated by the same formula; the rows are scaled by
//     1/sqrt(pivot) at the end.  The result I_k goes to the diagonal block of X;
//   * the panel L_ik = M_ik I_k^T (i > k, one block per wave) and the trailing
//     update M_ij -= L_ik L_jk^T (k < j <= i) on the fp64 matrix core;
// then the strictly lower blocks of the inverse from the 2 x 2 split into
// 32 x 32 halves, inv([[A, 0], [B, C]]) = [[A^-1, 0], [-C^-1 B A^-1, C^-1]]:
//   stage 1: X_10 = -I_1 L_10 I_0, X_32 = -I_3 L_32 I_2, T01 = L_21 I_1,
//            T11 = L_31 I_1 and the first terms of T00 and T10 (T = B A^-1);
//   stage 2: T00 = L_20 I_0 + L_21 X_10, T10 = L_30 I_0 + L_31 X_10;
//   stage 3: X_20 = -I_2 T00, X_21 = -I_2 T01, X_30 = -(X_32 T00 + I_3 T10),
//            X_31 = -(X_32 T01 + I_3 T11);
// five block products on the longest path.  T lives in the unused upper blocks
// of X.  Every block of the inverse goes to Li (row-major, 64 wide; zeros above
// the block diagonal, NaN everywhere if a pivot failed) as soon as it is final.
// M is overwritten (its lower blocks become L); X: 64 x 64 doubles of LDS
// (pitch LDP).  Returns the first non-positive pivot (1-based) or 0.  Every
// thread of the workgroup must call it.
__device__ __forceinline__ int chol_inv64(double* M, double* X, double* Li) {
  __shared__ double rowb[2][16], isq_s[16];
  __shared__ int bad_s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lk = lane >> 4;
  auto blk = [&](double* base, int bi, int bj) { return base + (16 * bi) * LDP + 16 * bj; };
  if (tid == 0) bad_s = 0;
  for (int k = 0; k < 4; ++k) {
    if (w == 0 && lane < 16) {
      const double* Mkk = blk(M, k, k);
      double col[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) col[i] = Mkk[i * LDP + lane];
      int bad = 0;
      double my_ea = 0.0, piv_a = 0.0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // row j to LDS for the update; the pivot straight from lane j, so
        // that the reciprocal starts while the row is in flight
        double* rb = rowb[j & 1];
        rb[lane] = col[j];
        double r[16];
#pragma unroll
        for (int i = j + 1; i < 16; ++i) r[i] = rb[i];
        // the row's reads are in flight before the reciprocal chain starts
        __builtin_amdgcn_sched_barrier(0);
        const double piv = readlane_f64(col[j], j);
        if (lane == j) piv_a = piv;
        if (!(piv > 0.0) && bad == 0) bad = j + 1;
        // 1 / piv by the hardware reciprocal and two Newton steps (about 1 ulp;
        // a shorter chain than the IEEE division on the serial path)
        double inv = __builtin_amdgcn_rcp(piv);
        inv = fma(inv, fma(-piv, inv, 1.0), inv);
        inv = fma(inv, fma(-piv, inv, 1.0), inv);
        const double sc = lane == j ? 0.0 : col[j] * inv;
        if (lane == j) my_ea = -inv;
#pragma unroll
        for (int i = j + 1; i < 16; ++i) col[i] = fma(-r[i], sc, col[i]);
      }
      // rows scaled by 1 / sqrt(pivot) once the elimination is done (off the
      // serial path): lane a forms the factor of pivot a and publishes it
      isq_s[lane] = 1.0 / sqrt(piv_a);
      double* Xkk = blk(X, k, k);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double isq = isq_s[i];
        Xkk[i * LDP + lane] = i < lane ? 0.0 : (i == lane ? isq : col[i] * isq * my_ea);
      }
      if (bad && lane == 0 && bad_s == 0) bad_s = 16 * k + bad;
    }
    __syncthreads();  // I_k is in X
    if (k == 3) break;
    if (w < 3 - k) {  // panel: L_ik = M_ik I_k^T
      const int i = k + 1 + w;
      const f64x4 acc = prod16(blk(M, i, k), blk(X, k, k), 1, LDP, (f64x4){0.0, 0.0, 0.0, 0.0});
      double* Lik = blk(M, i, k);
#pragma unroll
      for (int e = 0; e < 4; ++e) Lik[(lk + 4 * e) * LDP + li] = acc[e];
    }
    __syncthreads();  // the panel is in M
    int idx = 0;  // trailing blocks (i, j), k < j <= i, round-robin over the waves
    for (int j = k + 1; j < 4; ++j)
      for (int i = j; i < 4; ++i, ++idx) {
        if (idx % 4 != w) continue;
        const f64x4 acc = prod16(blk(M, i, k), blk(M, j, k), 1, LDP, (f64x4){0.0, 0.0, 0.0, 0.0});
        double* Mij = blk(M, i, j);
#pragma unroll
        for (int e = 0; e < 4; ++e) Mij[(lk + 4 * e) * LDP + li] -= acc[e];
      }
    __syncthreads();  // the trailing blocks are updated
  }
  const int bad = bad_s;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  // this lane's elements of block (bi, bj) of Li
  auto put = [&](int bi, int bj, const f64x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Li[(16 * bi + lk + 4 * e) * NB + 16 * bj + li] = bad ? NAN : v[e];
  };
  auto put_lds = [&](double* b, const f64x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) b[(lk + 4 * e) * LDP + li] = v[e];
  };
  // the diagonal blocks and the zero blocks above them
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, a = e % NB;
    if ((i >> 4) <= (a >> 4)) Li[e] = bad ? NAN : ((i >> 4) < (a >> 4) ? 0.0 : X[i * LDP + a]);
  }
  double* T00 = blk(X, 0, 2);
  double* T01 = blk(X, 0, 3);
  double* T10 = blk(X, 1, 2);
  double* T11 = blk(X, 1, 3);
  f64x4 part = zero;
  if (w == 0) {
    put_lds(blk(X, 1, 0), prod16(blk(M, 1, 0), blk(X, 0, 0), LDP, 1, zero));  // L_10 I_0, then X_10 in its place
    const f64x4 x10 = -prod16(blk(X, 1, 1), blk(X, 1, 0), LDP, 1, zero);
    put_lds(blk(X, 1, 0), x10);
    put(1, 0, x10);
  } else if (w == 1) {
    put_lds(blk(X, 3, 2), prod16(blk(M, 3, 2), blk(X, 2, 2), LDP, 1, zero));
    const f64x4 x32 = -prod16(blk(X, 3, 3), blk(X, 3, 2), LDP, 1, zero);
    put_lds(blk(X, 3, 2), x32);
    put(3, 2, x32);
  } else if (w == 2) {
    put_lds(T01, prod16(blk(M, 2, 1), blk(X, 1, 1), LDP, 1, zero));
    part = prod16(blk(M, 2, 0), blk(X, 0, 0), LDP, 1, zero);
  } else {
    put_lds(T11, prod16(blk(M, 3, 1), blk(X, 1, 1), LDP, 1, zero));
    part = prod16(blk(M, 3, 0), blk(X, 0, 0), LDP, 1, zero);
  }
  lds_barrier();  // X_10, X_32, T01, T11 are in X
  if (w == 2) put_lds(T00, prod16(blk(M, 2, 1), blk(X, 1, 0), LDP, 1, part));
  if (w == 3) put_lds(T10, prod16(blk(M, 3, 1), blk(X, 1, 0), LDP, 1, part));
  lds_barrier();  // T00 and T10 are in X
  if (w == 0) {
    put(2, 0, -prod16(blk(X, 2, 2), T00, LDP, 1, zero));
  } else if (w == 1) {
    put(2, 1, -prod16(blk(X, 2, 2), T01, LDP, 1, zero));
  } else if (w == 2) {
    put(3, 0, -prod16(blk(X, 3, 3), T10, LDP, 1, prod16(blk(X, 3, 2), T00, LDP, 1, zero)));
  } else {
    put(3, 1, -prod16(blk(X, 3, 3), T11, LDP, 1, prod16(blk(X, 3, 2), T01, LDP, 1, zero)));
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
  int z;  // explicit form (one block column per update, contraction block kb)
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
// Explicit form (z): the panel also finishes block row kb of Z = inv(L),
// Z_kb,j = inv(L_kk) Z_kb,j for j < kb (Z_kk = inv(L_kk) is kept in Li), and
// does not apply inv(L)^T to the last row; the update also carries Z,
// Z_ij -= L_ik Z_kj for i > k, j <= k (the first touch of Z_ik stores
// -L_ik inv(L_kk)), and adds the finished row k to the solution,
// XF_ij += Z_ki^T X_kj for i <= k (the first touch, i = k, stores).  A last
// update with no trailing, X or Z blocks adds row nb - 1.
// Diagonal blocks keep only inv(L_kk) (in Li); the strictly lower blocks of A
// become L.  Every launch writes blocks that no other workgroup of it reads.
__global__ __launch_bounds__(256, 2) void solve_step_kernel(StepArgs g, int D, double* Aall, double* Xall,
                                                           double* Liall, int32_t* info, double* Zall,
                                                           double* XFall) {
  __shared__ double As[NB * LDP], Bs[NB * LDP];
  const int l = blockIdx.y;
  const int nb = D / NB;
  const int b = blockIdx.x;
  double* A = Aall + (int64_t)l * D * D;
  double* X = Xall + (int64_t)l * D * D;
  double* Z = g.z ? Zall + (int64_t)l * D * D : nullptr;
  double* XF = g.z ? XFall + (int64_t)l * D * D : nullptr;
  double* Li = Liall + (int64_t)l * D * NB;
  auto blk = [&](double* M, int bi, int bj) { return M + (int64_t)bi * NB * D + (int64_t)bj * NB; };
  auto linv = [&](int k) { return Li + (int64_t)k * NB * NB; };
  f64x4 acc[2][2] = {};
  double* fac_li = nullptr;  // set when this workgroup factors a diagonal block (in As)
  int fac_base = 0;
  auto product = [&](BlockOp x, BlockOp y, bool accumulate) {
    const Staged sx = stage_load(x), sy = stage_load(y);  // both blocks' loads in flight together
    stage_store(As, sx, x.trans);
    stage_store(Bs, sy, y.trans);
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
        store_block(acc, blk(A, i, kb), D, kStore);
      } else if (b >= m + nb) {  // explicit form: Z_kb,j for j < kb
        const int j = b - m - nb;
        product(BlockOp{linv(kb), NB, 0}, BlockOp{blk(Z, kb, j), D, 0}, false);
        store_block(acc, blk(Z, kb, j), D, kStore);
      } else {
        const int j = b - m;
        product(BlockOp{linv(kb), NB, 0}, BlockOp{blk(X, kb, j), D, 0}, false);
        if (m == 0 && !g.z) {
          __syncthreads();
          for_acc(acc, [&](int r, int c, double v) { Bs[r * LDP + c] = v; });
          stage(As, BlockOp{linv(kb), NB, 1});
          __syncthreads();
          mma64(As, Bs, acc);
        }
        store_block(acc, blk(X, kb, j), D, kStore);
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
        const bool fac = i == g.j_lo && j == g.j_lo;  // the next diagonal block: finish it and factor it here
        double old[16];  // its elements at this thread's product positions, loaded ahead of the product
        if (fac) {
          int e = 0;
          for_acc(acc, [&](int r, int c, double) { old[e++] = blk(A, i, i)[(int64_t)r * D + c]; });
        }
        sum_products([&](int k) { return BlockOp{blk(A, i, k), D, 0}; },
                     [&](int k) { return BlockOp{blk(A, j, k), D, 1}; });
        if (fac) {
          __syncthreads();
          int e = 0;
          for_acc(acc, [&](int r, int c, double v) { As[r * LDP + c] = old[e++] - v; });
          __syncthreads();
          fac_li = linv(i);
          fac_base = i * NB;
        } else {
          store_block(acc, blk(A, i, j), D, kSub);
        }
        break;
      }
      const int nx = (g.x_hi - g.x_lo) * nb;
      if (q < nx) {
        const int i = g.x_lo + q / nb, jx = q % nb;
        sum_products([&](int k) { return BlockOp{blk(A, i, k), D, 0}; },
                     [&](int k) { return BlockOp{blk(X, k, jx), D, 0}; });
        store_block(acc, blk(X, i, jx), D, kSub);
        break;
      }
      // explicit form, contraction block k = kb
      q -= nx;
      const int k = g.kb, nz = (nb - 1 - k) * (k + 1);
      if (q < nz) {  // Z_i,jz -= L_ik Z_k,jz for i > k, jz <= k
        const int i = k + 1 + q / (k + 1), jz = q % (k + 1);
        product(BlockOp{blk(A, i, k), D, 0}, jz == k ? BlockOp{linv(k), NB, 0} : BlockOp{blk(Z, k, jz), D, 0},
                false);
        store_block(acc, blk(Z, i, jz), D, jz == k ? kStoreNeg : kSub);
        break;
      }
      q -= nz;
      {  // XF_i,jx += Z_k,i^T X_k,jx for i <= k
        const int i = q / nb, jx = q % nb;
        product(i == k ? BlockOp{linv(k), NB, 1} : BlockOp{blk(Z, k, i), D, 1}, BlockOp{blk(X, k, jx), D, 0},
                false);
        store_block(acc, blk(XF, i, jx), D, i == k ? kStore : kAdd);
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
        store_block(acc, blk(X, i, j), D, kStore);
      } else {
        store_block(acc, blk(X, i, j), D, kSub);
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
  const int z = explicit_form(L, D) ? 1 : 0;
  auto launch = [&](StepArgs g, int blocks) {
    g.z = z;
    if (blocks > 0)
      hipLaunchKernelGGL(solve_step_kernel, dim3((unsigned)blocks, (unsigned)L), dim3(256), 0, stream, g, D, s.A,
                         s.X, s.Linv, info, s.Z, s.XF);
  };
  auto strip = [&](int j_lo, int j_hi) {  // A blocks on or below the diagonal in columns [j_lo, j_hi)
    int n = 0;
    for (int j = j_lo; j < j_hi; ++j) n += nb - j;
    return n;
  };
  // explicit form: the Z and solution blocks an update by block column kb adds
  auto zx = [&](int kb) { return z ? (nb - 1 - kb) * (kb + 1) + (kb + 1) * nb : 0; };
  launch(StepArgs{kPotrf0, 0, 0, 0, 0, 0, 0, 0, -1}, 1);
  for (int g0 = 0; g0 < nb; g0 += P) {
    const int g1 = std::min(g0 + P, nb);
    for (int kb = g0; kb < g1; ++kb) {
      launch(StepArgs{kPanel, kb, 0, 0, 0, 0, 0, 0, -1}, (nb - 1 - kb) + nb + (z ? kb : 0));
      if (kb + 1 < g1)  // the rest of the group, by column kb
        launch(StepArgs{kUpdate, kb, kb, kb + 1, kb + 1, g1, kb + 1, g1, -1}, strip(kb + 1, g1) + (g1 - kb - 1) * nb);
      else if (g1 < nb)  // everything past the group, by the whole group
        launch(StepArgs{kUpdate, kb, g0, g1, g1, nb, g1, nb, -1}, strip(g1, nb) + (nb - g1) * nb + zx(kb));
    }
  }
  if (z)  // the last block row's share of the solution
    launch(StepArgs{kUpdate, nb - 1, nb - 1, nb, nb, nb, nb, nb, -1}, zx(nb - 1));
  for (int g0 = (nb - 1) / P * P; g0 >= 0 && !z; g0 -= P) {
    const int g1 = std::min(g0 + P, nb);
    for (int kb = g1 - 1; kb > g0; --kb)  // rows of the group, by row kb
      launch(StepArgs{kBwd, kb, kb, kb + 1, 0, 0, g0, kb, kb - 1}, (kb - g0) * nb);
    if (g0 > 0)  // rows before the group, by the whole group
      launch(StepArgs{kBwd, g0, g0, g1, 0, 0, 0, g0, g0 - 1}, g0 * nb);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(kEpsBlocks, L), dim3(256), 0, stream, D, z ? s.XF : s.X, C, ms, info,
                     dW, w, w_dt, w_eff, s.part);
  hipLaunchKernelGGL(eps_kernel, dim3(L), dim3(256), 0, stream, r2, s.lam, info, s.part, eps);
  return check_launch("solve kernels");
}

}  // namespace ispa
