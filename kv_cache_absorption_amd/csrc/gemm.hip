// MFMA tile GEMM for the regression statistics and the output projection.
//
// A workgroup computes a 128 x 128 tile of acc[m][n] = sum_k X[m][k] Y[n][k]
// with 4 waves in a 2 x 2 grid, each wave 64 x 64 = 2 x 2 tiles of
// v_mfma_f32_32x32x16_{bf16,f16}.  Both operands are staged in LDS as
// [row][k] (k contiguous, rows padded to 40 elements so the 16-byte fragment
// reads of 16 lanes hit distinct banks).  Operands whose memory layout is
// [k][row] are transposed on the way in: each thread gathers one 32-bit pair
// of rows for 8 consecutive k and writes two 16-byte rows.  Stages of 32 k
// are double-buffered; the next stage's global loads are in flight during the
// current stage's MFMAs.
//
// The statistics contract over token rows (G = A^T A, C = A^T R), which is
// the strided direction of the row-major activations, hence the transposing
// loader; R is written transposed by the producing GEMM so the C product
// reads it directly.
#include "gemm.hpp"

namespace ispa {

namespace {

constexpr int LDS_STRIDE = kGemmBK + 8;  // 40 elements

template <int MT>
__device__ __forceinline__ uint32_t to_pair(float a, float b) {
  return MT == ISPA_BF16 ? pack_bf16(a, b) : pack_f16(a, b);
}
__device__ __forceinline__ float half_to_f32(uint32_t bits, int dt) {
  return dt == ISPA_BF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
}

// Registers holding one stage of one operand (128 rows x 32 k) for this
// thread.  XL: layout (kDirect / kTrans); F32: the source holds fp32.
template <int XL, bool F32>
struct StageRegs;
template <>
struct StageRegs<kDirect, false> {
  u32x4 v[2];
};
template <>
struct StageRegs<kDirect, true> {
  f32x4 v[4];
};
template <>
struct StageRegs<kTrans, false> {
  uint32_t v[8];
};

template <int XL, bool F32>
__device__ __forceinline__ void load_stage(const void* base, int64_t ld, int64_t rows_total, int64_t K,
                                           int64_t row0, int64_t k0, int tid, StageRegs<XL, F32>& s) {
  if constexpr (XL == kDirect) {
    // 2 chunks of 8 k per thread: chunk c -> row c/4, k 8*(c%4)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int64_t row = row0 + (c >> 2);
      const int64_t k = k0 + (c & 3) * 8;
      if constexpr (F32) {
        const float* src = (const float*)base + row * ld + k;
        f32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (row < rows_total) {
          if (k + 8 <= K) {
            a = *(const f32x4*)src;
            b = *(const f32x4*)(src + 4);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (k + e < K) a[e] = src[e];
              if (k + 4 + e < K) b[e] = src[4 + e];
            }
          }
        }
        s.v[2 * i] = a;
        s.v[2 * i + 1] = b;
      } else {
        const uint16_t* src = (const uint16_t*)base + row * ld + k;
        u32x4 v = {0, 0, 0, 0};
        if (row < rows_total) {
          if (k + 8 <= K) {
            v = *(const u32x4*)src;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = (k + 2 * e < K) ? (uint32_t)src[2 * e] : 0u;
              const uint32_t hi = (k + 2 * e + 1 < K) ? (uint32_t)src[2 * e + 1] : 0u;
              v[e] = lo | (hi << 16);
            }
          }
        }
        s.v[i] = v;
      }
    }
  } else {
    // transposed source [k][row]: item = (row pair rp, k group kg)
    const int rp = tid & 63, kg = tid >> 6;
    const int64_t row = row0 + 2 * rp;
    const uint16_t* src = (const uint16_t*)base + row;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = k0 + kg * 8 + j;
      uint32_t v = 0;
      if (k < K && row < rows_total) v = *(const uint32_t*)(src + k * ld);
      s.v[j] = v;
    }
  }
}

// 16-bit pair (lo, hi) of type dt -> pair of type MT
template <int MT>
__device__ __forceinline__ uint32_t conv_pair(uint32_t w, int dt) {
  if (dt == MT) return w;
  return to_pair<MT>(half_to_f32(w & 0xffffu, dt), half_to_f32(w >> 16, dt));
}

template <int MT, int XL, bool F32>
__device__ __forceinline__ void store_stage(int dt, int tid, const StageRegs<XL, F32>& s, uint16_t* lds) {
  if constexpr (XL == kDirect) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      u32x4 v;
      if constexpr (F32) {
        const f32x4 a = s.v[2 * i], b = s.v[2 * i + 1];
        v[0] = to_pair<MT>(a[0], a[1]);
        v[1] = to_pair<MT>(a[2], a[3]);
        v[2] = to_pair<MT>(b[0], b[1]);
        v[3] = to_pair<MT>(b[2], b[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = conv_pair<MT>(s.v[i][e], dt);
      }
      *(u32x4*)(lds + (c >> 2) * LDS_STRIDE + (c & 3) * 8) = v;
    }
  } else {
    const int rp = tid & 63, kg = tid >> 6;
    u32x4 lo, hi;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = conv_pair<MT>(s.v[2 * m], dt), b = conv_pair<MT>(s.v[2 * m + 1], dt);
      lo[m] = (a & 0xffffu) | (b << 16);
      hi[m] = (a >> 16) | (b & 0xffff0000u);
    }
    *(u32x4*)(lds + (2 * rp) * LDS_STRIDE + kg * 8) = lo;
    *(u32x4*)(lds + (2 * rp + 1) * LDS_STRIDE + kg * 8) = hi;
  }
}

template <int MT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (MT == ISPA_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

template <int MT, int XL, bool XF32, int YL>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kGemmBM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[2][kGemmBN * LDS_STRIDE];
  __shared__ double red[4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hh = lane >> 5, lq = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- which tile and which K range: blocks are (split, tile) with the tile
  // fastest, so the workgroups sharing an XCD work on neighbouring tiles
  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t n_kind0 = p.tri ? (uint32_t)(p.tiles_m * (p.tiles_m + 1) / 2) : (uint32_t)(p.tiles_m * p.tiles_n);
  const uint32_t n_tiles = n_kind0 + (p.two_kinds ? (uint32_t)(p.tiles_m * p.tiles_n) : 0u);
  const uint32_t split = bid / n_tiles;
  uint32_t t = bid - split * n_tiles;
  const bool kind1 = t >= n_kind0;
  if (kind1) t -= n_kind0;
  int tm, tn;
  if (p.tri && !kind1) {
    // upper-triangle tiles (tm <= tn), row by row
    tm = 0;
    while (t >= (uint32_t)(p.tiles_n - tm)) {
      t -= p.tiles_n - tm;
      ++tm;
    }
    tn = tm + (int)t;
  } else {
    tm = t / p.tiles_n;
    tn = t % p.tiles_n;
  }
  const void* yp = kind1 ? p.y2.p : p.y.p;
  const int64_t yld = kind1 ? p.y2.ld : p.y.ld;
  const int64_t m0 = (int64_t)tm * kGemmBM, n0 = (int64_t)tn * kGemmBN;
  const int64_t kb = (int64_t)split * p.kchunk;
  const int64_t ke = min(p.K, kb + p.kchunk);
  const int nk = ke > kb ? (int)((ke - kb + kGemmBK - 1) / kGemmBK) : 0;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

  StageRegs<XL, XF32> xr;
  StageRegs<YL, false> yr;
  if (nk > 0) {
    load_stage(p.x.p, p.x.ld, p.M, ke, m0, kb, tid, xr);
    load_stage(yp, yld, p.N, ke, n0, kb, tid, yr);
    store_stage<MT>(p.x.dt, tid, xr, Xs[0]);
    store_stage<MT>(p.y.dt, tid, yr, Ys[0]);
  }
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const bool next = kt + 1 < nk;
    if (next) {
      load_stage(p.x.p, p.x.ld, p.M, ke, m0, kb + (int64_t)(kt + 1) * kGemmBK, tid, xr);
      load_stage(yp, yld, p.N, ke, n0, kb + (int64_t)(kt + 1) * kGemmBK, tid, yr);
    }
    const uint16_t* xs = Xs[buf];
    const uint16_t* ys = Ys[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const u32x4*)(xs + (wm * 64 + i * 32 + lq) * LDS_STRIDE + ks * 16 + hh * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *(const u32x4*)(ys + (wn * 64 + j * 32 + lq) * LDS_STRIDE + ks * 16 + hh * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<MT>(a[i], b[j], acc[i][j]);
    }
    if (next) {
      store_stage<MT>(p.x.dt, tid, xr, Xs[buf ^ 1]);
      store_stage<MT>(p.y.dt, tid, yr, Ys[buf ^ 1]);
    }
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue
  if (p.epi == kStoreRt) {
    // R row-major as 16-bit (mfma type), plus this workgroup's sum of squares
    double ss = 0.0;
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + j * 32 + lq;
        float ssf = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + hh * 4 + (e & 3);
          if (m < p.M && n < p.N) {
            const float v = acc[i][j][e];
            out[m * p.ld_out + n] = (uint16_t)(to_pair<MT>(v, 0.0f) & 0xffffu);
            ssf += v * v;
          }
        }
        ss += (double)ssf;
      }
    }
    // workgroup sum of squares
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (tid == 0) p.sq_partials[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    return;
  }

  float* outf = (float*)(kind1 ? p.out2 : p.out);
  const bool tri_tile = p.tri && !kind1;
  const bool atomic = p.ksplit > 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + lq;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + hh * 4 + (e & 3);
        if (m >= p.M || n >= p.N) continue;
        if (p.epi == kAccum) {
          if (tri_tile && m > n) continue;
          if (atomic)
            unsafeAtomicAdd(outf + m * p.ld_out + n, acc[i][j][e]);
          else
            outf[m * p.ld_out + n] += acc[i][j][e];
        } else {
          store_from_f32(p.out, m * p.ld_out + n, acc[i][j][e], p.out_dt);
        }
      }
    }
  }
}

// ---- fp32 parity-mode kernels -------------------------------------------------
__global__ void r_f32_kernel(int64_t n, int D, const float* dl, const float* w, float* R) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * D) return;
  const int64_t r = gid / D;
  const int j = gid % D;
  float acc = 0.0f;
  for (int k = 0; k < D; ++k) acc = fmaf(dl[r * D + k], w[(int64_t)k * D + j], acc);
  R[gid] = acc;
}

__global__ void sumsq_f32_kernel(int64_t total, const float* R, double* partials) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    s += (double)R[i] * (double)R[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) partials[blockIdx.x] = red[0];
}

__global__ void gc_f32_kernel(int64_t n, int D, const float* a, const float* R, float* G, float* C) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)D * D) return;
  const int i = gid / D, j = gid % D;
  float g = 0.0f, c = 0.0f;
  for (int64_t r = 0; r < n; ++r) {
    const float ai = a[r * D + i];
    g = fmaf(ai, a[r * D + j], g);
    c = fmaf(ai, R[r * D + j], c);
  }
  if (i <= j) G[gid] += g;
  C[gid] += c;
}

__global__ void proj_f32_kernel(int64_t n, int D, const float* x, const float* w, void* y, int y_dt) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * D) return;
  const int64_t r = gid / D;
  const int j = gid % D;
  float acc = 0.0f;
  for (int k = 0; k < D; ++k) acc = fmaf(x[r * D + k], w[(int64_t)k * D + j], acc);
  store_from_f32(y, gid, acc, y_dt);
}

__global__ void reduce_add_kernel(const double* partials, int64_t n, double* r2) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += partials[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *r2 += red[0];
}

}  // namespace

ispa_status launch_gemm(const GemmParams& p, int mfma_dt, hipStream_t stream, int* n_blocks_out) {
  const int64_t n0 = p.tri ? (int64_t)p.tiles_m * (p.tiles_m + 1) / 2 : (int64_t)p.tiles_m * p.tiles_n;
  const int64_t blocks = (n0 + (p.two_kinds ? (int64_t)p.tiles_m * p.tiles_n : 0)) * p.ksplit;
  if (n_blocks_out) *n_blocks_out = (int)blocks;
  if (p.ksplit < 1 || p.kchunk % kGemmBK || (int64_t)p.ksplit * p.kchunk < p.K) {
    set_error("gemm: bad K split");
    return ISPA_ERR_INVALID_ARG;
  }
  if (blocks == 0) return ISPA_OK;
  const bool xf32 = p.x.dt == ISPA_F32;
  if (p.x.layout == kTrans && (xf32 || p.y.dt == ISPA_F32)) {
    set_error("gemm: transposed fp32 operands are not supported");
    return ISPA_ERR_UNSUPPORTED;
  }
#define ISPA_GEMM_LAUNCH(MT, XL, XF, YL) \
  hipLaunchKernelGGL((gemm_kernel<MT, XL, XF, YL>), dim3((unsigned)blocks), dim3(256), 0, stream, p)
#define ISPA_GEMM_BY_MT(XL, XF, YL)              \
  do {                                          \
    if (mfma_dt == ISPA_BF16)                   \
      ISPA_GEMM_LAUNCH(ISPA_BF16, XL, XF, YL);  \
    else                                        \
      ISPA_GEMM_LAUNCH(ISPA_F16, XL, XF, YL);   \
  } while (0)
  if (p.x.layout == kDirect && xf32 && p.y.layout == kTrans) ISPA_GEMM_BY_MT(kDirect, true, kTrans);
  else if (p.x.layout == kDirect && !xf32 && p.y.layout == kTrans) ISPA_GEMM_BY_MT(kDirect, false, kTrans);
  else if (p.x.layout == kTrans && p.y.layout == kTrans) ISPA_GEMM_BY_MT(kTrans, false, kTrans);
  else if (p.x.layout == kTrans && p.y.layout == kDirect && p.y.dt != ISPA_F32) ISPA_GEMM_BY_MT(kTrans, false, kDirect);
  else {
    set_error("gemm: operand layout combination not built");
    return ISPA_ERR_UNSUPPORTED;
  }
#undef ISPA_GEMM_BY_MT
#undef ISPA_GEMM_LAUNCH
  return check_launch("gemm_kernel");
}

ispa_status launch_reduce_add(const double* partials, int64_t n, double* r2, hipStream_t stream) {
  hipLaunchKernelGGL(reduce_add_kernel, dim3(1), dim3(256), 0, stream, partials, n, r2);
  return check_launch("reduce_add_kernel");
}

ispa_status launch_stats_f32(int64_t n, int32_t D, const float* a, const float* dl, const float* w,
                             float* G, float* C, double* r2, void* ws, hipStream_t stream) {
  float* R = (float*)ws;
  double* partials = (double*)((char*)ws + align256((size_t)n * D * 4));
  const int64_t tot = n * D;
  if (tot > 0) {
    hipLaunchKernelGGL(r_f32_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, n, D, dl, w, R);
    hipLaunchKernelGGL(sumsq_f32_kernel, dim3(64), dim3(256), 0, stream, tot, R, partials);
    hipLaunchKernelGGL(reduce_add_kernel, dim3(1), dim3(256), 0, stream, partials, (int64_t)64, r2);
    hipLaunchKernelGGL(gc_f32_kernel, dim3((unsigned)(((int64_t)D * D + 255) / 256)), dim3(256), 0, stream,
                       n, D, a, R, G, C);
  }
  return check_launch("stats f32 kernels");
}

ispa_status launch_proj_f32(int64_t n, int32_t D, const float* x, const float* w, void* y,
                            int32_t y_dt, hipStream_t stream) {
  const int64_t tot = n * D;
  if (tot == 0) return ISPA_OK;
  hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, n, D, x, w,
                     y, y_dt);
  return check_launch("proj_f32_kernel");
}

}  // namespace ispa
