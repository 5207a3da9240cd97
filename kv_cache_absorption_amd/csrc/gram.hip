// K-contiguous MFMA GEMM ("NT": acc[m][n] = sum_k X[m][k] Y[n][k], both operands
// stored with k contiguous) for the regression statistics, and the transpose
// that produces such operands.
//
// The statistics contract over token rows (G = A^T A, C = A^T R) and over the
// input width (R = dA W).  Transposing A_loc and W once per call into the
// workspace, and writing R transposed, turns every product into this NT form so
// both operands can be moved straight from global memory into LDS:
//   * 128 x 128 output tile per workgroup, 4 waves as 2 x 2, each 64 x 64
//     = 2 x 2 tiles of v_mfma_f32_32x32x16_{f16,bf16};
//   * K stages of 32: each operand tile is 128 rows x 64 bytes in LDS, filled by
//     buffer loads with the LDS flag (16 bytes per lane, no VGPR staging), two
//     stages ahead in a ring of four (64 KB, so two workgroups share a CU and
//     hide each other's LDS latency); one barrier per stage;
//   * 16-byte chunks of a row are XOR-swizzled with (row / 4) mod 4 so the
//     16-byte fragment reads of 16 consecutive rows use 16 distinct bank groups;
//   * the fragments of the next 16-wide k slice are read while the MFMAs of the
//     current one run;
//   * operand rows past the matrix reload the last valid row (results there
//     are discarded); the token dimension is zero-padded to a multiple of 32 so
//     no K masking is needed.
#include "gram.hpp"

#include <algorithm>

namespace ispa {

namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int NBUF = 4, PD = 2;          // ring slots; stages loaded ahead
constexpr int ROWB = BK * 2;              // bytes per tile row (64)
constexpr int RPI = 1024 / ROWB;          // rows per 1 KB load instruction (16)
constexpr int TILEB = BM * ROWB;          // 8 KB per operand tile
constexpr int LPW = TILEB / 1024 / 4;     // 1 KB load instructions per wave per operand (2)
constexpr int LOADS_PER_STAGE = 2 * LPW;  // per wave

__device__ __forceinline__ int gswz(int row, int ch) { return ch ^ ((row >> 2) & 3); }

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_off, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_off), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_stage(bool one_newer) {
  if (one_newer)
    __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_PER_STAGE);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int MT>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (MT == ISPA_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

template <int MT>
__global__ __launch_bounds__(256, 2) void nt_gemm_kernel(const NtGemmParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * 2 * TILEB];
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hh = lane >> 5, lq = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile: (split, tile) with the tile fastest; first-kind tiles may be an
  // upper triangle, second-kind tiles a full grid with another y operand
  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t n_kind0 = p.tri ? (uint32_t)(p.tiles_m * (p.tiles_m + 1) / 2) : (uint32_t)(p.tiles_m * p.tiles_n);
  const uint32_t n_tiles = n_kind0 + (p.two_kinds ? (uint32_t)(p.tiles_m * p.tiles_n) : 0u);
  const uint32_t split = bid / n_tiles;
  uint32_t t = bid - split * n_tiles;
  const bool kind1 = t >= n_kind0;
  if (kind1) t -= n_kind0;
  int tm, tn;
  if (p.tri && !kind1) {
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
  const char* yp = (const char*)(kind1 ? p.y2 : p.y);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = (int64_t)split * p.kchunk;
  const int64_t ke = min(p.K, kb + p.kchunk);
  const int ns = ke > kb ? (int)((ke - kb) / BK) : 0;  // K is a multiple of BK

  // ---- operand sources: rows of 2*ld bytes; rows past the end reload the last one
  const int64_t xrows = p.M, yrows = p.y_rows;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)p.x + m0 * p.ldx * 2), 0, (int)(min<int64_t>(BM, xrows - m0) * p.ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(yp + n0 * p.ldy * 2), 0, (int)(min<int64_t>(BN, yrows - n0) * p.ldy * 2), 0x00020000);
  int xo[LPW], yo[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (wave * LPW + i) * RPI + lane / (ROWB / 16);  // RPI rows per 1 KB instruction
    const int slot = lane % (ROWB / 16);
    const int ch = gswz(row, slot);
    const int xr = (int)min<int64_t>(row, xrows - m0 - 1), yr = (int)min<int64_t>(row, yrows - n0 - 1);
    xo[i] = xr * (int)(p.ldx * 2) + ch * 16;
    yo[i] = yr * (int)(p.ldy * 2) + ch * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds;
  auto issue = [&](int s, int buf) {
    const int soff = (int)((kb + (int64_t)s * BK) * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const uint32_t dst = (wave * LPW + i) * 1024;
      lds_dma16(rx, lds0 + (buf * 2 + 0) * TILEB + dst, xo[i], soff);
      lds_dma16(ry, lds0 + (buf * 2 + 1) * TILEB + dst, yo[i], soff);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

  int issued = 0, lbuf = 0;
  for (; issued < PD && issued < ns; ++issued) {
    issue(issued, lbuf);
    lbuf = lbuf + 1 == NBUF ? 0 : lbuf + 1;
  }
  wait_stage(issued > 1);
  __syncthreads();

  int cbuf = 0;
  for (int s = 0; s < ns; ++s) {
    if (issued < ns) {
      issue(issued, lbuf);
      lbuf = lbuf + 1 == NBUF ? 0 : lbuf + 1;
      ++issued;
    }
    const char* xs = lds + (cbuf * 2 + 0) * TILEB;
    const char* ys = lds + (cbuf * 2 + 1) * TILEB;
    auto frags = [&](int ks, u32x4 (&a)[2], u32x4 (&b)[2]) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + lq;
        a[i] = *(const u32x4*)(xs + row * ROWB + gswz(row, 2 * ks + hh) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + lq;
        b[j] = *(const u32x4*)(ys + row * ROWB + gswz(row, 2 * ks + hh) * 16);
      }
    };
    u32x4 a0[2], b0[2], a1[2], b1[2];
    frags(0, a0, b0);
    frags(1, a1, b1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma<MT>(a0[i], b0[j], acc[i][j]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma<MT>(a1[i], b1[j], acc[i][j]);
    // stage s+1 must be in LDS for the next iteration; the newer one may stay in flight
    wait_stage(issued > s + 2);
    __syncthreads();
    cbuf = cbuf + 1 == NBUF ? 0 : cbuf + 1;
  }

  // ---- epilogues
  if (p.epi == kNtStoreT) {
    // out[m][n] (16-bit, ld_out) for n < n_valid, zero for n_valid <= n < N; sum of squares
    uint16_t* out = (uint16_t*)p.out;
    double ss = 0.0;
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
            const bool ok = n < p.n_valid;
            const float v = ok ? acc[i][j][e] : 0.0f;
            out[m * p.ld_out + n] = (uint16_t)(MT == ISPA_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
            ssf += v * v;
          }
        }
        ss += (double)ssf;
      }
    }
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
        if (m >= p.M || n >= p.N || (tri_tile && m > n)) continue;
        if (atomic)
          unsafeAtomicAdd(outf + m * p.ld_out + n, acc[i][j][e]);
        else
          outf[m * p.ld_out + n] += acc[i][j][e];
      }
    }
  }
}

// out[c][r] = in[r][c] for r < rows, 0 for rows <= r < rows_pad (16-bit elements).
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* in, int64_t ld_in, int64_t rows,
                                                          int64_t cols, uint16_t* out, int64_t ld_out,
                                                          int64_t rows_pad) {
  __shared__ uint16_t tile[64][66];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = ty + 16 * i;
    const int64_t r = r0 + rr, c = c0 + tx * 4;
    u32x2 v = {0u, 0u};
    if (r < rows && c < cols) v = *(const u32x2*)(in + r * ld_in + c);
    tile[rr][tx * 4 + 0] = (uint16_t)(v[0] & 0xffffu);
    tile[rr][tx * 4 + 1] = (uint16_t)(v[0] >> 16);
    tile[rr][tx * 4 + 2] = (uint16_t)(v[1] & 0xffffu);
    tile[rr][tx * 4 + 3] = (uint16_t)(v[1] >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = ty + 16 * i;
    const int64_t c = c0 + cc, r = r0 + tx * 4;
    if (c < cols && r < rows_pad) {
      const uint32_t lo = (uint32_t)tile[tx * 4 + 0][cc] | ((uint32_t)tile[tx * 4 + 1][cc] << 16);
      const uint32_t hi = (uint32_t)tile[tx * 4 + 2][cc] | ((uint32_t)tile[tx * 4 + 3][cc] << 16);
      *(u32x2*)(out + c * ld_out + r) = (u32x2){lo, hi};
    }
  }
}

// 16-bit conversion of a matrix (bf16 <-> f16) into a contiguous buffer
__global__ void convert16_kernel(const uint16_t* in, int64_t n, int in_dt, uint16_t* out, int out_dt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float f = in_dt == ISPA_BF16 ? bf16_bits_to_f32(in[i]) : f16_bits_to_f32(in[i]);
  out[i] = (uint16_t)(out_dt == ISPA_BF16 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f));
}

}  // namespace

ispa_status launch_nt_gemm(const NtGemmParams& p, int mfma_dt, hipStream_t stream, int* n_blocks_out) {
  const int64_t n0 = p.tri ? (int64_t)p.tiles_m * (p.tiles_m + 1) / 2 : (int64_t)p.tiles_m * p.tiles_n;
  const int64_t blocks = (n0 + (p.two_kinds ? (int64_t)p.tiles_m * p.tiles_n : 0)) * p.ksplit;
  if (n_blocks_out) *n_blocks_out = (int)blocks;
  if (p.K % BK || p.kchunk % BK || p.ksplit < 1 || (int64_t)p.ksplit * p.kchunk < p.K || p.ldx % 8 || p.ldy % 8) {
    set_error("nt_gemm: K, split or leading dimensions not aligned");
    return ISPA_ERR_INVALID_ARG;
  }
  if (blocks == 0) return ISPA_OK;
  if (mfma_dt == ISPA_BF16)
    hipLaunchKernelGGL(nt_gemm_kernel<ISPA_BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(nt_gemm_kernel<ISPA_F16>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return check_launch("nt_gemm_kernel");
}

ispa_status launch_transpose16(const void* in, int64_t ld_in, int64_t rows, int64_t cols, void* out,
                               int64_t ld_out, int64_t rows_pad, hipStream_t stream) {
  if (rows_pad == 0 || cols == 0) return ISPA_OK;
  const dim3 grid((unsigned)((rows_pad + 63) / 64), (unsigned)((cols + 63) / 64));
  hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, stream, (const uint16_t*)in, ld_in, rows, cols,
                     (uint16_t*)out, ld_out, rows_pad);
  return check_launch("transpose16_kernel");
}

ispa_status launch_convert16(const void* in, int64_t n, int in_dt, void* out, int out_dt, hipStream_t stream) {
  if (n == 0) return ISPA_OK;
  hipLaunchKernelGGL(convert16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)in, n, in_dt, (uint16_t*)out, out_dt);
  return check_launch("convert16_kernel");
}

}  // namespace ispa
