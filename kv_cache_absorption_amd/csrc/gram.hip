// K-contiguous MFMA GEMM ("NT": acc[m][n] = sum_k X[m][k] Y[n][k], both operands
// stored with k contiguous) for the regression statistics, and the transpose
// that produces such operands.
//
// The statistics contract over token rows (G = A^T A, C = A^T R) and over the
// input width (R = dA W).  Transposing A_loc and W once per call into the
// workspace, and writing R transposed, turns every product into this NT form so
// both operands can be moved straight from global memory into LDS:
//   * 256 x (2 WN) output tile per workgroup, 4 waves as 2 x 2, each 128 x WN
//     (WN = 128 or 64) = 4 x WN/32 tiles of v_mfma_f32_32x32x16_{f16,bf16}
//     whose accumulators live in the accumulation registers; a fragment read
//     from LDS feeds WN/32 (or 4) MFMAs, so LDS traffic stays at 0.5-0.75 KB
//     per MFMA and one wave per SIMD keeps the matrix core busy;
//   * K stages of 32: each operand tile is 256 (or 2 WN) rows x 64 bytes in LDS,
//     filled by buffer loads with the LDS flag (16 bytes per lane, no VGPR
//     staging), PD stages ahead in a ring of PD + 2 (3 and 5 for 256-wide
//     tiles, 4 and 6 for 128-wide: 96 KB in flight per CU, enough to cover the
//     L2 and HBM latency at the MFMA rate); one barrier per stage;
//   * 16-byte chunks of a row are XOR-swizzled with (row / 4) mod 4 so the
//     16-byte fragment reads of 16 consecutive rows use 16 distinct bank groups;
//   * the fragments of both 16-wide k slices of a stage are read before its MFMAs
//     run (the next stage's arrive meanwhile);
//   * the MFMA takes the Y fragment as its A operand and the X fragment as its B
//     operand, so each lane's accumulator holds four consecutive output columns
//     of one row: the epilogue reads, adds and writes 16-byte vectors;
//   * operand rows past the matrix reload the last valid row (results there
//     are discarded); the token dimension is zero-padded to a multiple of 32 so
//     no K masking is needed.
// The same kernel takes FP8 E4M3 operands for the W8A8 post-switch projection:
// 1-byte elements in the same 64-byte LDS rows (64 k per stage), one
// v_mfma_scale_f32_32x32x64_f8f6f4 per output block and stage over both
// fragments of the stage, and a store that multiplies by the row and column
// scales.
#include "gram.hpp"

#include <algorithm>

namespace ispa {

namespace {

constexpr int BM = kNtBM, BK = kNtBK;
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define ISPA_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
constexpr int ROWB = BK * 2;              // bytes per tile row (64)
constexpr int RPI = 1024 / ROWB;          // rows per 1 KB load instruction (16)

__device__ __forceinline__ int gswz(int row, int ch) { return ch ^ ((row >> 2) & 3); }

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_off, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_off), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

// fp8 product over a whole 64-byte K stage: each operand's two 16-byte
// fragments (k slices 0 and 1 of the stage) form the 32 bytes a lane supplies.
// Both operands take their bytes from the same row offsets, so the pairing of
// k indices is the same on both sides and the sum runs over the stage's 64 k.
__device__ __forceinline__ f32x16 mfma_e4m3(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  // format 0 (E4M3) for both operands; block scale exponent 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
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

// Tile (tm, tn) of the t-th workgroup of a grid (or of its upper triangle, tm <=
// tn): columns are taken in groups of eight and, inside a group, rows in order
// with the group's columns fastest.  Consecutive workgroups, which run at the
// same time on one XCD, then cover a compact block of tiles (four rows by eight
// columns) and share its operand rows in that XCD's L2.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, bool tri, int& tm, int& tn) {
  constexpr int GC = 8;
  for (int c0 = 0; c0 < tiles_n; c0 += GC) {
    const int nc = min(GC, tiles_n - c0);
    if (!tri) {
      if (t < tiles_m * nc) {
        tm = t / nc;
        tn = c0 + t % nc;
        return;
      }
      t -= tiles_m * nc;
      continue;
    }
    for (int r = 0; r < c0 + nc; ++r) {  // row r holds columns max(c0, r) .. c0 + nc - 1
      const int w = c0 + nc - max(c0, r);
      if (t < w) {
        tm = r;
        tn = max(c0, r) + t;
        return;
      }
      t -= w;
    }
  }
  tm = tn = 0;  // not reached for t below the tile count
}

template <int MT, int WN>
__global__ __launch_bounds__(256, 1) void nt_gemm_kernel(const NtGemmParams p) {
  constexpr bool F8 = MT == kMtE4M3;
  constexpr int ES = F8 ? 1 : 2;     // bytes per element
  constexpr int BKE = ROWB / ES;     // elements per K stage (32, or 64 for fp8)
  constexpr int BN = 2 * WN;
  constexpr int NJ = WN / 32;                 // 32-column blocks per wave
  constexpr int XB = BM * ROWB, YB = BN * ROWB;  // bytes per stage of each operand
  constexpr int XL = XB / 1024 / 4, YL = YB / 1024 / 4;  // 1 KB loads per wave per stage
  constexpr int LOADS = XL + YL;
  constexpr int PD = WN == 128 ? 3 : 4;  // stages loaded ahead
  constexpr int NBUF = PD + 2;           // ring slots
  static_assert(NBUF * (XB + YB) <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * (XB + YB)];
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
  grouped_tile((int)t, p.tiles_m, p.tiles_n, p.tri && !kind1, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);  // workgroup-uniform: keeps the buffer
  tn = __builtin_amdgcn_readfirstlane(tn);  // descriptors in scalar registers
  const char* yp = (const char*)(kind1 ? p.y2 : p.y);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = (int64_t)split * p.kchunk;
  const int64_t ke = min(p.K, kb + p.kchunk);
  const int ns = ke > kb ? (int)((ke - kb) / BKE) : 0;  // K is a multiple of BKE

  // ---- operand sources: rows of 2*ld bytes; rows past the end reload the last one
  const int64_t xrows = p.M, yrows = p.y_rows;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)p.x + m0 * p.ldx * ES), 0, (int)(min<int64_t>(BM, xrows - m0) * p.ldx * ES), 0x00020000);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(yp + n0 * p.ldy * ES), 0, (int)(min<int64_t>(BN, yrows - n0) * p.ldy * ES), 0x00020000);
  int xo[XL], yo[YL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int row = (wave * XL + i) * RPI + lane / (ROWB / 16);  // RPI rows per 1 KB instruction
    const int xr = (int)min<int64_t>(row, xrows - m0 - 1);
    xo[i] = xr * (int)(p.ldx * ES) + gswz(row, lane % (ROWB / 16)) * 16;
  }
#pragma unroll
  for (int i = 0; i < YL; ++i) {
    const int row = (wave * YL + i) * RPI + lane / (ROWB / 16);
    const int yr = (int)min<int64_t>(row, yrows - n0 - 1);
    yo[i] = yr * (int)(p.ldy * ES) + gswz(row, lane % (ROWB / 16)) * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds;
  auto issue = [&](int s, int buf) {
    const int soff = (int)((kb + (int64_t)s * BKE) * ES);
    const uint32_t xb = lds0 + buf * (XB + YB), yb = xb + XB;
#pragma unroll
    for (int i = 0; i < XL; ++i) lds_dma16(rx, xb + (wave * XL + i) * 1024, xo[i], soff);
#pragma unroll
    for (int i = 0; i < YL; ++i) lds_dma16(ry, yb + (wave * YL + i) * 1024, yo[i], soff);
  };
  // wait until at most `newer` stages of loads are outstanding (0 <= newer < PD)
  auto wait_stage = [&](int newer) {
    if constexpr (LOADS == 8) {
      if (newer <= 0)
        __builtin_amdgcn_s_waitcnt(0x0F70);
      else if (newer == 1)
        __builtin_amdgcn_s_waitcnt(0x0F78);
      else
        __builtin_amdgcn_s_waitcnt(0x4F70);  // 16: vmcnt bits 5:4 sit in simm16 bits 15:14
    } else {
      static_assert(LOADS == 6, "stage load count");
      if (newer <= 0)
        __builtin_amdgcn_s_waitcnt(0x0F70);
      else if (newer == 1)
        __builtin_amdgcn_s_waitcnt(0x0F76);
      else if (newer == 2)
        __builtin_amdgcn_s_waitcnt(0x0F7C);
      else
        __builtin_amdgcn_s_waitcnt(0x4F72);  // 18
    }
  };

  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x16){};

  // fragments of one 16-wide k slice of a stage: the wave's X rows and Y rows
  auto frags = [&](int buf, int ks, u32x4 (&a)[4], u32x4 (&b)[NJ]) {
    const char* xs = lds + buf * (XB + YB);
    const char* ys = xs + XB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + lq;
      a[i] = *(const u32x4*)(xs + row * ROWB + gswz(row, 2 * ks + hh) * 16);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = wn * WN + j * 32 + lq;
      b[j] = *(const u32x4*)(ys + row * ROWB + gswz(row, 2 * ks + hh) * 16);
    }
  };
  // acc[i][j] holds out^T for row block i and column block j (lane: row lq,
  // columns (e/4)*8 + hh*4 + e%4)
  auto mfmas = [&](const u32x4 (&a)[4], const u32x4 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma<MT>(b[j], a[i], acc[i][j]);
  };
  // fp8: one MFMA per output block over both slices of a stage
  auto mfmas8 = [&](const u32x4 (&a0)[4], const u32x4 (&b0)[NJ], const u32x4 (&a1)[4], const u32x4 (&b1)[NJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_e4m3(b0[j], b1[j], a0[i], a1[i], acc[i][j]);
  };

  int issued = 0, lbuf = 0;
  for (; issued < PD && issued < ns; ++issued) {
    issue(issued, lbuf);
    lbuf = lbuf + 1 == NBUF ? 0 : lbuf + 1;
  }
  // The MFMAs of one k slice run from registers while the next slice's
  // fragments are read between them.  Per stage s: slice 0's MFMAs with slice 1
  // read; the wait and barrier for stage s + 1; slice 1's MFMAs with stage
  // s + 1's slice 0 read.  A slot refilled in iteration s held stage
  // s + PD - NBUF = s - 2, last read in iteration s - 2 before its barrier.
  u32x4 fa0[4], fb0[NJ], fa1[4], fb1[NJ];
  if (ns > 0) {
    wait_stage(issued - 1);
    __syncthreads();
    frags(0, 0, fa0, fb0);
  }
  // The last stage is peeled off so that the loop body has no path around
  // its barrier: the slice-1 MFMAs after the barrier then see their fragments
  // as complete and do not wait for the next stage's reads.
  int cbuf = 0;
  for (int s = 0; s + 1 < ns; ++s) {
    if (issued < ns) {
      issue(issued, lbuf);
      lbuf = lbuf + 1 == NBUF ? 0 : lbuf + 1;
      ++issued;
    }
    frags(cbuf, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);  // keep each phase's reads ahead of the MFMAs they overlap
    if constexpr (F8)
      mfmas8(fa0, fb0, fa1, fb1);  // the whole stage, before the barrier: both slices are in registers
    else
      mfmas(fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    const int nbuf = cbuf + 1 == NBUF ? 0 : cbuf + 1;
    wait_stage(issued - (s + 2));  // stage s + 1 is in LDS
    __syncthreads();
    frags(nbuf, 0, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!F8) mfmas(fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    cbuf = nbuf;
  }
  if (ns > 0) {  // every stage has been issued by now
    frags(cbuf, 1, fa1, fb1);
    if constexpr (F8) {
      mfmas8(fa0, fb0, fa1, fb1);
    } else {
      mfmas(fa0, fb0);
      mfmas(fa1, fb1);
    }
  }

  // ---- epilogues: lane holds out[m][n .. n+3] in acc[i][j][4 g .. 4 g + 3] with
  // m = row block i + lq and n = column block j + 8 g + 4 hh
  if (p.epi == kNtStoreT) {
    // out[m][n] (16-bit, ld_out) for n < n_valid, zero for n_valid <= n < N; sum of squares
    uint16_t* out = (uint16_t*)p.out;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lq;
      float ssf = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn * WN + j * 32 + g * 8 + hh * 4;  // N is a multiple of 4
          if (m < p.M && n < p.N) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = n + e < p.n_valid ? acc[i][j][g * 4 + e] : 0.0f;
              ssf += v[e] * v[e];
            }
            const uint32_t lo = MT == ISPA_BF16 ? pack_bf16(v[0], v[1]) : pack_f16(v[0], v[1]);
            const uint32_t hi = MT == ISPA_BF16 ? pack_bf16(v[2], v[3]) : pack_f16(v[2], v[3]);
            *(u32x2*)(out + m * p.ld_out + n) = (u32x2){lo, hi};
          }
        }
      }
      ss += (double)ssf;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    double* red = (double*)lds;
    __syncthreads();  // every wave is done with the ring
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (tid == 0) p.sq_partials[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    return;
  }
  if (p.epi == kNtStoreScaled) {
    // dequantising store: acc * sx[m] * sy[n], in out_dt
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lq;
      if (m >= p.M) continue;
      const float sxm = p.sx[m];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn * WN + j * 32 + g * 8 + hh * 4;  // N is a multiple of 4
          if (n >= p.N) continue;
          const f32x4 sy = *(const f32x4*)(p.sy + n);
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][g * 4 + e] * sxm * sy[e];
          if (p.out_dt == ISPA_F32) {
            *(f32x4*)((float*)p.out + m * p.ld_out + n) = v;
          } else {
            const bool bf = p.out_dt == ISPA_BF16;
            auto pk = [&](float x, float y) { return bf ? pack_bf16(x, y) : pack_f16(x, y); };
            *(u32x2*)((uint16_t*)p.out + m * p.ld_out + n) = (u32x2){pk(v[0], v[1]), pk(v[2], v[3])};
          }
        }
    }
    return;
  }
  if (p.epi == kNtStore) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lq;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn * WN + j * 32 + g * 8 + hh * 4;  // N is a multiple of 4
          if (n >= p.N) continue;
          const f32x4 v = {acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
          if (p.out_dt == ISPA_F32) {
            *(f32x4*)((float*)p.out + m * p.ld_out + n) = v;
          } else {
            const bool bf = p.out_dt == ISPA_BF16;
            auto pk = [&](float x, float y) { return bf ? pack_bf16(x, y) : pack_f16(x, y); };
            *(u32x2*)((uint16_t*)p.out + m * p.ld_out + n) = (u32x2){pk(v[0], v[1]), pk(v[2], v[3])};
          }
        }
    }
    return;
  }
  float* outf = (float*)(kind1 ? p.out2 : p.out);
  const bool tri_tile = p.tri && !kind1;
  if (p.ksplit > 1) {
    // partial sums of this split, stored in the output's layout (no triangle mask:
    // the reduction applies it)
    float* part = p.part + ((int64_t)split * (p.two_kinds ? 2 : 1) + (kind1 ? 1 : 0)) * p.M * p.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lq;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn * WN + j * 32 + g * 8 + hh * 4;
          if (n < p.N)
            *(f32x4*)(part + m * p.ld_out + n) =
                (f32x4){acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + i * 32 + lq;
    if (m >= p.M) continue;
    float* row = outf + m * p.ld_out;
    // read all of this row block's vectors first so their latencies overlap
    f32x4 cur[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WN + j * 32 + g * 8 + hh * 4;  // N is a multiple of 4
        cur[j][g] = n < p.N ? *(const f32x4*)(row + n) : (f32x4){};
      }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WN + j * 32 + g * 8 + hh * 4;
        if (n >= p.N) continue;
        f32x4 v = cur[j][g];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += acc[i][j][g * 4 + e];
        if (!tri_tile || m <= n) {
          *(f32x4*)(row + n) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)  // the diagonal crosses this vector: upper part only
            if (m <= n + e) row[n + e] = v[e];
        }
      }
  }
}

// ---- symmetric rank-k update of X = [A_loc | dA] (the grouped statistics) ----
//
// X^T X over a chunk's token rows, upper block triangle only, 256 x 256 tiles
// of the 2 nbh x 2 nbh block grid (nbh = 256-column blocks per half): tile
// (I, J), I <= J, is G = A_loc^T A_loc for I, J < nbh, M = A_loc^T dA for
// I < nbh <= J and H = dA^T dA for nbh <= I.  The operands are read as the
// merge left them, row-major [n, D] 16-bit with the token index as k:
//   * a K stage is 32 token rows x 256 columns (512 contiguous bytes per row)
//     of each operand, moved from global memory straight into an LDS ring by
//     buffer loads with the LDS flag (16 bytes per lane), 3 stages ahead in
//     5 slots of 32 KB; the 16-byte chunks of row r are XOR-permuted by
//     4 (r mod 8) so the transposing fragment reads below spread over the banks;
//   * fragments come from ds_read_b64_tr_b16: a 16-lane group reads 4 token
//     rows x 16 columns and each lane receives one column's 4 tokens; two
//     such reads (tokens +0..3 and +8..11 of a 16-token slice, per wave half
//     +4) form the 8 k values of a v_mfma_f32_32x32x16 operand, in the same
//     k order on both sides of the product;
//   * kSyrkWaves waves: 4 as 2 x 2, each 128 x 128 (16 accumulators of 32 x 32),
//     or 8 as 2 x 4, each 128 x 64 (8 accumulators), two waves per SIMD; the
//     operands are swapped so a lane holds 4 consecutive output columns;
//   * a diagonal tile (I == J) loads one operand and reads both fragments
//     from it;
//   * the token range is split S ways (S fixed by D so that the launch fills
//     the chip); split s adds into its own copy of G, M and H in the per-layer
//     state, so no partial sums travel and no reduction runs per chunk; the
//     copies are added at the switch.  Token rows past n read as zero (buffer
//     range), columns past D repeat the last valid chunk (their outputs are
//     not stored).
constexpr int SY_BM = 256, SY_BK = 32;
constexpr int SY_ROWB = SY_BM * 2;         // bytes per LDS row of one operand
constexpr int SY_OPB = SY_BK * SY_ROWB;    // 16 KB per operand and stage
constexpr int SY_PD = 3, SY_NBUF = 5;      // stages in flight, ring slots
static_assert(SY_NBUF * 2 * SY_OPB <= 160 * 1024, "LDS budget");
constexpr int kSyrkWaves = 8;

template <int MT, bool DIAG, int NW>
__device__ __forceinline__ void syrk_tile(const SyrkParams& p, char* lds, int tm, int tn, int split) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int NJ = NW == 4 ? 4 : 2;         // 32-column blocks per wave
  constexpr int LPW = 16 / NW;                // 1 KB loads per wave, operand and stage
  constexpr int LOADS = DIAG ? LPW : 2 * LPW;  // per wave and stage
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hh = lane >> 5, lq = lane & 31, g16 = lane >> 4, s16 = lane & 15;
  const int wm = NW == 4 ? wave >> 1 : wave >> 2, wn = NW == 4 ? wave & 1 : wave & 3;
  const int nbh = p.nbh;
  // operand halves and column offsets of the two blocks
  const bool xb = tm >= nbh, yb = tn >= nbh;
  const int64_t cx = (int64_t)(xb ? tm - nbh : tm) * SY_BM, cy = (int64_t)(yb ? tn - nbh : tn) * SY_BM;
  const int64_t kb = (int64_t)split * p.kchunk;
  const int64_t ke = min(p.n, kb + p.kchunk);
  const int ns = ke > kb ? (int)((ke - kb + SY_BK - 1) / SY_BK) : 0;
  const int64_t ldb = p.lda * 2;  // row pitch in bytes
  // buffer descriptors over this split's rows of each block: rows past ke are
  // out of range (read as zero)
  auto rsrc = [&](bool half_b, int64_t col0) {
    const char* base = (const char*)(half_b ? p.b : p.a) + kb * ldb + col0 * 2;
    const int64_t rows = ke - kb;
    const int64_t bytes = rows > 0 ? (rows - 1) * ldb + (p.D - col0) * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rx = rsrc(xb, cx), ry = rsrc(yb, cy);
  // this lane's part of load instruction i (0..LPW-1) of its wave: LDS row
  // 2 q + hh (q = LPW wave + i), physical chunk lq holding logical chunk lq ^ 4 (row mod 8)
  int xo[LPW], yo[LPW];
  {
    const int lastx = (int)((p.D - cx) / 8) - 1, lasty = (int)((p.D - cy) / 8) - 1;  // last valid chunk
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = 2 * (wave * LPW + i) + hh;
      const int lch = lq ^ ((row & 7) << 2);
      xo[i] = row * (int)ldb + min(lch, lastx) * 16;
      yo[i] = row * (int)ldb + min(lch, lasty) * 16;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds;
  // the stage's row offset goes into the per-lane offset (not the scalar
  // one) so that the buffer range check sees it: rows past the split's end
  // then read as zero
  auto issue = [&](int s, int buf) {
    const int so = (int)((int64_t)s * SY_BK * ldb);
    const uint32_t xd = lds0 + buf * 2 * SY_OPB, yd = xd + SY_OPB;
#pragma unroll
    for (int i = 0; i < LPW; ++i) lds_dma16(rx, xd + (wave * LPW + i) * 1024, xo[i] + so, 0);
    if constexpr (!DIAG) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) lds_dma16(ry, yd + (wave * LPW + i) * 1024, yo[i] + so, 0);
    }
  };
  // wait until at most `newer` stages of loads are outstanding (0 <= newer < SY_PD)
  auto wait_stage = [&](int newer) {
    constexpr int v1 = LOADS, v2 = 2 * LOADS;
    if (newer <= 0)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (newer == 1)
      __builtin_amdgcn_s_waitcnt((v1 & 15) | ((v1 >> 4) << 14) | 0x0F70);
    else
      __builtin_amdgcn_s_waitcnt((v2 & 15) | ((v2 >> 4) << 14) | 0x0F70);
  };
  // per-lane fragment offsets inside a stage: LDS row 4 hh + (s16 >> 2) (+8 for the
  // second read, +16 per k slice), column block c0 + 32 b: chunk
  // (c0 / 8 + 4 b) ^ 4 (row mod 8), plus (g16 & 1) * 2 + (s16 & 3) / 2 and a
  // half-chunk (s16 & 1) * 8
  int fx[4], fy[NJ];
  {
    const int r = 4 * hh + (s16 >> 2);
    const int fl = r & 7;
    const int low = ((g16 & 1) * 2 + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) fx[b] = r * SY_ROWB + ((((wm * 4 + b) ^ fl) << 2) << 4) + low;
#pragma unroll
    for (int b = 0; b < NJ; ++b) fy[b] = r * SY_ROWB + ((((wn * NJ + b) ^ fl) << 2) << 4) + low;
  }
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  auto read8 = [&](const char* base, int off) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS_PTR(s16x4, base + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS_PTR(s16x4, base + off + 8 * SY_ROWB));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(u32x4, v);
  };
  auto frags = [&](int buf, int ks, u32x4 (&a)[4], u32x4 (&b)[NJ]) {
    const char* xs = lds + buf * 2 * SY_OPB + ks * 16 * SY_ROWB;
    const char* ys = DIAG ? xs : xs + SY_OPB;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = read8(xs, fx[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = read8(ys, fy[j]);
  };
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x16){};
  auto mfmas = [&](const u32x4 (&a)[4], const u32x4 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma<MT>(b[j], a[i], acc[i][j]);
  };

  int issued = 0, lbuf = 0;
  for (; issued < SY_PD && issued < ns; ++issued) {
    issue(issued, lbuf);
    lbuf = lbuf + 1 == SY_NBUF ? 0 : lbuf + 1;
  }
  u32x4 fa0[4], fb0[NJ], fa1[4], fb1[NJ];
  if (ns > 0) {
    wait_stage(issued - 1);
    __syncthreads();
    frags(0, 0, fa0, fb0);
  }
  // Per stage s: slice 1's fragments are read while slice 0's MFMAs run; the
  // wait and barrier for stage s + 1; then stage s + 1's slice 0 is read while
  // slice 1's MFMAs run.  A slot refilled in iteration s held stage s - 2,
  // last read before iteration s - 1's barrier.
  // One MFMA, then one fragment read of the other slice, 16 times: the reads
  // of a phase write registers that its MFMAs do not use, so no MFMA waits
  // for a read issued in its own phase (with all 16 reads first, the LDS
  // counter cannot tell the older fragments from the new ones, and the first
  // MFMA waited for two of the new reads).
  // (8 waves: 8 MFMAs and 12 reads per phase, two reads after each of the first four)
  auto interleave = [&]() {
    if constexpr (NW == 4) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  int cbuf = 0;
  for (int s = 0; s + 1 < ns; ++s) {
    if (issued < ns) {
      issue(issued, lbuf);
      lbuf = lbuf + 1 == SY_NBUF ? 0 : lbuf + 1;
      ++issued;
    }
    __builtin_amdgcn_sched_barrier(0);
    frags(cbuf, 1, fa1, fb1);
    mfmas(fa0, fb0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    const int nbuf = cbuf + 1 == SY_NBUF ? 0 : cbuf + 1;
    wait_stage(issued - (s + 2));  // stage s + 1 is in LDS
    __syncthreads();
    frags(nbuf, 0, fa0, fb0);
    mfmas(fa1, fb1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    cbuf = nbuf;
  }
  if (ns > 0) {
    frags(cbuf, 1, fa1, fb1);
    mfmas(fa0, fb0);
    mfmas(fa1, fb1);
  }

  // ---- epilogue: this split's copy of the output block += acc.  Lane holds
  // out[m][n .. n+3] in acc[i][j][4 g .. 4 g + 3], m = wm*128 + 32 i + lq and
  // n = wn*128 + 32 j + 8 g + 4 hh inside the tile.
  const int which = !xb && !yb ? 0 : (!xb ? 1 : 2);  // G, M or H
  float* out = p.state + (int64_t)split * p.split_stride + (int64_t)which * p.D * p.D;
  const int64_t m0 = cx + wm * 128, n0 = cy + wn * 32 * NJ;  // this wave's 128 x 32 NJ block
  if (m0 + 128 <= p.D && n0 + 32 * NJ <= p.D) {
    // The block lies inside D (every block when D is a multiple of 256): no
    // per-vector checks, the 16 loads of a 32-row block go out together, and
    // the next block's loads are issued before this one is added and stored.
    auto ld = [&](int i, f32x4(&c)[NJ][4]) __attribute__((always_inline)) {
      const float* row = out + (m0 + i * 32 + lq) * p.D + n0 + hh * 4;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) c[j][g] = *(const f32x4*)(row + j * 32 + g * 8);
    };
    auto st = [&](int i, const f32x4(&c)[NJ][4]) __attribute__((always_inline)) {
      float* row = out + (m0 + i * 32 + lq) * p.D + n0 + hh * 4;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v = c[j][g];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += acc[i][j][g * 4 + e];
          *(f32x4*)(row + j * 32 + g * 8) = v;
        }
    };
    f32x4 c0[NJ][4], c1[NJ][4];
    ld(0, c0);
    ld(1, c1);
    st(0, c0);
    ld(2, c0);
    st(1, c1);
    ld(3, c1);
    st(2, c0);
    st(3, c1);
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = cx + wm * 128 + i * 32 + lq;
    if (m >= p.D) continue;
    float* row = out + m * p.D;
    f32x4 cur[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + j * 32 + g * 8 + hh * 4;  // D is a multiple of 64
        cur[j][g] = n < p.D ? *(const f32x4*)(row + n) : (f32x4){};
      }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + j * 32 + g * 8 + hh * 4;
        if (n >= p.D) continue;
        f32x4 v = cur[j][g];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += acc[i][j][g * 4 + e];
        *(f32x4*)(row + n) = v;
      }
  }
}

template <int MT>
__global__ __launch_bounds__(kSyrkWaves * 64, 1) void syrk_kernel(const SyrkParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[SY_NBUF * 2 * SY_OPB];
  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int split = (int)(bid / (uint32_t)p.n_tiles);
  const int t = (int)(bid - (uint32_t)split * (uint32_t)p.n_tiles);
  int tm, tn;
  grouped_tile(t, 2 * p.nbh, 2 * p.nbh, true, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  if (tm == tn)
    syrk_tile<MT, true, kSyrkWaves>(p, lds, tm, tn, split);
  else
    syrk_tile<MT, false, kSyrkWaves>(p, lds, tm, tn, split);
}

// ---- the statistics at the switch, from the per-layer state ----
// One thread per 4 consecutive columns of one row: the S split copies added;
// G's upper triangle stored (entries below the diagonal untouched); M split
// into three bf16 planes whose sum is M to fp32 accuracy (each plane the
// rounding of what the previous ones left), stored one after another as
// [3][D][D] for the C = M W product; and this row's share of
// r2 = <H, W W^T> = sum_i H_ii P_ii + 2 sum_{i<j} H_ij P_ij (P = W W^T, the
// sum of its np K-split partial products, upper triangle) in fp64, one
// partial per workgroup.
__global__ __launch_bounds__(256) void gram_sum_kernel(const float* state, int64_t split_stride, int S, int32_t D,
                                                       float* G, const float* P, int np, uint16_t* planes,
                                                       double* partials) {
  const int64_t vpr = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t DD = (int64_t)D * D;
  double part = 0.0;
  if (gid < (int64_t)D * vpr) {
    const int64_t i = gid / vpr, j = (gid % vpr) * 4;
    const int64_t o = i * D + j;
    f32x4 g = {}, m = {}, h = {};
    for (int sp = 0; sp < S; ++sp) {
      const float* st = state + sp * split_stride;
      g += *(const f32x4*)(st + o);
      m += *(const f32x4*)(st + DD + o);
      h += *(const f32x4*)(st + 2 * DD + o);
    }
    if (j + 3 >= i) {
      if (j >= i) {
        *(f32x4*)(G + o) = g;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e >= i) G[o + e] = g[e];
      }
    }
    uint32_t w[3][2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      float r0 = m[e], r1 = m[e + 1];
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const uint32_t pk = pack_bf16(r0, r1);
        w[pl][e / 2] = pk;
        r0 -= bf16_bits_to_f32(pk & 0xffffu);
        r1 -= bf16_bits_to_f32(pk >> 16);
      }
    }
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) *(u32x2*)(planes + pl * DD + o) = (u32x2){w[pl][0], w[pl][1]};
    if (j + 3 >= i) {
      f32x4 pv = *(const f32x4*)(P + o);
      for (int sp = 1; sp < np; ++sp) pv += *(const f32x4*)(P + sp * DD + o);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e >= i) part += (j + e == i ? 1.0 : 2.0) * (double)h[e] * (double)pv[e];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  __shared__ double red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// C = c3[0] + c3[1] + c3[2] (the three planes' products), 4 per thread
__global__ __launch_bounds__(256) void sum3_kernel(const float* c3, int64_t n, float* C) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  *(f32x4*)(C + i) = (*(const f32x4*)(c3 + i) + *(const f32x4*)(c3 + n + i)) + *(const f32x4*)(c3 + 2 * n + i);
}

// *out = sum of n partials (one workgroup, fixed order: deterministic)
__global__ __launch_bounds__(256) void sum_set_kernel(const double* partials, int64_t n, double* out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += partials[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// out[c][r] = in[r][c] for r < rows, 0 for rows <= r < rows_pad (16-bit elements),
// converted from in_dt to out_dt (bf16 <-> f16, round to nearest even) when they differ
__device__ __forceinline__ uint16_t conv16(uint32_t v, int in_dt, int out_dt) {
  if (in_dt == out_dt) return (uint16_t)v;
  const float f = in_dt == ISPA_BF16 ? bf16_bits_to_f32((uint16_t)v) : f16_bits_to_f32((uint16_t)v);
  return (uint16_t)(out_dt == ISPA_BF16 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f));
}

// Up to two transposes in one launch: workgroups [0, j[0].nblk) take job 0,
// the rest job 1; inside a job the 64 x 64 blocks go row block fastest.
struct T16Job {
  const uint16_t* in;
  uint16_t* out;
  int64_t ld_in, rows, cols, ld_out, rows_pad;
  int32_t in_dt, out_dt;
  int32_t gx, nblk;  // 64-row blocks over rows_pad; all blocks of the job
};
struct T16Jobs {
  T16Job j[2];
};

__global__ __launch_bounds__(256) void transpose16_kernel(const T16Jobs js) {
  __shared__ uint16_t tile[64][66];
  const bool second = (int)blockIdx.x >= js.j[0].nblk;
  const T16Job t = second ? js.j[1] : js.j[0];
  const int b = second ? (int)blockIdx.x - js.j[0].nblk : (int)blockIdx.x;
  const uint16_t* in = t.in;
  uint16_t* out = t.out;
  const int64_t ld_in = t.ld_in, rows = t.rows, cols = t.cols, ld_out = t.ld_out, rows_pad = t.rows_pad;
  const int in_dt = t.in_dt, out_dt = t.out_dt;
  const int64_t r0 = (int64_t)(b % t.gx) * 64, c0 = (int64_t)(b / t.gx) * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = ty + 16 * i;
    const int64_t r = r0 + rr, c = c0 + tx * 4;
    u32x2 v = {0u, 0u};
    if (r < rows && c < cols) v = *(const u32x2*)(in + r * ld_in + c);
    tile[rr][tx * 4 + 0] = conv16(v[0] & 0xffffu, in_dt, out_dt);
    tile[rr][tx * 4 + 1] = conv16(v[0] >> 16, in_dt, out_dt);
    tile[rr][tx * 4 + 2] = conv16(v[1] & 0xffffu, in_dt, out_dt);
    tile[rr][tx * 4 + 3] = conv16(v[1] >> 16, in_dt, out_dt);
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

// Symmetric per-row FP8 E4M3 quantisation, one workgroup per row: the row's
// absolute maximum, then its codes four at a time (the second pass re-reads the
// row from cache).  Both divisions are the compiler's IEEE fp32 division
// (correctly rounded: no fast-math flags), so the codes are those of the same
// arithmetic done in any IEEE fp32 implementation.  v_cvt_pk_fp8_f32 rounds to
// nearest even and does not saturate (480 and above become NaN), hence the
// clamp to +-448; a magnitude that rounds to zero is stored as code 0.
template <typename InT>
__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(const InT* in, int in_dt, int64_t ld_in, int64_t cols,
                                                              uint8_t* codes, int64_t ld_codes, float* scales) {
  const int64_t r = blockIdx.x;
  const InT* row = in + r * ld_in;
  auto to_f32 = [&](uint32_t b) { return in_dt == ISPA_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b); };
  auto load4 = [&](int64_t c) {
    f32x4 v;
    if constexpr (sizeof(InT) == 4) {
      v = *(const f32x4*)(row + c);
    } else {
      const u32x2 w = *(const u32x2*)(row + c);
      v[0] = to_f32(w[0] & 0xffffu);
      v[1] = to_f32(w[0] >> 16);
      v[2] = to_f32(w[1] & 0xffffu);
      v[3] = to_f32(w[1] >> 16);
    }
    return v;
  };
  float amax = 0.0f;
  for (int64_t c = 4 * (int64_t)threadIdx.x; c < cols; c += 1024) {
    const f32x4 v = load4(c);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax / 448.0f;
  if (threadIdx.x == 0) scales[r] = scale;
  uint8_t* out = codes + r * ld_codes;
  for (int64_t c = 4 * (int64_t)threadIdx.x; c < cols; c += 1024) {
    uint32_t w = 0u;
    if (scale > 0.0f) {
      const f32x4 v = load4(c);
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(v[e] / scale, -448.0f), 448.0f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
      w = (uint32_t)pk;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (((w >> (8 * b)) & 0x7fu) == 0u) w &= ~(0xffu << (8 * b));
    }
    *(uint32_t*)(out + c) = w;
  }
}

// out[m][n .. n+3] += sum_s part[s][kind][m][n .. n+3]; the first kind keeps the
// upper triangle (m <= n) only when tri is set.  The last workgroup instead adds
// the n_sq per-workgroup sums of squares to *r2 (fixed order: deterministic).
__global__ __launch_bounds__(256) void split_reduce_kernel(float* out0, float* out1, const float* part, int64_t M,
                                                           int64_t N, int64_t ld, int ksplit, int tri, int two,
                                                           const double* sq, int64_t n_sq, double* r2) {
  if (blockIdx.x == gridDim.x - 1) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n_sq; i += 256) s += sq[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
      if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
      __syncthreads();
    }
    if (threadIdx.x == 0 && r2) *r2 += red[0];
    return;
  }
  const int64_t vecs_per_row = N / 4;
  const int64_t per_kind = M * vecs_per_row;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= per_kind * (two ? 2 : 1)) return;
  const int kind = gid >= per_kind ? 1 : 0;
  const int64_t v = gid - kind * per_kind;
  const int64_t m = v / vecs_per_row, n = (v % vecs_per_row) * 4;
  if (kind == 0 && tri && m > n + 3) return;  // entirely below the diagonal
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ksplit; ++s)
    acc += *(const f32x4*)(part + ((int64_t)s * (two ? 2 : 1) + kind) * M * ld + m * ld + n);
  float* row = (kind ? out1 : out0) + m * ld;
  if (kind == 0 && tri && m > n) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (m <= n + e) row[n + e] += acc[e];
    return;
  }
  *(f32x4*)(row + n) += acc;
}

}  // namespace

ispa_status launch_nt_gemm(const NtGemmParams& p, int mfma_dt, hipStream_t stream, int* n_blocks_out) {
  const int64_t n0 = p.tri ? (int64_t)p.tiles_m * (p.tiles_m + 1) / 2 : (int64_t)p.tiles_m * p.tiles_n;
  const int64_t blocks = (n0 + (p.two_kinds ? (int64_t)p.tiles_m * p.tiles_n : 0)) * p.ksplit;
  if (n_blocks_out) *n_blocks_out = (int)blocks;
  const bool f8 = mfma_dt == kMtE4M3;
  const int64_t bke = f8 ? 2 * BK : BK, lda = f8 ? 16 : 8;
  if (p.K % bke || p.kchunk % bke || p.ksplit < 1 || (int64_t)p.ksplit * p.kchunk < p.K || p.ldx % lda ||
      p.ldy % lda || (p.bn != 256 && p.bn != 128) || (p.tri && p.bn != BM) || p.N % 4 || p.ld_out % 4 ||
      (p.epi == kNtAccum && p.ksplit > 1 && !p.part) || (p.epi == kNtStoreScaled && (!p.sx || !p.sy)) ||
      (f8 && p.epi != kNtStore && p.epi != kNtStoreScaled)) {
    set_error("nt_gemm: K, split, tile or leading dimensions not aligned");
    return ISPA_ERR_INVALID_ARG;
  }
  if (blocks == 0) return ISPA_OK;
  const dim3 grid((unsigned)blocks), block(256);
  if (f8) {
    if (p.bn == 256)
      hipLaunchKernelGGL((nt_gemm_kernel<kMtE4M3, 128>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((nt_gemm_kernel<kMtE4M3, 64>), grid, block, 0, stream, p);
  } else if (mfma_dt == ISPA_BF16) {
    if (p.bn == 256)
      hipLaunchKernelGGL((nt_gemm_kernel<ISPA_BF16, 128>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((nt_gemm_kernel<ISPA_BF16, 64>), grid, block, 0, stream, p);
  } else {
    if (p.bn == 256)
      hipLaunchKernelGGL((nt_gemm_kernel<ISPA_F16, 128>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((nt_gemm_kernel<ISPA_F16, 64>), grid, block, 0, stream, p);
  }
  return check_launch("nt_gemm_kernel");
}

ispa_status launch_quant_rows_e4m3(const void* in, int in_dt, int64_t ld_in, int64_t rows, int64_t cols,
                                   uint8_t* codes, int64_t ld_codes, float* scales, hipStream_t stream) {
  if (rows <= 0) return ISPA_OK;
  if (cols < 0 || cols % 4 || ld_in % 4 || ld_codes % 4 || ld_in < cols || ld_codes < cols || rows > INT32_MAX) {
    set_error("quant_rows_e4m3: cols, ld_in and ld_codes must be multiples of 4 (ld >= cols)");
    return ISPA_ERR_INVALID_ARG;
  }
  if (in_dt == ISPA_F32)
    hipLaunchKernelGGL(quant_rows_e4m3_kernel<float>, dim3((unsigned)rows), dim3(256), 0, stream,
                       (const float*)in, in_dt, ld_in, cols, codes, ld_codes, scales);
  else
    hipLaunchKernelGGL(quant_rows_e4m3_kernel<uint16_t>, dim3((unsigned)rows), dim3(256), 0, stream,
                       (const uint16_t*)in, in_dt, ld_in, cols, codes, ld_codes, scales);
  return check_launch("quant_rows_e4m3_kernel");
}

ispa_status launch_nt_split_reduce(const NtGemmParams& p, const double* sq, int64_t n_sq, double* r2,
                                   hipStream_t stream) {
  const int64_t items = p.ksplit > 1 ? p.M * (p.N / 4) * (p.two_kinds ? 2 : 1) : 0;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((items + 255) / 256 + 1)), dim3(256), 0, stream,
                     (float*)p.out, (float*)p.out2, p.part, p.M, p.N, p.ld_out, p.ksplit, p.tri, p.two_kinds, sq,
                     n_sq, r2);
  return check_launch("split_reduce_kernel");
}

int gram_splits(int32_t D) {
  const int64_t nb = 2 * ((D + 255) / 256);
  const int64_t tiles = nb * (nb + 1) / 2;
  return (int)std::max<int64_t>(1, std::min<int64_t>(4, 256 / tiles));
}

ispa_status launch_syrk(const SyrkParams& p, int mfma_dt, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_tiles * p.ksplit;
  if (p.D % 64 || p.lda % 8 || p.kchunk % 32 || p.kchunk * p.lda * 2 >= ((int64_t)1 << 31) ||
      (int64_t)p.ksplit * p.kchunk < p.n || blocks > INT32_MAX) {
    set_error("syrk: width, leading dimension or token split out of range");
    return ISPA_ERR_INVALID_ARG;
  }
  if (blocks == 0 || p.n == 0) return ISPA_OK;
  if (mfma_dt == ISPA_BF16)
    hipLaunchKernelGGL(syrk_kernel<ISPA_BF16>, dim3((unsigned)blocks), dim3(kSyrkWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(syrk_kernel<ISPA_F16>, dim3((unsigned)blocks), dim3(kSyrkWaves * 64), 0, stream, p);
  return check_launch("syrk_kernel");
}

// K split of P = W W^T: upper-triangle tiles of 256, split so that the launch
// fills the chip (1 when the triangle alone does)
static int finalize_p_split(int32_t D) {
  const int tm = (D + kNtBM - 1) / kNtBM;
  const int tiles = tm * (tm + 1) / 2;
  int ks = std::max(1, std::min(6, 256 / tiles));
  while (ks > 1 && (D / kNtBK) % ks) --ks;  // K stages divide evenly
  return ks;
}

size_t gram_finalize_ws_bytes(int32_t D) {
  const size_t d = (size_t)D;
  const size_t blocks = (d * (d / 4) + 255) / 256;
  const size_t pbuf = std::max<size_t>((size_t)finalize_p_split(D) * d * d * 4, 3 * d * d * 4);
  return align256(3 * d * d * 2) + align256(d * d * 2) + align256(pbuf) + align256(blocks * 8);
}

ispa_status launch_gram_finalize(int32_t D, const float* state, int64_t split_stride, int S, const uint16_t* w,
                                 float* G, float* C, double* r2, void* ws, hipStream_t stream) {
  const size_t d = (size_t)D;
  char* wp = (char*)ws;
  uint16_t* planes = (uint16_t*)wp;  // M as three bf16 planes, [3][D][D]
  wp += align256(3 * d * d * 2);
  uint16_t* wt = (uint16_t*)wp;  // W^T
  wp += align256(d * d * 2);
  float* pbuf = (float*)wp;  // P = W W^T (or its K-split partial sums), then the planes' products [3][D][D]
  wp += align256(std::max<size_t>((size_t)finalize_p_split(D) * d * d * 4, 3 * d * d * 4));
  double* partials = (double*)wp;
  ispa_status st;
  {
    const Transpose16 t{w, wt, D, D, D, D, D, ISPA_BF16, ISPA_BF16};
    if ((st = launch_transpose16(&t, 1, stream))) return st;
  }
  // P = W W^T (rows of W are k-contiguous on both sides), upper-triangle tiles;
  // with a K split each split stores its partial product and gram_sum_kernel
  // adds them
  const int ks = finalize_p_split(D);
  NtGemmParams pp{};
  pp.M = D;
  pp.N = D;
  pp.K = D;
  pp.x = w;
  pp.ldx = D;
  pp.y = w;
  pp.ldy = D;
  pp.y_rows = D;
  pp.epi = ks > 1 ? kNtAccum : kNtStore;
  pp.out = pbuf;
  pp.out_dt = ISPA_F32;
  pp.ld_out = D;
  pp.bn = kNtBM;
  pp.tri = 1;
  pp.tiles_m = (D + kNtBM - 1) / kNtBM;
  pp.tiles_n = pp.tiles_m;
  pp.ksplit = ks;
  pp.kchunk = D / ks;
  pp.part = pbuf;
  if ((st = launch_nt_gemm(pp, ISPA_BF16, stream, nullptr))) return st;
  const int64_t blocks = ((int64_t)D * (D / 4) + 255) / 256;
  hipLaunchKernelGGL(gram_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, state, split_stride, S, D, G,
                     (const float*)pbuf, ks, planes, partials);
  if ((st = check_launch("gram_sum_kernel"))) return st;
  // the three planes' products with W in one launch: [3 D][D] x W (the planes
  // stacked as rows), then C = their sum
  NtGemmParams cp{};
  cp.M = 3 * (int64_t)D;
  cp.N = D;
  cp.K = D;
  cp.x = planes;
  cp.ldx = D;
  cp.y = wt;
  cp.ldy = D;
  cp.y_rows = D;
  cp.epi = kNtStore;
  cp.out = pbuf;
  cp.out_dt = ISPA_F32;
  cp.ld_out = D;
  cp.bn = 128;
  cp.tiles_m = (int)((3 * (int64_t)D + kNtBM - 1) / kNtBM);
  cp.tiles_n = (D + 127) / 128;
  cp.ksplit = 1;
  cp.kchunk = D;
  if ((st = launch_nt_gemm(cp, ISPA_BF16, stream, nullptr))) return st;
  const int64_t n = (int64_t)D * D;
  hipLaunchKernelGGL(sum3_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, (const float*)pbuf, n,
                     C);
  if ((st = check_launch("sum3_kernel"))) return st;
  hipLaunchKernelGGL(sum_set_kernel, dim3(1), dim3(256), 0, stream, (const double*)partials, blocks, r2);
  return check_launch("sum_set_kernel");
}

int64_t nt_stats_split(int32_t D, int64_t np) {
  // one workgroup per CU: split the token range when there are fewer tiles than CUs
  const int64_t tm = (D + kNtBM - 1) / kNtBM;
  const int64_t tiles = tm * (tm + 1) / 2 + tm * tm;
  const int64_t stages = np / kNtBK;
  const int64_t split = std::max<int64_t>(1, std::min<int64_t>(256 / tiles, stages / 8));
  const int64_t kchunk = (stages + split - 1) / split;
  return (stages + kchunk - 1) / kchunk;
}

static T16Job t16_job(const Transpose16& t) {
  T16Job j{};
  j.in = (const uint16_t*)t.in;
  j.out = (uint16_t*)t.out;
  j.ld_in = t.ld_in;
  j.rows = t.rows;
  j.cols = t.cols;
  j.ld_out = t.ld_out;
  j.rows_pad = t.rows_pad;
  j.in_dt = t.in_dt;
  j.out_dt = t.out_dt;
  j.gx = (int32_t)((t.rows_pad + 63) / 64);
  j.nblk = t.rows_pad > 0 && t.cols > 0 ? j.gx * (int32_t)((t.cols + 63) / 64) : 0;
  return j;
}

ispa_status launch_transpose16(const Transpose16* jobs, int n_jobs, hipStream_t stream) {
  if (n_jobs < 1 || n_jobs > 2) {
    set_error("launch_transpose16: 1 or 2 jobs");
    return ISPA_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n_jobs; ++i) {
    const int64_t blocks = (jobs[i].rows_pad + 63) / 64 * ((jobs[i].cols + 63) / 64);
    if (jobs[i].rows_pad < 0 || jobs[i].cols < 0 || blocks > (int64_t)INT32_MAX / 2) {
      set_error("launch_transpose16: matrix too large");
      return ISPA_ERR_INVALID_ARG;
    }
  }
  T16Jobs js{};
  js.j[0] = t16_job(jobs[0]);
  if (n_jobs == 2) js.j[1] = t16_job(jobs[1]);
  const int64_t total = (int64_t)js.j[0].nblk + js.j[1].nblk;
  if (total == 0) return ISPA_OK;
  hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)total), dim3(256), 0, stream, js);
  return check_launch("transpose16_kernel");
}

ispa_status launch_transpose16(const void* in, int64_t ld_in, int64_t rows, int64_t cols, void* out,
                               int64_t ld_out, int64_t rows_pad, int in_dt, int out_dt, hipStream_t stream) {
  const Transpose16 t{in, out, ld_in, rows, cols, ld_out, rows_pad, in_dt, out_dt};
  return launch_transpose16(&t, 1, stream);
}

}  // namespace ispa
