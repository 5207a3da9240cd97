// Quantised local attention on the fp8 matrix core (the post-switch L-Layer
// with W8A8 quantisation, EN review, Key Findings, the Figure 7 item; the
// pages give no scheme, the one here is ours).
//
// Operands are OCP FP8 E4M3 codes with power-of-two scales: K and V per cache
// chunk and head, Q per query row and head.  A scale is the least 2^e
// (e >= -126) with amax <= 448 * 2^e, so x / scale is exact and the code is its
// round-to-nearest-even E4M3 value (a magnitude that rounds to zero is stored
// as 0x00).  Power-of-two scales are what the matrix core's E8M0 block scales
// express, so v_mfma_scale_f32_32x32x64_f8f6f4 applies them itself.
//
// Cache format of one chunk of n keys (T = ceil(n / 64) tiles, keys past n are
// zero codes), per head h and tile t an 8 KB block at (h * T + t) * 8192:
//   K: 64 key rows of 128 bytes; 16-byte chunk c of row r is stored at chunk
//      position c ^ ((r >> 1) & 7), so the 16-byte fragment reads of 16
//      consecutive rows hit 16 different LDS bank groups.
//   V: transposed, 128 rows (one per d) of 64 key positions; position p holds
//      key ((p >> 4) & 1) * 32 + ((p >> 2) & 3) * 8 + (p >> 5) * 4 + (p & 3),
//      the order in which the score accumulator holds the keys, so a lane's
//      32 bytes of row d are the V^T operand that pairs with its own 32
//      probabilities; 16-byte chunk c of row d is stored at c ^ ((d >> 2) & 3).
// The attention kernel copies tiles into LDS unchanged (one 16-byte load per
// lane per tile and operand) and reads every fragment with ds_read_b128.
//
// Attention (d = 128): one workgroup = 8 waves x 32 queries of one head,
// key tiles of 64, the tile pipeline of the bf16 kernel:
//   * S^T = K Q^T: two v_mfma_scale_f32_32x32x64_f8f6f4 per 32-key block, the
//     K tile as A (block scale: the chunk's K exponent), the wave's queries as
//     B (block scale: each query's own exponent); each lane's accumulator is
//     16 scores of one query.
//   * P = exp2(S c - m) rounded to E4M3 (c = scale * log2 e) and packed in the
//     accumulator's key order, so it is the B operand of O^T = V^T P^T as it
//     stands; V^T takes the chunk's V exponent as its block scale.
//   * The row sum l is a fifth product, ones^T P^T on the matrix core: it sums
//     the rounded probabilities that O uses, in fp32, and costs no VALU.
//   * Lazy re-basing with head-room: m is raised only when a tile's row
//     maximum exceeds it by more than 8 (log2 units), and then to that
//     maximum minus 5, so P <= 2^8 < 448 always and the largest P after a
//     re-basing is 2^5: probabilities down to 2^-11 of the row maximum stay
//     in E4M3's normal range.
//   * K and V^T tiles are double-buffered in two rings of four 8 KB slots,
//     K of tile u loaded four iterations ahead, V two; one barrier per tile.
#include "attn8.hpp"

#include <algorithm>
#include <cmath>

namespace ispa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- scales -------------------------------------------------------------------
// The least e >= -126 with amax <= 448 * 2^e (0 for amax = 0), from the bits of
// amax: amax = f 2^k with f in [1/2, 1) and 448 = 0.875 * 2^9, so e = k - 9 when
// f <= 0.875 (mantissa field <= 0x600000) and k - 8 otherwise.
__device__ __forceinline__ int pow2_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int fld = (int)((b >> 23) & 0xffu);
  if (amax == 0.0f) return 0;
  if (fld == 0) return -126;  // subnormal amax: the floor
  const int k = fld - 126;
  const int e = (b & 0x7fffffu) <= 0x600000u ? k - 9 : k - 8;
  return e < -126 ? -126 : e;
}
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
// E8M0 block-scale byte of a power-of-two fp32 scale (a normal number)
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }

// four values (already divided by the scale, |y| <= 448) -> four E4M3 codes
// (v_cvt_pk_fp8_f32 rounds to nearest even; -0 is stored as +0)
__device__ __forceinline__ uint32_t e4m3x4(float y0, float y1, float y2, float y3) {
  int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, pk, true);
  uint32_t w = (uint32_t)pk;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (((w >> (8 * b)) & 0x7fu) == 0u) w &= ~(0xffu << (8 * b));
  return w;
}

template <typename InT>
__device__ __forceinline__ f32x4 load4(const InT* p, int dt) {
  if constexpr (sizeof(InT) == 4) {
    return *(const f32x4*)p;
  } else {
    const u32x2 w = *(const u32x2*)p;
    f32x4 v;
    if (dt == ISPA_BF16) {
      v[0] = bf16_bits_to_f32(w[0] & 0xffffu);
      v[1] = bf16_bits_to_f32(w[0] >> 16);
      v[2] = bf16_bits_to_f32(w[1] & 0xffffu);
      v[3] = bf16_bits_to_f32(w[1] >> 16);
    } else {
      v[0] = f16_bits_to_f32(w[0] & 0xffffu);
      v[1] = f16_bits_to_f32(w[0] >> 16);
      v[2] = f16_bits_to_f32(w[1] & 0xffffu);
      v[3] = f16_bits_to_f32(w[1] >> 16);
    }
    return v;
  }
}
__device__ __forceinline__ float amax4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}
// 16 consecutive values times inv (a power of two: exact) -> 16 codes
template <typename InT>
__device__ __forceinline__ u32x4 encode16(const InT* p, int dt, float inv) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 x = load4(p + 4 * i, dt);
    w[i] = e4m3x4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
  }
  return w;
}

__device__ __forceinline__ float block_max256(float x, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  __syncthreads();  // red may still be read by an earlier reduction
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---- K/V quantiser -------------------------------------------------------------
// Pass 1, one workgroup per (tile, head): the tile's maxima of |K| and |V|.
template <typename InT>
__global__ __launch_bounds__(256) void quant_kv_amax_kernel(const InT* k, int64_t ks, const InT* v, int64_t vs,
                                                            int64_t n, int32_t H, int32_t tiles, int dt, float* ws) {
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y;
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;  // row of the tile, 32-value quarter
  const int64_t key = (int64_t)t * kF8Keys + r;
  float ak = 0.0f, av = 0.0f;
  if (key < n) {
    const InT* kp = k + key * ks + (int64_t)h * kF8D + part * 32;
    const InT* vp = v + key * vs + (int64_t)h * kF8D + part * 32;
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      ak = fmaxf(ak, amax4(load4(kp + c, dt)));
      av = fmaxf(av, amax4(load4(vp + c, dt)));
    }
  }
  ak = block_max256(ak, red);
  av = block_max256(av, red);
  if (threadIdx.x == 0) {
    ws[((int64_t)0 * H + h) * tiles + t] = ak;
    ws[((int64_t)1 * H + h) * tiles + t] = av;
  }
}

// Pass 2, one workgroup per (tile, head): the head's scales from the tile
// maxima, then the tile's K codes (swizzled rows) and V^T codes (permuted key
// positions, swizzled rows) through LDS.
template <typename InT>
__global__ __launch_bounds__(256) void quant_kv_encode_kernel(const InT* k, int64_t ks, const InT* v, int64_t vs,
                                                              int64_t n, int32_t H, int32_t tiles, int dt,
                                                              const float* ws, uint8_t* kc, uint8_t* vc,
                                                              float* ksc, float* vsc) {
  __shared__ __attribute__((aligned(16))) uint8_t vt[kF8Keys][kF8D];  // V codes of the tile, key-major
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  float ak = 0.0f, av = 0.0f;
  for (int i = tid; i < tiles; i += 256) {
    ak = fmaxf(ak, ws[(int64_t)h * tiles + i]);
    av = fmaxf(av, ws[((int64_t)H + h) * tiles + i]);
  }
  ak = block_max256(ak, red);
  av = block_max256(av, red);
  const int ek = pow2_exp(ak), ev = pow2_exp(av);
  if (t == 0 && tid == 0) {
    ksc[h] = exp2i(ek);
    vsc[h] = exp2i(ev);
  }
  const float ik = exp2i(-ek), iv = exp2i(-ev);
  uint8_t* kt = kc + ((int64_t)h * tiles + t) * kF8TileBytes;
  uint8_t* vtt = vc + ((int64_t)h * tiles + t) * kF8TileBytes;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ci = tid + j * 256;  // row ci >> 3, 16-value chunk ci & 7
    const int r = ci >> 3, c = ci & 7;
    const int64_t key = (int64_t)t * kF8Keys + r;
    u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
    if (key < n) {
      kw = encode16(k + key * ks + (int64_t)h * kF8D + c * 16, dt, ik);
      vw = encode16(v + key * vs + (int64_t)h * kF8D + c * 16, dt, iv);
    }
    *(u32x4*)(kt + r * kF8D + ((c ^ ((r >> 1) & 7)) << 4)) = kw;
    *(u32x4*)(&vt[r][c * 16]) = vw;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int oi = tid + j * 256;  // V^T row d = oi >> 2, position chunk oi & 3
    const int d = oi >> 2, cp = oi & 3;
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int pos = cp * 16 + b;
      const int key = ((pos >> 4) & 1) * 32 + ((pos >> 2) & 3) * 8 + (pos >> 5) * 4 + (pos & 3);
      w[b >> 2] |= (uint32_t)vt[key][d] << (8 * (b & 3));
    }
    *(u32x4*)(vtt + d * kF8Keys + ((cp ^ ((d >> 2) & 3)) << 4)) = w;
  }
}

// ---- Q quantiser ---------------------------------------------------------------
// 32 lanes per (row, head): four values each, the row's maximum by shuffles.
template <typename InT>
__global__ __launch_bounds__(256) void quant_q_kernel(const InT* q, int64_t qs, int64_t n_q, int32_t H, int dt,
                                                      uint8_t* qc, float* qsc) {
  const int64_t pairs = n_q * H;
  int64_t pr = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const bool live = pr < pairs;
  if (!live) pr = pairs - 1;  // the group runs its shuffles on a valid row and stores nothing
  const int l = threadIdx.x & 31;
  const int64_t row = pr / H;
  const int h = (int)(pr - row * H);
  const f32x4 x = load4(q + row * qs + (int64_t)h * kF8D + l * 4, dt);
  float a = amax4(x);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  const int e = pow2_exp(a);
  const float inv = exp2i(-e);
  const uint32_t w = e4m3x4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
  if (live) {
    *(uint32_t*)(qc + pr * kF8D + l * 4) = w;
    if (l == 0) qsc[pr] = exp2i(e);
  }
}

// ---- attention -------------------------------------------------------------------
namespace f8 {
constexpr int DH = kF8D;
constexpr int WAVES = 8;
constexpr int BQ = WAVES * 32;
constexpr int BK = kF8Keys;
constexpr int TILEB = kF8TileBytes;
constexpr int NSLOT = 4;
constexpr int VBASE = NSLOT * TILEB;
constexpr float kLazy = 8.0f;  // re-base when a tile's maximum exceeds m by more than this (log2 units)
constexpr float kHead = 5.0f;  // ... and then to that maximum minus this
static_assert(TILEB == WAVES * 64 * 16, "one 16-byte load per lane per tile");
// s_waitcnt immediate: at most n vector memory operations outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
}  // namespace f8

struct Attn8Params {
  const uint8_t* q;
  const float* qs;
  int64_t n_q;
  int32_t H;
  int32_t n_qtiles;
  float c;  // scale * log2(e)
  int32_t n_segs;
  int32_t n_tiles;
  int32_t tiles[kF8MaxSegs];  // tiles of each segment
  int32_t nlast[kF8MaxSegs];  // keys in each segment's last tile
  const uint8_t* k[kF8MaxSegs];
  const uint8_t* v[kF8MaxSegs];
  const float* ks[kF8MaxSegs];
  const float* vs[kF8MaxSegs];
  void* o;
  int32_t o_dt;
  float* lse;
};

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_off, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_off), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ i32x8 cat8(u32x4 a, u32x4 b) {
  return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__global__ __launch_bounds__(f8::WAVES * 64, 1) void attn_fp8_d128_kernel(const Attn8Params p) {
  using namespace f8;
  __shared__ __attribute__((aligned(1024))) char lds[2 * NSLOT * TILEB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int lq = lane & 31;

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qtile = logical % p.n_qtiles;
  const int head = logical / p.n_qtiles;
  const float c = p.c;

  // this lane's query (B operand of S^T = K Q^T): bytes [mi*64 + hh*32, +32)
  const int64_t qrow = (int64_t)qtile * BQ + wave * 32 + lq;
  i32x8 qf[2];
  int eq = 127;
  {
    u32x4 a[4] = {};
    if (qrow < p.n_q) {
      const uint8_t* qp = p.q + (qrow * p.H + head) * DH + hh * 32;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const u32x4*)(qp + (i >> 1) * 64 + (i & 1) * 16);
      eq = e8m0_of(p.qs[qrow * p.H + head]);
    }
    qf[0] = cat8(a[0], a[1]);
    qf[1] = cat8(a[2], a[3]);
  }
  // the segments' block-scale bytes for this head, in LDS (read on segment changes)
  __shared__ uint8_t e8tab[2][kF8MaxSegs];
  if (tid < p.n_segs) {
    e8tab[0][tid] = (uint8_t)e8m0_of(p.ks[tid][head]);
    e8tab[1][tid] = (uint8_t)e8m0_of(p.vs[tid][head]);
  }
  __syncthreads();

  // Cursors over the tiles in order (every segment has at least one tile: the
  // host drops empty ones).  A load cursor holds its tile's address; past the
  // last tile it is not live and its loads get an empty descriptor.  The info
  // cursor holds its tile's segment data: keys in the segment's last tile and
  // the two scale bytes.
  struct LoadCur {
    int s, left;
    bool live;
    const char* addr;
  };
  struct InfoCur {
    int s, left, nlast, ek, ev;
    bool live;
  };
  auto load_seek = [&](LoadCur& cu, int s, bool is_v) __attribute__((always_inline)) {
    cu.s = s;
    cu.live = s < p.n_segs;
    if (cu.live) {
      cu.left = p.tiles[s];
      cu.addr = (const char*)(is_v ? p.v[s] : p.k[s]) + (int64_t)head * p.tiles[s] * TILEB;
    } else {
      cu.left = 1 << 30;
    }
  };
  auto load_step = [&](LoadCur& cu, bool is_v) __attribute__((always_inline)) {
    cu.addr += TILEB;
    if (--cu.left == 0) {
      asm volatile("" ::: "memory");  // a segment change: a branch
      load_seek(cu, cu.s + 1, is_v);
    }
  };
  auto info_seek = [&](InfoCur& cu, int s) __attribute__((always_inline)) {
    cu.s = s;
    cu.live = s < p.n_segs;
    if (cu.live) {
      cu.left = p.tiles[s];
      cu.nlast = p.nlast[s];
      cu.ek = __builtin_amdgcn_readfirstlane((int)e8tab[0][s]);
      cu.ev = __builtin_amdgcn_readfirstlane((int)e8tab[1][s]);
    } else {
      cu.left = 1 << 30;
      cu.nlast = 0;
      cu.ek = cu.ev = 127;
    }
  };
  auto info_step = [&](InfoCur& cu) __attribute__((always_inline)) {
    if (--cu.left == 0) {
      asm volatile("" ::: "memory");
      info_seek(cu, cu.s + 1);
    }
  };
  auto info_nv = [&](const InfoCur& cu) __attribute__((always_inline)) {
    return !cu.live ? 0 : (cu.left == 1 ? cu.nlast : BK);
  };

  // per-lane LDS byte offsets.  K: row kb*32 + lq, chunk mi*4 + hh*2 + j at
  // position chunk ^ ((lq >> 1) & 7).  V^T: row dt*32 + lq, chunk hh*2 + j at
  // chunk ^ ((lq >> 2) & 3).
  uint32_t koff[2][2], voff[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int j = 0; j < 2; ++j) koff[mi][j] = lq * DH + (((mi * 4 + hh * 2 + j) ^ ((lq >> 1) & 7)) << 4);
#pragma unroll
  for (int j = 0; j < 2; ++j) voff[j] = VBASE + lq * BK + (((hh * 2 + j) ^ ((lq >> 2) & 3)) << 4);
  auto k_frag = [&](int ks, int kb, int mi) __attribute__((always_inline)) {
    const u32x4 a = *(const u32x4*)(lds + ks + kb * 32 * DH + koff[mi][0]);
    const u32x4 b = *(const u32x4*)(lds + ks + kb * 32 * DH + koff[mi][1]);
    return cat8(a, b);
  };
  auto v_frag = [&](int vs, int dt) __attribute__((always_inline)) {
    const u32x4 a = *(const u32x4*)(lds + vs + dt * 32 * BK + voff[0]);
    const u32x4 b = *(const u32x4*)(lds + vs + dt * 32 * BK + voff[1]);
    return cat8(a, b);
  };

  const uint32_t lds0 = lds_addr(lds);
  const int gvoff = wave * 1024 + lane * 16;  // this lane's 16 bytes of a tile
  auto issue = [&](const LoadCur& cu, uint32_t dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)cu.addr, 0, cu.live ? TILEB : 0, 0x00020000);
    lds_dma16(r, dst + wave * 1024, gvoff);
  };

  f32x16 O[4], L = {}, S[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) O[i] = (f32x16){};
  float m = -INFINITY;
  i32x8 P[2];
  P[1] = (i32x8){};  // P_{-1}
  i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
  asm volatile("" : "+v"(ones));  // held in registers, not rebuilt for every product

  const int n_tiles = p.n_tiles;
  if (n_tiles > 0) {
    // a zeroed V slot 3 for iteration 0 (P_{-1} = 0; zero codes are no NaN)
    *(u32x4*)(lds + VBASE + 3 * TILEB + tid * 16) = (u32x4){0u, 0u, 0u, 0u};
    LoadCur kc, vc;  // in iteration t: K loads of tile t + 4, V loads of tile t + 2
    InfoCur ic;      // in iteration t: tile t + 1
    kc.addr = vc.addr = nullptr;
    load_seek(kc, 0, false);
    load_seek(vc, 0, true);
    info_seek(ic, 0);
    // prologue: K_0 .. K_3, V_0, V_1 in the order iterations -4 .. -1 issue them
    for (int i = -4; i < 0; ++i) {
      issue(kc, lds0 + ((i + 4) & 3) * TILEB);
      load_step(kc, false);
      if (i >= -2) {
        issue(vc, lds0 + VBASE + ((i + 2) & 3) * TILEB);
        load_step(vc, true);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));  // K_0 and K_1 are in LDS
    __syncthreads();
    int nv_cur = info_nv(ic), ev_cur = ic.ev, ev_prev = 127;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = mfma8(k_frag(0, kb, 0), qf[0], (f32x16){}, ic.ek, eq);
      S[kb] = mfma8(k_frag(0, kb, 1), qf[1], S[kb], ic.ek, eq);
    }
    info_step(ic);
    auto blk_max = [&](int kb) __attribute__((always_inline)) {
      float mx = S[kb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[kb][i]);
      return mx;
    };
    float mx0 = blk_max(0);
    __syncthreads();  // every wave has read K_0 before iteration 0 loads K_4 into its slot

    // P_t dword w (w = kb * 4 + j) holds the codes of S_t[kb][4j .. 4j + 3]
    auto exp4 = [&](int cb, int w) __attribute__((always_inline)) {
      const int kb = w >> 2, j = w & 3;
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(S[kb][4 * j + i], c, -m));
      // both halves of the word are written, so the conversion merges into the
      // slot's old contents (P_{t-2}, consumed) instead of a zeroed register
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], P[cb][w], false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], pk, true);
      P[cb][w] = pk;
    };

    // Iteration t: K ring slot u = t mod 4 receives K_{t+4}; P_t goes to P[cb]
    auto run_iter = [&](const int u, const int cb) __attribute__((always_inline)) {
      const int nv_n = info_nv(ic), ek_n = ic.ek, ev_n = ic.ev;  // tile t + 1
      if (nv_cur < BK) {  // keys past the end of the segment (all of them past the last tile) score -inf
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int lim = nv_cur - kb * 32 - hh * 4;  // element i is key kb*32 + (i/4)*8 + hh*4 + i%4
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kb][i] = ((i >> 2) * 8 + (i & 3) < lim) ? S[kb][i] : -INFINITY;
        }
        mx0 = blk_max(0);
      }
      // lazy re-basing from the tile's row maximum (lanes l and l ^ 32 hold the two key halves of a query)
      bool resc = false;
      float alpha = 1.0f;
      {
        const float ml = fmaxf(mx0, blk_max(1));
        const float mx = pair_max_halves(ml) * c;
        const bool up = mx - m > kLazy;
        if (__any(up)) {
          asm volatile("" ::: "memory");
          const float mn = up ? mx - kHead : m;
          alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 when m = -inf
          m = mn;
          L *= alpha;
          resc = true;
        }
      }
      const int ks = ((u + 1) & 3) * TILEB, vs = ((u + 3) & 3) * TILEB;
      // half 1: O^T += V_{t-1}^T P_{t-1}^T on the matrix core, P_t on the VALU
      {
        i32x8 vf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[i] = v_frag(vs, i);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          exp4(cb, 2 * i);
          exp4(cb, 2 * i + 1);
          O[i] = mfma8(vf[i], P[cb ^ 1], O[i], ev_prev, 127);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // P_t is formed here, not sunk past the re-basing branch into its users
        asm volatile("" ::"v"(P[cb][0]), "v"(P[cb][1]), "v"(P[cb][2]), "v"(P[cb][3]), "v"(P[cb][4]),
                     "v"(P[cb][5]), "v"(P[cb][6]), "v"(P[cb][7]));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (resc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] *= alpha;
      }
      // half 2: S_{t+1} = K_{t+1} Q^T and l += ones^T P_t^T on the matrix core; the
      // iteration's loads; the block-0 maxima of S_{t+1}
      {
        i32x8 kf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = k_frag(ks, i >> 1, i & 1);
        L = mfma8(ones, P[cb], L, 127, 127);
        issue(kc, lds0 + u * TILEB);
        issue(vc, lds0 + VBASE + ((u + 2) & 3) * TILEB);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kb = i >> 1, mi = i & 1;
          S[kb] = mfma8(kf[i], qf[mi], mi == 0 ? (f32x16){} : S[kb], ek_n, eq);
        }
        mx0 = blk_max(0);
        // the products are issued here, before the barrier, not sunk into the next iteration
        asm volatile("" ::"v"(S[0]), "v"(S[1]), "v"(L), "v"(mx0));
        __builtin_amdgcn_sched_barrier(0);
        load_step(kc, false);
        load_step(vc, true);
      }
      ev_prev = ev_cur;
      ev_cur = ev_n;
      nv_cur = nv_n;
      info_step(ic);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
      __syncthreads();
    };
    for (int t = 0;;) {
      run_iter(0, 0);
      if (++t > n_tiles) break;
      run_iter(1, 1);
      if (++t > n_tiles) break;
      run_iter(2, 0);
      if (++t > n_tiles) break;
      run_iter(3, 1);
      if (++t > n_tiles) break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no LDS write in flight at the end
  }

  // epilogue: o = O / l (l is in every element of L), lse = (m + log2 l) ln 2
  if (qrow >= p.n_q) return;
  const float l = L[0];
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const int64_t base = (qrow * p.H + head) * (int64_t)DH + hh * 4;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 v = {O[dt][g4 * 4] * inv, O[dt][g4 * 4 + 1] * inv, O[dt][g4 * 4 + 2] * inv,
                       O[dt][g4 * 4 + 3] * inv};
      const int64_t at = base + dt * 32 + g4 * 8;
      if (p.o_dt == ISPA_F32) {
        *(f32x4*)((float*)p.o + at) = v;
      } else if (p.o_dt == ISPA_BF16) {
        *(u32x2*)((uint16_t*)p.o + at) = (u32x2){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      } else {
        *(u32x2*)((uint16_t*)p.o + at) = (u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])};
      }
    }
  if (p.lse && hh == 0) p.lse[qrow * p.H + head] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

// ---- host launchers -----------------------------------------------------------------
size_t quant_kv_ws_bytes(int64_t n, int32_t H) {
  if (n <= 0 || H <= 0) return 0;
  return align256((size_t)2 * H * f8_tiles(n) * sizeof(float));
}

ispa_status launch_quant_kv_fp8(int dt, int64_t n, int32_t H, const void* k, int64_t k_stride, const void* v,
                                int64_t v_stride, uint8_t* k_codes, uint8_t* v_codes, float* k_scales,
                                float* v_scales, void* ws, hipStream_t stream) {
  if (n <= 0) return ISPA_OK;
  const int64_t tiles = f8_tiles(n);
  if (tiles > 65535 || H > 65535) {
    set_error("quantize_kv_fp8: more than 65535 tiles or heads");
    return ISPA_ERR_INVALID_ARG;
  }
  const dim3 grid((unsigned)tiles, (unsigned)H), block(256);
  float* w = (float*)ws;
  if (dt == ISPA_F32) {
    hipLaunchKernelGGL(quant_kv_amax_kernel<float>, grid, block, 0, stream, (const float*)k, k_stride,
                       (const float*)v, v_stride, n, H, (int32_t)tiles, dt, w);
    hipLaunchKernelGGL(quant_kv_encode_kernel<float>, grid, block, 0, stream, (const float*)k, k_stride,
                       (const float*)v, v_stride, n, H, (int32_t)tiles, dt, (const float*)w, k_codes, v_codes,
                       k_scales, v_scales);
  } else {
    hipLaunchKernelGGL(quant_kv_amax_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t*)k, k_stride,
                       (const uint16_t*)v, v_stride, n, H, (int32_t)tiles, dt, w);
    hipLaunchKernelGGL(quant_kv_encode_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t*)k, k_stride,
                       (const uint16_t*)v, v_stride, n, H, (int32_t)tiles, dt, (const float*)w, k_codes, v_codes,
                       k_scales, v_scales);
  }
  return check_launch("quant_kv_fp8 kernels");
}

ispa_status launch_quant_q_fp8(int dt, int64_t n_q, int32_t H, const void* q, int64_t q_stride, uint8_t* q_codes,
                               float* q_scales, hipStream_t stream) {
  const int64_t pairs = n_q * H;
  if (pairs <= 0) return ISPA_OK;
  const int64_t blocks = (pairs + 7) / 8;
  if (blocks > 0x7fffffff) {
    set_error("quantize_q_fp8: too many rows");
    return ISPA_ERR_INVALID_ARG;
  }
  if (dt == ISPA_F32)
    hipLaunchKernelGGL(quant_q_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, (const float*)q,
                       q_stride, n_q, H, dt, q_codes, q_scales);
  else
    hipLaunchKernelGGL(quant_q_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)q, q_stride, n_q, H, dt, q_codes, q_scales);
  return check_launch("quant_q_kernel");
}

ispa_status launch_attn_fp8(int64_t n_q, int32_t H, float scale, const uint8_t* q_codes, const float* q_scales,
                            const Attn8Seg* segs, int n_segs, void* o, int o_dt, float* lse, hipStream_t stream) {
  if (n_q <= 0) return ISPA_OK;
  Attn8Params p{};
  p.q = q_codes;
  p.qs = q_scales;
  p.n_q = n_q;
  p.H = H;
  p.n_qtiles = (int32_t)((n_q + f8::BQ - 1) / f8::BQ);
  p.c = scale * kLog2e;
  int64_t total = 0;
  int ns = 0;
  for (int s = 0; s < n_segs; ++s) {  // empty segments are dropped
    const int64_t t = f8_tiles(segs[s].n);
    if (t == 0) continue;
    p.tiles[ns] = (int32_t)t;
    p.nlast[ns] = (int32_t)(segs[s].n - (t - 1) * kF8Keys);
    p.k[ns] = segs[s].k;
    p.v[ns] = segs[s].v;
    p.ks[ns] = segs[s].ks;
    p.vs[ns] = segs[s].vs;
    ++ns;
    total += t;
  }
  p.n_segs = ns;
  if (total >= (1 << 30) || (int64_t)p.n_qtiles * H > 0x7fffffff) {
    set_error("attn_fp8: too many key tiles or workgroups");
    return ISPA_ERR_INVALID_ARG;
  }
  p.n_tiles = (int32_t)total;
  p.o = o;
  p.o_dt = o_dt;
  p.lse = lse;
  hipLaunchKernelGGL(attn_fp8_d128_kernel, dim3((unsigned)(p.n_qtiles * H)), dim3(f8::WAVES * 64), 0, stream, p);
  return check_launch("attn_fp8_d128_kernel");
}

}  // namespace ispa
