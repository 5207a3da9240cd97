// Attention over key groups, returning normalised output and log-sum-exp.
//
// Per query row and head the kernels compute, over the keys of one job,
//   lse = ln sum_j exp(s_j),  o = sum_j exp(s_j - lse) v_j,  s_j = scale <q, k_j>
// with a running (online) maximum so the score matrix is never stored.  This
// is the per-group state the dual-stream warmup relies on (EN review, Key
// Design 1: each group returns its weighted values and its LSE).
//
// bf16 path (d = 64 or 128), one workgroup = 4 waves x 32 queries of one head:
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the key tile is the A operand
//     (read row-wise from LDS), the wave's 32 queries are the B operand (kept
//     in registers).  In the 32x32 accumulator each lane then holds 16 scores
//     of ONE query, so the row max and row sum are in-register reductions plus
//     one exchange between the two wave halves (v_permlane32_swap).
//   * O^T = V^T P^T: V is staged transposed in LDS ([d][key]) so each lane's A
//     fragment is one 16-byte LDS read; the P fragment is the lane's own scores
//     converted to bf16, with the key order inside LDS permuted to match the
//     accumulator layout (swap of key bits 2 and 3).
//   * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global
//     loads are in flight while the current one is computed; one barrier per
//     tile.
//   * The running maximum is only raised when some lane's tile maximum exceeds
//     it by more than 8 (log2 units), so the O rescale is rare; exp2 arguments
//     stay <= 8 and the result is unchanged in exact arithmetic.
//   * Workgroups are mapped XCD-contiguously so the q-tiles of one (job, head)
//     share an L2.
// f32 path: one thread per (query, head), plain fp32 loop (parity mode).
#include "attn.hpp"

#include <algorithm>
#include <cmath>

namespace ispa {

namespace {

constexpr int kBQ = 128;  // queries per workgroup
constexpr int kBK = 64;   // keys per tile

// Cursor over the tiles of one job: segments in order, rows clipped to the
// job's key range, 64 rows per tile (the last tile of a segment may be short).
struct TileCursor {
  int seg;
  int64_t row;  // first row of the tile inside the segment
  int64_t end;  // one past the last row of this segment inside the job
};

__device__ __forceinline__ bool cursor_seek(const AttnParams& p, int g, int seg, int64_t kbeg,
                                            int64_t kend, TileCursor& cur) {
  // find the first segment >= seg with a non-empty intersection
  int64_t st = 0;
  for (int s = 0; s < p.n_segs[g]; ++s) {
    const int64_t n = p.segs[g][s].n;
    const int64_t a = kbeg > st ? kbeg : st;
    const int64_t b = kend < st + n ? kend : st + n;
    if (s >= seg && a < b) {
      cur.seg = s;
      cur.row = a - st;
      cur.end = b - st;
      return true;
    }
    st += n;
  }
  return false;
}

__device__ __forceinline__ bool cursor_next(const AttnParams& p, int g, int64_t kbeg, int64_t kend,
                                            TileCursor& cur) {
  cur.row += kBK;
  if (cur.row < cur.end) return true;
  return cursor_seek(p, g, cur.seg + 1, kbeg, kend, cur);
}

template <int BK>
__device__ __forceinline__ bool cursor_seek_bk(const AttnParams& p, int g, int seg, int64_t kbeg, int64_t kend,
                                               TileCursor& cur) {
  return cursor_seek(p, g, seg, kbeg, kend, cur);
}
template <int BK>
__device__ __forceinline__ bool cursor_next_bk(const AttnParams& p, int g, int64_t kbeg, int64_t kend,
                                               TileCursor& cur) {
  cur.row += BK;
  if (cur.row < cur.end) return true;
  return cursor_seek(p, g, cur.seg + 1, kbeg, kend, cur);
}

template <int DH>
struct BfTile {
  static constexpr int CH = DH / 8;          // 16-byte chunks per key row
  static constexpr int RPP = 256 / CH;       // rows per load pass
  static constexpr int KPASS = kBK / RPP;    // passes for the K tile
  static constexpr int NDP = DH / 2;         // d pairs
  static constexpr int VITEMS = NDP * 8 / 256;  // (d pair, 8-key group) items per thread
  static constexpr int KS = DH + 8;          // LDS row stride of K (elements)
  static constexpr int VS = kBK + 8;         // LDS row stride of V^T (elements)
};

template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const AttnParams p) {
  using T = BfTile<DH>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBK * T::KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DH * T::VS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;   // wave half
  const int lq = lane & 31;   // query column inside the wave

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qtile = logical % p.n_qtiles;
  const uint32_t rest = logical / p.n_qtiles;
  const int head = rest % p.H;
  const int jidx = rest / p.H;
  const AttnJob job = p.jobs[jidx];
  const int g = job.group;

  // ---- queries of this lane: B operand fragments, k = s*16 + hh*8 + [0,8)
  const int64_t qrow = (int64_t)qtile * kBQ + wave * 32 + lq;
  const bool qvalid = qrow < p.n_q;
  bf16x8 qf[DH / 16];
  {
    const uint16_t* qp = (const uint16_t*)p.q + qrow * p.q_stride + (int64_t)head * DH + hh * 8;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      u32x4 v = {0, 0, 0, 0};
      if (qvalid) v = *(const u32x4*)(qp + s * 16);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i) o[i] = (f32x16){};
  float m_c = -INFINITY;  // running max, already multiplied by c
  float l_part = 0.0f;    // this lane's share of the row sum
  const float c = p.c;

  // ---- tile loader state
  u32x4 kreg[T::KPASS];
  uint32_t vreg[T::VITEMS][8];

  auto load_tile = [&](const TileCursor& cur, int nvalid) {
    const AttnSeg sg = p.segs[g][cur.seg];
    const uint16_t* kb = (const uint16_t*)sg.k + cur.row * sg.ks + (int64_t)head * DH;
    const uint16_t* vb = (const uint16_t*)sg.v + cur.row * sg.vs + (int64_t)head * DH;
    const int ch = tid % T::CH;
#pragma unroll
    for (int ps = 0; ps < T::KPASS; ++ps) {
      const int r = ps * T::RPP + tid / T::CH;
      u32x4 v = {0, 0, 0, 0};
      if (r < nvalid) v = *(const u32x4*)(kb + (int64_t)r * sg.ks + ch * 8);
      kreg[ps] = v;
    }
#pragma unroll
    for (int it = 0; it < T::VITEMS; ++it) {
      const int item = tid + 256 * it;
      const int dp = item % T::NDP;
      const int pg = item / T::NDP;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = (pg >> 1) * 16 + (pg & 1) * 4 + (j & 3) + (j >> 2) * 8;
        uint32_t v = 0;
        if (kk < nvalid) v = *(const uint32_t*)(vb + (int64_t)kk * sg.vs + 2 * dp);
        vreg[it][j] = v;
      }
    }
  };

  auto store_tile = [&](int b) {
    const int ch = tid % T::CH;
#pragma unroll
    for (int ps = 0; ps < T::KPASS; ++ps) {
      const int r = ps * T::RPP + tid / T::CH;
      *(u32x4*)&Ks[b][r * T::KS + ch * 8] = kreg[ps];
    }
#pragma unroll
    for (int it = 0; it < T::VITEMS; ++it) {
      const int item = tid + 256 * it;
      const int dp = item % T::NDP;
      const int pg = item / T::NDP;
      u32x4 lo, hi;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a = vreg[it][2 * m], bb = vreg[it][2 * m + 1];
        lo[m] = (a & 0xffffu) | (bb << 16);
        hi[m] = (a >> 16) | (bb & 0xffff0000u);
      }
      *(u32x4*)&Vt[b][(2 * dp) * T::VS + pg * 8] = lo;
      *(u32x4*)&Vt[b][(2 * dp + 1) * T::VS + pg * 8] = hi;
    }
  };

  TileCursor cur;
  bool have = cursor_seek(p, g, 0, job.kbeg, job.kend, cur);
  int nvalid = have ? (int)min<int64_t>(kBK, cur.end - cur.row) : 0;
  if (have) {
    load_tile(cur, nvalid);
    store_tile(0);
  }
  __syncthreads();

  int b = 0;
  while (have) {
    const int nv_cur = nvalid;
    TileCursor nxt = cur;
    const bool have_next = cursor_next(p, g, job.kbeg, job.kend, nxt);
    int nv_next = 0;
    if (have_next) {
      nv_next = (int)min<int64_t>(kBK, nxt.end - nxt.row);
      load_tile(nxt, nv_next);
    }

    // ---- S^T = K Q^T for the two 32-key halves of the tile
    f32x16 s0 = {}, s1 = {};
    const uint16_t* kl = &Ks[b][0];
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      const bf16x8 a0 = *(const bf16x8*)(kl + lq * T::KS + s * 16 + hh * 8);
      const bf16x8 a1 = *(const bf16x8*)(kl + (32 + lq) * T::KS + s * 16 + hh * 8);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
    }
    if (nv_cur < kBK) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kidx = (i >> 2) * 8 + hh * 4 + (i & 3);
        if (kidx >= nv_cur) s0[i] = -INFINITY;
        if (32 + kidx >= nv_cur) s1[i] = -INFINITY;
      }
    }

    // ---- online softmax (row = this lane's query)
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    {
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    const float mxc = mx * c;
    if (__any(mxc > m_c + 8.0f)) {
      const float m_new = fmaxf(m_c, mxc);
      const float alpha = (m_c == -INFINITY) ? 0.0f : exp2f(m_c - m_new);
      if (m_new != -INFINITY) {
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < DH / 32; ++i) o[i] *= alpha;
        m_c = m_new;
      }
    }
    const float m_use = (m_c == -INFINITY) ? 0.0f : m_c;
    bf16x8 pf[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x4 w;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i = gp * 8 + 2 * m;
          const float x0 = t ? s1[i] : s0[i];
          const float x1 = t ? s1[i + 1] : s0[i + 1];
          const float p0 = exp2f(fmaf(x0, c, -m_use));
          const float p1 = exp2f(fmaf(x1, c, -m_use));
          const uint32_t pk = pack_bf16(p0, p1);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                   __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                                   l_part, false);
          w[m] = pk;
        }
        pf[t * 2 + gp] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // ---- O^T += V^T P^T
    const uint16_t* vl = &Vt[b][0];
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const bf16x8 a = *(const bf16x8*)(vl + (dt * 32 + lq) * T::VS + sl * 16 + hh * 8);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[sl], o[dt], 0, 0, 0);
      }
    }

    if (have_next) store_tile(b ^ 1);
    __syncthreads();
    b ^= 1;
    cur = nxt;
    nvalid = nv_next;
    have = have_next;
  }

  // ---- finalise
  float l_tot;
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
    l_tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (!qvalid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* op = job.o + (qrow * p.H + head) * (int64_t)DH;
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = dt * 32 + g4 * 8 + hh * 4;
      f32x4 v = {o[dt][g4 * 4 + 0] * inv, o[dt][g4 * 4 + 1] * inv, o[dt][g4 * 4 + 2] * inv,
                 o[dt][g4 * 4 + 3] * inv};
      *(f32x4*)(op + d0) = v;
    }
  }
  if (hh == 0) {
    job.lse[qrow * p.H + head] = l_tot > 0.0f ? (m_c + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---- d = 128 pipelined kernel ----------------------------------------------
//
// 4 waves x 64 queries (two 32-query blocks per wave, so every K or V^T
// fragment read from LDS feeds two MFMAs); key tiles of 32.
//   * K and V tiles go from global memory straight into LDS (buffer loads with
//     the LDS flag, no VGPR staging), row-major with the 16-byte chunks of a
//     row XOR-swizzled (see swz) so that both the 16-byte K fragment reads and
//     the transposing V reads are free of bank conflicts.
//   * The V^T fragment of O^T = V^T P^T is read with ds_read_b64_tr_b16: in each
//     16-lane group, lane 4r + c reads 4 consecutive d of key row r and the
//     transpose hands lane j the 4 keys at d = 4*(j/4) + j%4.  Two such reads give
//     the 8 keys of one MFMA slot set, in the order the score accumulator holds
//     them.
//   * Software pipeline of one tile: in iteration j the MFMAs of P_{j-1} V_{j-1}
//     and of K_{j+1} Q^T are issued while the softmax of tile j runs on the
//     VALU.  Tiles are loaded three iterations ahead into a ring of five LDS
//     buffers; one barrier per iteration.
namespace d128 {
constexpr int DH = 128;
constexpr int BQ = 256;
constexpr int BK = 32;
constexpr int PD = 3;                  // tiles loaded ahead
constexpr int NBUF = PD + 2;           // live: V_{j-1}, V_j, K_{j+1}, two in flight
constexpr int ROWB = DH * 2;           // bytes per key row in LDS
constexpr int TILEB = BK * ROWB;       // 8 KB per K (or V) tile
constexpr int LPW = TILEB / 1024 / 4;  // 1 KB load instructions per wave per tensor per tile
constexpr int LOADS_PER_TILE = 2 * LPW;
}  // namespace d128

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Tile cursor of the d = 128 kernel: the current segment's K/V row pointers (head
// applied) and byte strides are cached so a step touches kernel arguments only
// when it crosses into the next segment.
struct SegCursor {
  int seg;
  int64_t row, end;          // tile start row and one past the job's last row in this segment
  const char* kp;            // row 0 of the segment, this head
  const char* vp;
  int64_t ksb, vsb;          // row strides in bytes
};

__device__ __forceinline__ bool segc_seek(const AttnParams& p, int g, int head, int seg, int64_t kbeg,
                                          int64_t kend, SegCursor& c) {
  int64_t st = 0;
  for (int s = 0; s < p.n_segs[g]; ++s) {
    const AttnSeg sg = p.segs[g][s];
    const int64_t a = kbeg > st ? kbeg : st;
    const int64_t b = kend < st + sg.n ? kend : st + sg.n;
    if (s >= seg && a < b) {
      c.seg = s;
      c.row = a - st;
      c.end = b - st;
      c.ksb = sg.ks * 2;
      c.vsb = sg.vs * 2;
      c.kp = (const char*)sg.k + (int64_t)head * 256;
      c.vp = (const char*)sg.v + (int64_t)head * 256;
      return true;
    }
    st += sg.n;
  }
  return false;
}

template <int BK>
__device__ __forceinline__ void segc_next(const AttnParams& p, int g, int head, int64_t kbeg, int64_t kend,
                                          SegCursor& c) {
  c.row += BK;
  if (c.row >= c.end) segc_seek(p, g, head, c.seg + 1, kbeg, kend, c);
}

// 16-byte slot of chunk `ch` of key row `row` in an LDS tile: XOR with a
// permutation of (row mod 16) that sends rows 0..15 to distinct values (16-byte
// K reads of 16 consecutive rows hit 16 different slots) and rows 4a..4a+3 to
// values differing in bits 2-3 (the transposing V reads of 4 rows x 4 chunks hit
// 16 different slots).
__device__ __forceinline__ int swz(int row, int ch) { return ch ^ (((row & 3) << 2) | ((row >> 2) & 3)); }
#define ISPA_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt with vmcnt = n (n in {0, LOADS_PER_TILE}), expcnt/lgkmcnt untouched
  if (n == 0)
    __builtin_amdgcn_s_waitcnt(0x0F70);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70 | d128::LOADS_PER_TILE);
}

// One 16-byte-per-lane buffer load written straight to LDS at lds_off + 16*lane.
// Issued as a plain instruction so that the compiler does not serialise later
// LDS reads of other ring buffers behind it; completion is awaited explicitly
// with wait_vmcnt before the barrier that publishes the tile.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_off, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_off), "v"(voff), "s"(r)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

__global__ __launch_bounds__(256, 1) void attn_bf16_d128_kernel(const AttnParams p) {
  using namespace d128;
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * 2 * TILEB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int lq = lane & 31;
  const int g16 = lane >> 4;  // 16-lane group
  const int s16 = lane & 15;

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qtile = logical % p.n_qtiles;
  const uint32_t rest = logical / p.n_qtiles;
  const int head = rest % p.H;
  const int jidx = rest / p.H;
  const AttnJob job = p.jobs[jidx];
  const int g = job.group;

  // ---- this lane's queries (B operand of S^T = K Q^T): block qb, slice s
  const int64_t qrow0 = (int64_t)qtile * BQ + wave * 64 + lq;
  bf16x8 qf[2][DH / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t qrow = qrow0 + qb * 32;
    const uint16_t* qp = (const uint16_t*)p.q + qrow * p.q_stride + (int64_t)head * DH + hh * 8;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      u32x4 v = {0, 0, 0, 0};
      if (qrow < p.n_q) v = *(const u32x4*)(qp + s * 16);
      qf[qb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tiles of this job
  int n_tiles = 0;
  {
    int64_t st = 0;
    for (int s = 0; s < p.n_segs[g]; ++s) {
      const int64_t n = p.segs[g][s].n;
      const int64_t a = job.kbeg > st ? job.kbeg : st;
      const int64_t b = job.kend < st + n ? job.kend : st + n;
      if (a < b) n_tiles += (int)((b - a + BK - 1) / BK);
      st += n;
    }
  }

  // load geometry: instruction i of this wave fills LDS rows (wave*LPW + i)*4 + g16,
  // 16-byte slot s16, which holds global chunk swz(row, s16)
  const uint32_t lds0 = lds_addr(lds);

  auto issue = [&](const SegCursor& cur, int buf) {
    const int nvalid = (int)min<int64_t>(BK, cur.end - cur.row);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cur.kp + cur.row * cur.ksb), 0, (int)(nvalid * cur.ksb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cur.vp + cur.row * cur.vsb), 0, (int)(nvalid * cur.vsb), 0x00020000);
    const uint32_t kdst = lds0 + (buf * 2 + 0) * TILEB;
    const uint32_t vdst = lds0 + (buf * 2 + 1) * TILEB;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int lrow = (wave * LPW + i) * 4 + g16;
      const int row = lrow < nvalid ? lrow : nvalid - 1;  // rows past the end reload a valid row
      const int chunk = swz(lrow, s16);
      const uint32_t dst = (wave * LPW + i) * 1024;
      lds_dma16(rk, kdst + dst, (int)(row * cur.ksb) + chunk * 16);
      lds_dma16(rv, vdst + dst, (int)(row * cur.vsb) + chunk * 16);
    }
  };

  // K fragment for slice s: row lq, 16-byte chunk 2s + hh (swizzled)
  auto k_frag = [&](const char* kb, int s) {
    return *(const bf16x8*)(kb + lq * ROWB + swz(lq, 2 * s + hh) * 16);
  };
  // V^T fragment for key slice gp (16 keys), d-tile dt: two transposing reads
  auto v_frag = [&](const char* vb, int gp, int dt) {
    const int r = s16 >> 2, cc = s16 & 3;
    const int colb = dt * 64 + (g16 & 1) * 32 + cc * 8;  // byte column of the 4 d values
    const int row0 = gp * 16 + (g16 >> 1) * 4 + r;
    const int row1 = row0 + 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        ISPA_LDS_PTR(s16x4, vb + row0 * ROWB + (swz(row0, colb >> 4) << 4) + (colb & 15)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        ISPA_LDS_PTR(s16x4, vb + row1 * ROWB + (swz(row1, colb >> 4) << 4) + (colb & 15)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 o[2][DH / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < DH / 32; ++i) o[qb][i] = (f32x16){};
  float m_c[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.0f, 0.0f};
  const float c = p.c;

  // ---- prologue: issue tiles 0 .. PD-1, wait for tiles 0 and 1
  SegCursor lcur, ccur;
  segc_seek(p, g, head, 0, job.kbeg, job.kend, lcur);
  ccur = lcur;
  int issued = 0, lbuf = 0;  // tiles issued so far; ring slot of the next issue
  for (; issued < PD && issued < n_tiles; ++issued) {
    issue(lcur, lbuf);
    lbuf = lbuf + 1 == NBUF ? 0 : lbuf + 1;
    segc_next<BK>(p, g, head, job.kbeg, job.kend, lcur);
  }
  wait_vmcnt(issued > 2 ? LOADS_PER_TILE : 0);
  __syncthreads();

  f32x16 S_a[2], S_b[2];
  bf16x8 P_a[2][2], P_b[2][2];
  {
    const char* kb = lds;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      const bf16x8 a = k_frag(kb, s);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        S_a[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][s], s == 0 ? (f32x16){} : S_a[qb], 0, 0, 0);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) P_b[qb][gp] = (bf16x8){};  // P_{-1} = 0: the first PV adds nothing
  }

  // One pipeline step for tile j: O += V_{j-1}^T P_{j-1} and S_{j+1} = K_{j+1} Q^T
  // on the matrix cores while the VALU turns S_j into P_j.
  int cbuf = 0;  // ring slot of tile j
  auto step = [&](int j, f32x16 (&s_in)[2], f32x16 (&s_out)[2], const bf16x8 (&p_in)[2][2],
                  bf16x8 (&p_out)[2][2]) {
    const int nv = (int)min<int64_t>(BK, ccur.end - ccur.row);
    segc_next<BK>(p, g, head, job.kbeg, job.kend, ccur);
    if (issued < n_tiles) {
      issue(lcur, lbuf);
      lbuf = lbuf + 1 == NBUF ? 0 : lbuf + 1;
      segc_next<BK>(p, g, head, job.kbeg, job.kend, lcur);
      ++issued;
    }
    const int pbuf = j == 0 ? 0 : (cbuf == 0 ? NBUF - 1 : cbuf - 1);  // tile j-1 (tile 0 when j = 0)
    const int nbuf = cbuf + 1 == NBUF ? 0 : cbuf + 1;                  // tile j+1
    if (nv < BK) {  // last tile of a segment: keys past its end score -inf
      const int lim = nv - hh * 4;  // element i is a valid key iff (i/4)*8 + i%4 < lim
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s_in[qb][i] = ((i >> 2) * 8 + (i & 3) < lim) ? s_in[qb][i] : -INFINITY;
    }
    // (A) P_{j-1} V_{j-1} (tile 0's V with P = 0 when j = 0) + mask + row max
    {
      const char* vb = lds + (pbuf * 2 + 1) * TILEB;
#pragma unroll
      for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) {
          const bf16x8 a = v_frag(vb, gp, dt);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p_in[qb][gp], o[qb][dt], 0, 0, 0);
        }
    }
    float mxc[2];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = s_in[qb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s_in[qb][i]);
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      mxc[qb] = mx * c;
      need |= mxc[qb] > m_c[qb] + 8.0f;
    }
    // rare: raise the running maximum and rescale O and l
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_new = fmaxf(m_c[qb], mxc[qb]);
        if (m_new != -INFINITY) {
          const float alpha = (m_c[qb] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_c[qb] - m_new);
          l_part[qb] *= alpha;
#pragma unroll
          for (int i = 0; i < DH / 32; ++i) o[qb][i] *= alpha;
          m_c[qb] = m_new;
        }
      }
    }
    // (B) S_{j+1} = K_{j+1} Q^T (discarded after the last tile) + P_j = exp2(S_j c - m)
    {
      const char* kb = lds + (nbuf * 2 + 0) * TILEB;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        const bf16x8 a = k_frag(kb, s);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s_out[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][s], s == 0 ? (f32x16){} : s_out[qb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_use = (m_c[qb] == -INFINITY) ? 0.0f : m_c[qb];
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x4 w;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i = gp * 8 + 2 * m;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s_in[qb][i], c, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s_in[qb][i + 1], c, -m_use));
          const uint32_t pk = pack_bf16(p0, p1);
          l_part[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                       __builtin_bit_cast(bf16x2, 0x3f803f80u), l_part[qb], false);
          w[m] = pk;
        }
        p_out[qb][gp] = __builtin_bit_cast(bf16x8, w);
      }
    }
    // tile j+2 must be in LDS for the next step; newer loads may stay in flight
    wait_vmcnt(issued > j + 3 ? LOADS_PER_TILE : 0);
    __syncthreads();
    cbuf = nbuf;
  };

  auto final_pv = [&](const bf16x8 (&pl)[2][2]) {
    const char* vb = lds + (((n_tiles - 1) % NBUF) * 2 + 1) * TILEB;  // tile n-1
#pragma unroll
    for (int gp = 0; gp < 2; ++gp)
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) {
        const bf16x8 a = v_frag(vb, gp, dt);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pl[qb][gp], o[qb][dt], 0, 0, 0);
      }
  };

  int j = 0;
  for (; j + 2 <= n_tiles; j += 2) {
    step(j, S_a, S_b, P_b, P_a);
    step(j + 1, S_b, S_a, P_a, P_b);
  }
  if (j < n_tiles) {
    step(j, S_a, S_b, P_b, P_a);
    final_pv(P_a);
  } else if (n_tiles > 0) {
    final_pv(P_b);
  }

  // ---- finalise
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[qb]), __float_as_uint(l_part[qb]), false, false);
    const float l_tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const int64_t qrow = qrow0 + qb * 32;
    if (qrow >= p.n_q) continue;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* op = job.o + (qrow * p.H + head) * (int64_t)DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + g4 * 8 + hh * 4;
        f32x4 v = {o[qb][dt][g4 * 4 + 0] * inv, o[qb][dt][g4 * 4 + 1] * inv, o[qb][dt][g4 * 4 + 2] * inv,
                   o[qb][dt][g4 * 4 + 3] * inv};
        *(f32x4*)(op + d0) = v;
      }
    }
    if (hh == 0) job.lse[qrow * p.H + head] = l_tot > 0.0f ? (m_c[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// fp32 reference-precision path: one thread per (query, head, job).
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnParams p) {
  const int64_t pairs = p.n_q * p.H;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int jidx = blockIdx.y;
  if (gid >= pairs) return;
  const int64_t qrow = gid / p.H;
  const int head = gid % p.H;
  const AttnJob job = p.jobs[jidx];
  const int g = job.group;
  const float* qp = (const float*)p.q + qrow * p.q_stride + (int64_t)head * DH;
  float qv[DH], acc[DH];
#pragma unroll
  for (int t = 0; t < DH; ++t) {
    qv[t] = qp[t];
    acc[t] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const float c = p.c;
  int64_t st = 0;
  for (int s = 0; s < p.n_segs[g]; ++s) {
    const AttnSeg sg = p.segs[g][s];
    const int64_t a = job.kbeg > st ? job.kbeg : st;
    const int64_t bnd = job.kend < st + sg.n ? job.kend : st + sg.n;
    for (int64_t j = a; j < bnd; ++j) {
      const float* kp = (const float*)sg.k + (j - st) * sg.ks + (int64_t)head * DH;
      const float* vp = (const float*)sg.v + (j - st) * sg.vs + (int64_t)head * DH;
      float dot = 0.0f;
#pragma unroll
      for (int t = 0; t < DH; ++t) dot = fmaf(qv[t], kp[t], dot);
      const float sc = dot * c;
      if (sc > m) {
        const float alpha = exp2f(m - sc);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < DH; ++t) acc[t] *= alpha;
        m = sc;
      }
      const float pr = exp2f(sc - m);
      l += pr;
#pragma unroll
      for (int t = 0; t < DH; ++t) acc[t] = fmaf(pr, vp[t], acc[t]);
    }
    st += sg.n;
  }
  float* op = job.o + (qrow * p.H + head) * (int64_t)DH;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int t = 0; t < DH; ++t) op[t] = acc[t] * inv;
  job.lse[qrow * p.H + head] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  const int tpr = p.d >> 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / tpr;
  const int c4 = gid - row * tpr;
  if (row >= p.n_rows) return;
  float m = -INFINITY;
  for (int k = 0; k < p.n_parts; ++k) m = fmaxf(m, p.lse[k][row]);
  float L = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.0f;
    for (int k = 0; k < p.n_parts; ++k) {
      const float lk = p.lse[k][row];
      if (lk != -INFINITY) tot += expf(lk - m);
    }
    L = m + logf(tot);
  }
  const int64_t off = row * p.d + c4 * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, o0 = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.n_parts; ++k) {
    const float lk = p.lse[k][row];
    const f32x4 ok = *(const f32x4*)(p.o[k] + off);
    if (k == 0) o0 = ok;
    if (lk != -INFINITY && L != -INFINITY) acc += expf(lk - L) * ok;
  }
  if (p.o_full) *(f32x4*)(p.o_full + off) = acc;
  if (p.lse_full && c4 == 0) p.lse_full[row] = L;
  if (p.a0 || p.delta) {
    const f32x4 dl = acc - o0;
    if (p.out_dt == ISPA_F32) {
      if (p.a0) *(f32x4*)((float*)p.a0 + off) = o0;
      if (p.delta) *(f32x4*)((float*)p.delta + off) = dl;
    } else {
      const bool bf = p.out_dt == ISPA_BF16;
      auto pk = [&](float x, float y) { return bf ? pack_bf16(x, y) : pack_f16(x, y); };
      if (p.a0) *(u32x2*)((uint16_t*)p.a0 + off) = (u32x2){pk(o0[0], o0[1]), pk(o0[2], o0[3])};
      if (p.delta) *(u32x2*)((uint16_t*)p.delta + off) = (u32x2){pk(dl[0], dl[1]), pk(dl[2], dl[3])};
    }
  }
}

}  // namespace

ispa_status launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.n_rows == 0) return ISPA_OK;
  const int64_t threads = p.n_rows * (p.d / 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return check_launch("merge_kernel");
}

int attn_block_q(ispa_dtype dt, int32_t d) { return (dt == ISPA_BF16 && d == 128) ? d128::BQ : kBQ; }

SplitPlan plan_splits(int bq, int64_t n_q, int32_t H, const HostGroup* groups, int n_groups) {
  SplitPlan plan;
  int64_t shortest = 0;
  int nonempty = 0;
  for (int g = 0; g < n_groups; ++g) {
    plan.n_splits[g] = 1;
    plan.split_len[g] = groups[g].n_keys();
    const int64_t n = groups[g].n_keys();
    if (n > 0) {
      ++nonempty;
      shortest = shortest == 0 ? n : std::min(shortest, n);
    }
  }
  const int64_t qtiles = (n_q + bq - 1) / bq;
  const int64_t wgs = qtiles * H * std::max(nonempty, 1);
  // Enough workgroups already (several per CU slot): no split.
  constexpr int64_t kTargetWgs = 2048, kMinPiece = 2048;
  if (wgs >= kTargetWgs || nonempty == 0) return plan;
  int64_t piece;
  if (nonempty == 1) {
    // one key set: cut it so the launch reaches the target, pieces >= kMinPiece keys
    const int64_t want = (kTargetWgs + wgs - 1) / wgs;
    const int64_t most = std::max<int64_t>(1, shortest / kMinPiece);
    const int64_t s = std::min<int64_t>(std::min(want, most), 16);
    piece = (shortest + s - 1) / s;
  } else {
    // several groups: pieces about as long as the shortest group, so every
    // work unit has a similar cost
    piece = std::max<int64_t>(shortest, kMinPiece);
  }
  int total = n_groups;
  for (int g = 0; g < n_groups; ++g) {
    const int64_t n = groups[g].n_keys();
    int s = (int)std::max<int64_t>(1, (n + piece - 1) / piece);
    s = std::min(s, 16);
    if (total - 1 + s > kMaxJobs) s = std::max(1, kMaxJobs - (total - 1));
    total += s - 1;
    plan.n_splits[g] = s;
    plan.split_len[g] = s > 1 ? (((n + s - 1) / s + kBK - 1) / kBK) * kBK : n;
  }
  return plan;
}

size_t split_workspace_bytes(int64_t n_q, int32_t H, int32_t d, const SplitPlan& plan, int n_groups) {
  size_t total = 0;
  for (int g = 0; g < n_groups; ++g) {
    if (plan.n_splits[g] > 1) {
      total += plan.n_splits[g] * (align256((size_t)n_q * H * d * 4) + align256((size_t)n_q * H * 4));
    }
  }
  return total;
}

ispa_status run_group_attention(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale,
                                const void* q, int64_t q_stride, const HostGroup* groups,
                                int n_groups, float* const* o_out, float* const* lse_out,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_q == 0) return ISPA_OK;
  AttnParams p{};
  p.q = q;
  p.q_stride = q_stride;
  p.n_q = n_q;
  p.H = H;
  const int bq = attn_block_q(dt, d);
  p.n_qtiles = (int)((n_q + bq - 1) / bq);
  p.c = scale * kLog2e;
  for (int g = 0; g < n_groups; ++g) {
    p.n_segs[g] = groups[g].n_segs;
    for (int s = 0; s < groups[g].n_segs; ++s) {
      const ispa_seg& sg = groups[g].segs[s];
      p.segs[g][s] = AttnSeg{sg.k, sg.v, sg.n, sg.k_stride, sg.v_stride};
    }
  }
  const SplitPlan plan = plan_splits(bq, n_q, H, groups, n_groups);
  if (split_workspace_bytes(n_q, H, d, plan, n_groups) > ws_bytes) {
    set_error("attention workspace too small");
    return ISPA_ERR_WORKSPACE;
  }
  // jobs: longest first so the tail of the launch is short work
  struct Pending {
    int g;
    int64_t kb, ke;
    float* o;
    float* lse;
  };
  Pending pend[kMaxJobs];
  int nj = 0;
  char* wsp = (char*)ws;
  MergeParams merges[2];
  int n_merges = 0;
  for (int g = 0; g < n_groups; ++g) {
    const int64_t n = groups[g].n_keys();
    if (plan.n_splits[g] == 1) {
      pend[nj++] = Pending{g, 0, n, o_out[g], lse_out[g]};
      continue;
    }
    MergeParams mp{};
    mp.n_parts = plan.n_splits[g];
    mp.d = d;
    mp.n_rows = n_q * H;
    mp.o_full = o_out[g];
    mp.lse_full = lse_out[g];
    mp.out_dt = ISPA_F32;
    for (int s = 0; s < plan.n_splits[g]; ++s) {
      float* po = (float*)wsp;
      wsp += align256((size_t)n_q * H * d * 4);
      float* pl = (float*)wsp;
      wsp += align256((size_t)n_q * H * 4);
      const int64_t kb = std::min<int64_t>(n, s * plan.split_len[g]);
      const int64_t ke = std::min<int64_t>(n, (s + 1) * plan.split_len[g]);
      pend[nj++] = Pending{g, kb, ke, po, pl};
      mp.o[s] = po;
      mp.lse[s] = pl;
    }
    merges[n_merges++] = mp;
  }
  std::stable_sort(pend, pend + nj, [](const Pending& a, const Pending& b) {
    return (a.ke - a.kb) > (b.ke - b.kb);
  });
  p.n_jobs = nj;
  for (int j = 0; j < nj; ++j) {
    p.jobs[j] = AttnJob{pend[j].g, 0, pend[j].kb, pend[j].ke, pend[j].o, pend[j].lse};
  }
  if (dt == ISPA_BF16) {
    const int64_t blocks = (int64_t)p.n_qtiles * H * nj;
    if (d == 128)
      hipLaunchKernelGGL(attn_bf16_d128_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    const int64_t pairs = n_q * H;
    const dim3 grid((unsigned)((pairs + 63) / 64), (unsigned)nj);
    if (d == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, p);
  }
  ispa_status st = check_launch("attention kernel");
  if (st != ISPA_OK) return st;
  for (int i = 0; i < n_merges; ++i) {
    st = launch_merge(merges[i], stream);
    if (st != ISPA_OK) return st;
  }
  return ISPA_OK;
}

}  // namespace ispa
