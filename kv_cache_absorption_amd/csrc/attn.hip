// Attention over key groups, returning normalised output and log-sum-exp.
//
// Per query row and head the kernels compute, over the keys of one job,
//   lse = ln sum_j exp(s_j),  o = sum_j exp(s_j - lse) v_j,  s_j = scale <q, k_j>
// with a running (online) maximum so the score matrix is never stored.  This
// is the per-group state the dual-stream warmup relies on (EN review, Key
// Design 1: each group returns its weighted values and its LSE).
//
// bf16 path, d = 64: one workgroup = 4 waves x 32 queries of one head (d = 128
// has its own kernel further down, described there):
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

// ---- helpers of the d = 128 kernel --------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Tile cursor of the d = 128 kernel: the current segment's K/V row pointers (head
// applied) and byte strides are cached so a step touches kernel arguments only
// when it crosses into the next segment.
struct SegCursor {
  int seg;
  int64_t row, end;  // tile start row and one past the job's last row in this segment
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

// One 16-byte-per-lane buffer load written straight to LDS at lds_off + 16*lane.
// Issued as a plain instruction so that the compiler does not serialise later
// LDS reads of other ring buffers behind it; completion is awaited explicitly
// with s_waitcnt vmcnt before the barrier that publishes the tile.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_off, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_off), "v"(voff), "s"(r)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// XOR mask of the swizzle: swz(row, ch) == ch ^ swz_mask(row)
__device__ __forceinline__ int swz_mask(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// ---- d = 128 kernel ----------------------------------------------------------
//
// 8 waves x 32 queries of one head per workgroup (two waves per SIMD), key
// tiles of 64, one workgroup per CU.  Each wave software-pipelines its tiles
// so that the matrix core and the vector ALU work on different tiles in the
// same stretch of code (a wave's VALU instructions issue in the shadow of its
// own MFMAs).  Iteration t runs in two halves of 16 steps:
//   1. O += V_{t-1}^T P_{t-1}^T on the matrix core, while the VALU forms
//      P_t = exp2(S_t c - m) (c = scale * log2(e)) packed to bf16;
//   2. S_{t+1} = K_{t+1} Q^T on the matrix core (into the registers of S_t,
//      now consumed), while the VALU adds the row sums of P_t.
// Lazy re-basing without row maxima in the common path: the reference m is
// set 7 (log2 units) above the largest scaled score seen, so every P of the
// keys seen is at most 2^-7, and P_t is formed with the current m before any
// test.  Half 1 ORs the packed bf16 words of P_t; the exponent's top bit of
// either half is set exactly when some P >= 2 (or inf / NaN, as in the first
// tile, where m = -inf), i.e. when a score passes the largest seen by more
// than 8.  Only then (the first tile, and rarely after it) the tile's row
// maxima are taken, m is raised, l and O are scaled and P_t is formed again
// while S_t is still in its registers.  Any m gives the same result in exact
// arithmetic.
//   * One iteration form for every tile: iteration 0 multiplies a zeroed
//     P_{-1} with a zeroed V slot, and keys past the end of a segment (all keys
//     of the final iteration) are masked to -inf behind a uniform branch.
//   * Every LDS fragment address is a per-lane register plus an immediate: K
//     slots occupy the first 64 KB and V slots the second, and the tile loop
//     is unrolled by the ring size so the slot offsets are constants.  Each
//     step reads its fragment LA steps ahead; a scheduling boundary per step
//     keeps the compiler from sinking the reads onto their MFMAs.
//   * K and V tiles go from global memory straight into two rings of four
//     slots (buffer loads with the LDS flag, rows XOR-swizzled so that the
//     16-byte K reads and the transposing V reads are conflict-free).  K of
//     tile u is read in iteration u - 1 and issued in iteration u - 4; V of
//     tile u is read in iteration u + 1 and issued in iteration u - 2; one
//     barrier per iteration publishes the loads and frees the slots.
//   * S^T = K Q^T puts a query in each lane's accumulator column, so row
//     statistics are in-register reductions plus one v_permlane32_swap; the V^T
//     fragments of O^T = V^T P^T come from ds_read_b64_tr_b16 in the key order
//     of the score accumulator.
//   * QB query blocks per wave share each K or V fragment; QB = 1 with 8 waves
//     measured fastest (QB = 2 with 4 waves leaves one wave per SIMD and
//     nothing to cover its stalls).
namespace a5 {
constexpr int DH = 128;
constexpr int WAVES = 8;
constexpr int QB = 1;                  // 32-query blocks per wave
constexpr int BQ = WAVES * QB * 32;
constexpr int BK = 64;
constexpr int NSLOT = 4;               // ring slots for K and for V
constexpr int ROWB = DH * 2;
constexpr int TILEB = BK * ROWB;       // 16 KB per K (or V) tile
constexpr int VBASE = NSLOT * TILEB;   // V slots follow the K slots
constexpr int LPW = TILEB / 1024 / WAVES;  // 1 KB load instructions per wave per tile and tensor
constexpr int LA = 2;                  // LDS fragments read ahead of their MFMA
static_assert(LPW * WAVES * 1024 == TILEB, "tile load split");
static_assert(2 * NSLOT * TILEB <= 160 * 1024, "LDS budget");
// s_waitcnt immediate that waits until at most n vector memory operations are
// outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
}  // namespace a5

// kRuns: every job covers at most two runs of consecutive rows (one run per
// segment it overlaps); tile addresses are then computed from the tile index.
// kDual (with kRuns): one workgroup per (query tile, head) attends to the
// local group and then to the history group, each by the whole tile pipeline
// below (one pass per group).  Between the passes the local output goes to
// o_stash unnormalised, straight from the accumulators, and the running
// maximum and sum restart; the epilogue reads it back, merges the two groups
// by their log-sum-exp and writes A_loc, A_full - A_loc and the merged LSE,
// so no partial result is written per key piece and no merge kernel runs.
template <bool kRuns, bool kDual = false>
__global__ __launch_bounds__(a5::WAVES * 64, 1) void attn_bf16_d128_kernel(const AttnParams p) {
  using namespace a5;
  __shared__ __attribute__((aligned(1024))) char lds[2 * NSLOT * TILEB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int lq = lane & 31;
  const int g16 = lane >> 4;
  const int s16 = lane & 15;

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qtile = logical % p.n_qtiles;
  const uint32_t rest = logical / p.n_qtiles;
  const int head = rest % p.H;
  const int jidx = rest / p.H;
  const AttnJob job = p.jobs[jidx];
  const float c = p.c;

  // this lane's queries (B operand of S^T = K Q^T): block qb, slices of 16 d
  const int64_t qrow0 = (int64_t)qtile * BQ + wave * (QB * 32) + lq;
  bf16x8 qf[QB][DH / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t qrow = qrow0 + qb * 32;
    const uint16_t* qp = (const uint16_t*)p.q + qrow * p.q_stride + (int64_t)head * DH + hh * 8;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      u32x4 v = {0, 0, 0, 0};
      if (qrow < p.n_q) v = *(const u32x4*)(qp + s * 16);
      qf[qb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[QB][DH / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < DH / 32; ++i) o[qb][i] = (f32x16){};
  float m[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l_part[qb] = 0.0f;
  }
  float l_loc[QB], m_loc[QB];  // kDual: the local group's row sum (total) and maximum
  constexpr int kPasses = kDual ? 2 : 1;
#pragma unroll 1
  for (int pass = 0; pass < kPasses; ++pass) {
  const int g = kDual ? pass : job.group;
  int64_t kbeg = job.kbeg, kend = job.kend;
  if constexpr (kDual) {
    kbeg = 0;
    kend = 0;
    for (int s = 0; s < p.n_segs[g]; ++s) kend += p.segs[g][s].n;
    if (pass == 1) {
      // the local group is complete: keep its output, row sum and maximum and
      // restart for the history group
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[qb]), __float_as_uint(l_part[qb]), false,
                                                  false);
        l_loc[qb] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        m_loc[qb] = m[qb];
        m[qb] = -INFINITY;
        l_part[qb] = 0.0f;
        const int64_t qrow = qrow0 + qb * 32;
        float* sp = p.o_stash + (qrow * p.H + head) * (int64_t)DH + hh * 4;
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) {
          if (qrow < p.n_q) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              *(f32x4*)(sp + dt * 32 + g4 * 8) = (f32x4){o[qb][dt][g4 * 4], o[qb][dt][g4 * 4 + 1],
                                                         o[qb][dt][g4 * 4 + 2], o[qb][dt][g4 * 4 + 3]};
          }
          o[qb][dt] = (f32x16){};
        }
      }
    }
  }
  int n_tiles = 0;
  {
    int64_t st = 0;
    for (int s = 0; s < p.n_segs[g]; ++s) {
      const int64_t n = p.segs[g][s].n;
      const int64_t a = kbeg > st ? kbeg : st;
      const int64_t b = kend < st + n ? kend : st + n;
      if (a < b) n_tiles += (int)((b - a + BK - 1) / BK);
      st += n;
    }
  }

  // per-lane LDS byte offsets of the fragments; slot, key block and key group
  // offsets are immediates.  K row lq (of each 32-key block), 16-byte chunk
  // 2s + hh: the chunk bits sit below the row bits, so the offset of slice s is
  // kbase ^ (s << 5), one XOR in the VALU-light half of the iteration.
  const uint32_t kbase = lq * ROWB + ((hh ^ swz_mask(lq)) << 4);
  uint32_t voff0[DH / 32], voff1[DH / 32];  // V rows r0, r0 + 8 of each 16-key group, d-tile dt
  {
    const int r0 = (g16 >> 1) * 4 + (s16 >> 2), r1 = r0 + 8;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt) {
      const int colb = dt * 64 + (g16 & 1) * 32 + (s16 & 3) * 8;
      voff0[dt] = VBASE + r0 * ROWB + (((colb >> 4) ^ swz_mask(r0)) << 4) + (colb & 15);
      voff1[dt] = VBASE + r1 * ROWB + (((colb >> 4) ^ swz_mask(r1)) << 4) + (colb & 15);
    }
  }
  // fragment i of S = K Q^T: key block i / 8, d slice i % 8
  auto k_frag = [&](const int ks, const int i) __attribute__((always_inline)) {
    const uint32_t off = (i & 7) ? (kbase ^ ((uint32_t)(i & 7) << 5)) : kbase;
    return *(const bf16x8*)(lds + off + ks + (i >> 3) * 32 * ROWB);
  };
  auto v_frag = [&](const int vs, const int gp, const int dt) __attribute__((always_inline)) {
    const int off = vs + gp * 16 * ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS_PTR(s16x4, lds + voff0[dt] + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS_PTR(s16x4, lds + voff1[dt] + off));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  const uint32_t lds0 = lds_addr(lds);
  // K and V tile streams over the job's rows.  Inside a segment every full tile
  // takes the short path: a buffer descriptor over the tile's 64 rows, per-lane
  // offsets fixed for the segment, one 64-bit pointer step and a countdown; a
  // partial tile (its rows past the end reload a valid row) and the move to the
  // next segment take the long path.
  struct Stream {
    SegCursor c;
    const char* tile;  // first row of the next tile, this head
    int64_t sb;        // row stride in bytes
    int full;          // full tiles left from c.row in this segment
    int voff[LPW];     // this lane's byte offsets inside a full tile
  };
  auto stream_init = [&](Stream& st, const bool is_v) __attribute__((always_inline)) {
    const AttnSeg sg = p.segs[g][st.c.seg];  // segment pointers and strides, read on segment changes
    st.sb = (is_v ? sg.vs : sg.ks) * 2;
    st.tile = (const char*)(is_v ? sg.v : sg.k) + (int64_t)head * 256 + st.c.row * st.sb;
    st.full = (int)((st.c.end - st.c.row) / BK);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int lrow = (wave * LPW + i) * 4 + g16;
      st.voff[i] = lrow * (int)st.sb + swz(lrow, s16) * 16;
    }
  };
  // One tile load of this wave, prepared at the start of an iteration and issued
  // (LPW instructions) in the middle of it: a buffer descriptor, this lane's
  // byte offsets and the LDS destination.
  struct Load {
    __amdgpu_buffer_rsrc_t r;
    int voff[LPW];
    uint32_t dst;
  };
  // the stream's next tile into LDS at dst (then advance); when `real` is false
  // an empty descriptor stands in, so that every iteration issues the same
  // number of loads (they write nothing that is read: their slot is free)
  auto stream_prep = [&](Stream& st, const bool is_v, const uint32_t dst, const bool real) __attribute__((always_inline)) {
    Load ld;
    ld.dst = dst;
    if (!real) {
      ld.r = __builtin_amdgcn_make_buffer_rsrc((void*)st.tile, 0, 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < LPW; ++i) ld.voff[i] = 0;
      return ld;
    }
    if (st.full > 0) {
      ld.r = __builtin_amdgcn_make_buffer_rsrc((void*)st.tile, 0, (int)(BK * st.sb), 0x00020000);
#pragma unroll
      for (int i = 0; i < LPW; ++i) ld.voff[i] = st.voff[i];
      st.tile += BK * st.sb;
      st.c.row += BK;
      if (--st.full == 0 && st.c.row >= st.c.end) {
        asm volatile("" ::: "memory");  // the segment ends on a tile boundary: next segment
        if (segc_seek(p, g, head, st.c.seg + 1, kbeg, kend, st.c)) stream_init(st, is_v);
      }
      return ld;
    }
    asm volatile("" ::: "memory");  // partial tile: rows past the end reload the last valid row
    const int nvalid = (int)min<int64_t>(BK, st.c.end - st.c.row);
    ld.r = __builtin_amdgcn_make_buffer_rsrc((void*)st.tile, 0, (int)(nvalid * st.sb), 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int lrow = (wave * LPW + i) * 4 + g16;
      const int row = lrow < nvalid ? lrow : nvalid - 1;
      ld.voff[i] = (int)(row * st.sb) + swz(lrow, s16) * 16;
    }
    st.c.row += BK;
    if (segc_seek(p, g, head, st.c.seg + 1, kbeg, kend, st.c)) stream_init(st, is_v);
    return ld;
  };
  auto issue_load = [&](const Load& ld, const int i) __attribute__((always_inline)) {
    lds_dma16(ld.r, ld.dst + (wave * LPW + i) * 1024, ld.voff[i]);
  };
  Stream ks_, vs_;
  SegCursor ccur;
  int cfull = 0;  // full tiles left from ccur.row in its segment
  segc_seek(p, g, head, 0, kbeg, kend, ccur);
  ks_.c = vs_.c = ccur;
  stream_init(ks_, false);
  stream_init(vs_, true);
  cfull = (int)((ccur.end - ccur.row) / BK);
  // keys of the next tile in job order (64 for a full tile)
  auto next_nv_stream = [&]() __attribute__((always_inline)) {
    if (cfull > 0) {
      ccur.row += BK;
      if (--cfull == 0 && ccur.row >= ccur.end) {
        asm volatile("" ::: "memory");
        if (segc_seek(p, g, head, ccur.seg + 1, kbeg, kend, ccur)) cfull = (int)((ccur.end - ccur.row) / BK);
      }
      return BK;
    }
    asm volatile("" ::: "memory");
    const int nv = (int)(ccur.end - ccur.row);
    ccur.row += BK;
    if (segc_seek(p, g, head, ccur.seg + 1, kbeg, kend, ccur)) cfull = (int)((ccur.end - ccur.row) / BK);
    return nv;
  };

  // Two-run addressing: run r of the job starts at row base (this head) with
  // `tiles` tiles, the last holding `tail` keys.  The load of a tile is a few
  // scalar selects and one multiply; rows past the run's end reload its last
  // row (a per-lane min), and tiles past the job's end get an empty descriptor.
  struct Run {
    const char* k;
    const char* v;
    int ksb, vsb, tiles, tail;
  };
  Run r0{}, r1{};
  if constexpr (kRuns) {
    int64_t st = 0;
    int nr = 0;
    for (int s = 0; s < p.n_segs[g]; ++s) {
      const AttnSeg sg = p.segs[g][s];
      const int64_t a = kbeg > st ? kbeg : st;
      const int64_t b = kend < st + sg.n ? kend : st + sg.n;
      if (a < b) {
        Run r;
        r.ksb = (int)(sg.ks * 2);
        r.vsb = (int)(sg.vs * 2);
        r.k = (const char*)sg.k + (int64_t)head * 256 + (a - st) * r.ksb;
        r.v = (const char*)sg.v + (int64_t)head * 256 + (a - st) * r.vsb;
        r.tiles = (int)((b - a + BK - 1) / BK);
        r.tail = (int)(b - a) - (r.tiles - 1) * BK;
        if (nr == 0) r0 = r;
        else r1 = r;  // the host launches this form only for jobs of at most two runs
        ++nr;
      }
      st += sg.n;
    }
  }
  int swzo[LPW];  // this lane's chunk offset in its load rows
#pragma unroll
  for (int i = 0; i < LPW; ++i) swzo[i] = swz((wave * LPW + i) * 4 + g16, s16) * 16;
  // keys of tile `tile` of the job (0 past its end)
  auto run_nv = [&](const int tile) __attribute__((always_inline)) {
    const bool in1 = tile >= r0.tiles;
    const int tr = in1 ? tile - r0.tiles : tile;
    const int nv = tr < (in1 ? r1.tiles : r0.tiles) - 1 ? BK : (in1 ? r1.tail : r0.tail);
    return tile < n_tiles ? nv : 0;
  };
  auto run_load = [&](const int tile, const bool is_v, const uint32_t dst) __attribute__((always_inline)) {
    const bool in1 = tile >= r0.tiles;
    const int tr = in1 ? tile - r0.tiles : tile;
    const char* base = is_v ? (in1 ? r1.v : r0.v) : (in1 ? r1.k : r0.k);
    const int sb = is_v ? (in1 ? r1.vsb : r0.vsb) : (in1 ? r1.ksb : r0.ksb);
    const int nv = run_nv(tile);
    Load ld;
    ld.dst = dst;
    ld.r = __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)tr * (BK * sb)), 0, nv * sb, 0x00020000);
    const int lastrow = nv > 0 ? nv - 1 : 0;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int lrow = (wave * LPW + i) * 4 + g16;
      ld.voff[i] = min(lrow, lastrow) * sb + swzo[i];
    }
    return ld;
  };
  auto next_nv = [&](const int t) __attribute__((always_inline)) {
    if constexpr (kRuns) return run_nv(t);
    else return t < n_tiles ? next_nv_stream() : 0;
  };
  // Iteration i (prologue iterations -4 .. -1 included) loads K_{i+4} and, from
  // i = -2 on, V_{i+2}, real or stand-in, so the load count is the same in every
  // iteration.  At the end of iteration t, K_{t+2} and V_t (loaded in iteration
  // t - 2) must be in LDS while the 4 * LPW loads of iterations t - 1 and t
  // (K_{t+3}, V_{t+1}, K_{t+4}, V_{t+2}) may stay in flight; loads complete in
  // issue order.
  auto prep_k = [&](int i) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + ((i + 4) % NSLOT) * TILEB;
    if constexpr (kRuns) return run_load(i + 4, false, dst);
    else return stream_prep(ks_, false, dst, i + 4 < n_tiles);
  };
  auto prep_v = [&](int i) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + VBASE + ((i + 2) % NSLOT) * TILEB;
    if constexpr (kRuns) return run_load(i + 2, true, dst);
    else return stream_prep(vs_, true, dst, i + 2 < n_tiles);
  };
  auto wait_iter = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * LPW)); };

  f32x16 S[QB][2];  // [query block][key block]: S_t, then S_{t+1}
  // P as packed bf16 pairs [buffer][query block][pair]; pairs 4g .. 4g+3 form
  // the MFMA operand of key group g (32-bit words: the row sums read them one
  // at a time)
  uint32_t P[2][QB][16];
  auto p_frag = [&](const int b, const int qb, const int gp) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, (u32x4){P[b][qb][4 * gp], P[b][qb][4 * gp + 1], P[b][qb][4 * gp + 2],
                                              P[b][qb][4 * gp + 3]});
  };
  // P pair k of query block qb into P[b] (uses m)
  auto exp_pair = [&](const int b, const int qb, const int k) __attribute__((always_inline)) {
    const int blk = k >> 3, i = (k & 7) * 2;
    P[b][qb][k] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(S[qb][blk][i], c, -m[qb])),
                            __builtin_amdgcn_exp2f(fmaf(S[qb][blk][i + 1], c, -m[qb])));
  };
  // the same in two parts, so that the pack of pair k can go one step after its
  // exps (a VALU use right after a transcendental costs a wait state)
  auto exp_two = [&](const int qb, const int k, float (&e)[2]) __attribute__((always_inline)) {
    const int blk = k >> 3, i = (k & 7) * 2;
    e[0] = __builtin_amdgcn_exp2f(fmaf(S[qb][blk][i], c, -m[qb]));
    e[1] = __builtin_amdgcn_exp2f(fmaf(S[qb][blk][i + 1], c, -m[qb]));
  };
  // this lane's maximum over the 16 scores of key block blk of query block qb
  auto blk_max = [&](const int qb, const int blk) __attribute__((always_inline)) {
    float mx = S[qb][blk][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[qb][blk][i]);
    return mx;
  };
  // Re-basing (the rare path after half 1, entered when some packed P_t >= 2):
  // the tile's row maxima (lanes l and l + 32 hold the two key halves of one
  // query) raise m to max + kHead for every row whose maximum passed m - 0.5,
  // and l and O (which holds P_{t-1} V_{t-1}, formed with the old m) are scaled
  // by alpha = 2^(m_old - m_new), 0 when m_old = -inf.  P_t is then formed again.
  constexpr float kHead = 7.0f;
  auto rebase = [&](const int cb) __attribute__((always_inline)) {
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mx_lane = fmaxf(blk_max(qb, 0), blk_max(qb, 1));
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx_lane), __float_as_uint(mx_lane), false, false);
      const float mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * c;
      const bool up = mx - m[qb] > 0.5f;
      alpha[qb] = up ? __builtin_amdgcn_exp2f(m[qb] - (mx + kHead)) : 1.0f;
      m[qb] = up ? mx + kHead : m[qb];
      l_part[qb] *= alpha[qb];
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) o[qb][dt] *= alpha[qb];
#pragma unroll
      for (int k = 0; k < 16; ++k) exp_pair(cb, qb, k);
    }
  };
  // Both halves of an iteration run 16 steps of QB MFMAs each (one per query
  // block, sharing one K or V fragment); the fragment of step i is read LA
  // steps ahead, and the last LA steps of half 1 read the first K fragments of
  // half 2 (K_{t+1} has been in LDS since the last barrier).  Every iteration has this one form: iteration 0 multiplies a
  // zeroed P_{-1} with a zeroed V slot, and scores of keys past the end of a
  // segment (all keys of iteration n_tiles) are masked to -inf, which makes
  // their P exactly 0.
  // half 1: step i = O^T += V^T P^T for key group i / 4, d-tile i % 4 (P_{t-1})
  // on the matrix core; P_t pair i on the VALU, and the OR of its packed words
  // into orw
  auto half1 = [&](const int vs, const int ks, const int cb, bf16x8(&kf)[16], uint32_t(&orw)[QB])
                   __attribute__((always_inline)) {
    bf16x8 vf[16];
#pragma unroll
    for (int i = 0; i < LA; ++i) vf[i] = v_frag(vs, i >> 2, i & 3);
    float e[2][QB][2];  // exps of pairs i (buffer i & 1), packed in step i + 1
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + LA < 16) vf[i + LA] = v_frag(vs, (i + LA) >> 2, (i + LA) & 3);
      else kf[i + LA - 16] = k_frag(ks, i + LA - 16);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        exp_two(qb, i, e[i & 1][qb]);
        if (i > 0) {
          P[cb][qb][i - 1] = pack_bf16(e[(i - 1) & 1][qb][0], e[(i - 1) & 1][qb][1]);
          orw[qb] = i == 1 ? P[cb][qb][0] : orw[qb] | P[cb][qb][i - 1];
        }
        if (i == 15) {
          P[cb][qb][15] = pack_bf16(e[1][qb][0], e[1][qb][1]);
          orw[qb] |= P[cb][qb][15];
        }
        o[qb][i & 3] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], p_frag(cb ^ 1, qb, i >> 2), o[qb][i & 3], 0, 0, 0);
      }
      // QB MFMAs, 2 LDS reads, 6 VALU per query block (2 FMA, 2 exp, pack, OR);
      // the step boundary keeps each read LA steps ahead of its MFMA
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6 * QB, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P_t is formed here, not sunk past the re-basing branch into its users
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t(&w)[16] = P[cb][qb];
      asm volatile("" ::"v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]),
                   "v"(w[8]), "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15]));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // half 2: step i = S_{t+1} += K Q^T for key block i / 8, d slice i % 8 on the
  // matrix core; row sum of P_t pair i on the VALU.  The iteration's loads are
  // issued here, spread over the half so that the waves do not queue behind
  // each other on the load path.
  auto half2 = [&](const int ks, const int cb, bf16x8(&kf)[16], const Load& lk, const Load& lv)
                   __attribute__((always_inline)) {
    static_assert(LPW == 2, "load placement in half 2");
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i == 1) issue_load(lk, 0);
      if (i == 5) issue_load(lk, 1);
      if (i == 9) issue_load(lv, 0);
      if (i == 13) issue_load(lv, 1);
      if (i + LA < 16) kf[i + LA] = k_frag(ks, i + LA);
      const int blk = i >> 3, sl = i & 7;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_part[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, P[cb][qb][i]),
                                                     __builtin_bit_cast(bf16x2, 0x3f803f80u), l_part[qb], false);
        S[qb][blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[qb][sl], sl == 0 ? (f32x16){} : S[qb][blk],
                                                             0, 0, 0);
      }
      // QB MFMAs, 1 LDS read, the address XOR and a row sum per query block
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 1 + QB, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Iteration t: ring slot u = t mod 4, P_t into buffer cb = t mod 2 (P_{t-1}
  // is in buffer cb ^ 1).
  auto run_iter = [&](const int t, const int u, const int cb) __attribute__((always_inline)) {
    const Load lk = prep_k(t), lv = prep_v(t);
    const int nv = next_nv(t);  // keys of tile t
    if (nv < BK) {  // keys past the end of the segment score -inf
      asm volatile("" ::: "memory");  // a branch, not a select in every iteration
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int lim = nv - blk * 32 - hh * 4;  // element i is key blk*32 + (i/4)*8 + hh*4 + i%4
#pragma unroll
          for (int i = 0; i < 16; ++i)
            S[qb][blk][i] = ((i >> 2) * 8 + (i & 3) < lim) ? S[qb][blk][i] : -INFINITY;
        }
      }
    }
    const int ks = ((u + 1) & 3) * TILEB, vs = ((u + 3) & 3) * TILEB;
    bf16x8 kf[16];
    uint32_t orw[QB];
    half1(vs, ks, cb, kf, orw);
    // some P_t >= 2 (exponent field >= 128 in either bf16 half), inf or NaN
    bool hot = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) hot = hot || (orw[qb] & 0x40004000u) != 0u;
    if (__any(hot)) {
      asm volatile("" ::: "memory");  // keep the rare path a branch (not speculated)
      rebase(cb);
    }
    half2(ks, cb, kf, lk, lv);
    wait_iter();
    __syncthreads();
  };
  if (n_tiles > 0) {
    // P_{-1} = 0 and a zeroed V slot 3 (read by iteration 0; first loaded by
    // iteration 1, after iteration 0's closing barrier): iteration 0 adds 0 to O
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int k = 0; k < 16; ++k) P[1][qb][k] = 0u;
    constexpr int ZB = TILEB / (WAVES * 64);  // bytes zeroed per thread
    static_assert(ZB % 16 == 0, "V slot zeroing");
#pragma unroll
    for (int j = 0; j < ZB; j += 16) *(u32x4*)(lds + VBASE + 3 * TILEB + tid * ZB + j) = (u32x4){0, 0, 0, 0};
    // prologue: iterations -4 .. -1 issue K_0..K_3, V_0, V_1; S_0 = K_0 Q^T
    for (int i = -4; i < 0; ++i) {
      const Load lk = prep_k(i);
#pragma unroll
      for (int j = 0; j < LPW; ++j) issue_load(lk, j);
      if (i + 2 >= 0) {
        const Load lv = prep_v(i);
#pragma unroll
        for (int j = 0; j < LPW; ++j) issue_load(lv, j);
      }
    }
    wait_iter();  // K_0 and K_1 are in LDS
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int blk = i >> 3, sl = i & 7;
      const bf16x8 kfr = k_frag(0, i);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        S[qb][blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qf[qb][sl], sl == 0 ? (f32x16){} : S[qb][blk],
                                                             0, 0, 0);
    }
    __syncthreads();  // every wave has read K_0 before iteration 0 loads K_4 into its slot
    // iterations 0 .. n_tiles, unrolled by the ring size
    for (int t = 0;;) {
      run_iter(t, 0, 0);
      if (++t > n_tiles) break;
      run_iter(t, 1, 1);
      if (++t > n_tiles) break;
      run_iter(t, 2, 0);
      if (++t > n_tiles) break;
      run_iter(t, 3, 1);
      if (++t > n_tiles) break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no LDS write in flight when the pass ends
  }
  }  // pass

  if constexpr (kDual) {
    // merge: A_full = (1 - sigma) A_loc + sigma O_hist with sigma the history
    // group's share of the softmax mass (from the two LSEs), so
    // A_full - A_loc = sigma (O_hist - A_loc), all in fp32
    const bool out_bf = p.out_dt == ISPA_BF16;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[qb]), __float_as_uint(l_part[qb]), false,
                                                false);
      const float l_h = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      const int64_t qrow = qrow0 + qb * 32;
      if (qrow >= p.n_q) continue;
      const float lse0 = l_loc[qb] > 0.0f ? m_loc[qb] + log2f(l_loc[qb]) : -INFINITY;  // log2 units
      const float lse1 = l_h > 0.0f ? m[qb] + log2f(l_h) : -INFINITY;
      const float mm = fmaxf(lse0, lse1);
      float sigma = 0.0f, lse = -INFINITY;
      if (mm != -INFINITY) {
        const float e0 = exp2f(lse0 - mm), e1 = exp2f(lse1 - mm);
        sigma = e1 / (e0 + e1);
        lse = (mm + log2f(e0 + e1)) * kLn2;
      }
      const float inv_h = l_h > 0.0f ? 1.0f / l_h : 0.0f;
      const float inv_l = l_loc[qb] > 0.0f ? 1.0f / l_loc[qb] : 0.0f;
      const int64_t base = (qrow * p.H + head) * (int64_t)DH;
      // this lane's own stores between the passes (complete: the first pass
      // ended with vmcnt(0)), read back
      const float* sp = p.o_stash + base + hh * 4;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = dt * 32 + g4 * 8 + hh * 4;
          const f32x4 ol = *(const f32x4*)(sp + dt * 32 + g4 * 8);
          float a[4], dl[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = ol[e] * inv_l;
            dl[e] = sigma * (o[qb][dt][g4 * 4 + e] * inv_h - a[e]);
          }
          *(u32x2*)((uint16_t*)p.a_loc + base + d0) =
              out_bf ? (u32x2){pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3])}
                     : (u32x2){pack_f16(a[0], a[1]), pack_f16(a[2], a[3])};
          *(u32x2*)((uint16_t*)p.delta + base + d0) =
              out_bf ? (u32x2){pack_bf16(dl[0], dl[1]), pack_bf16(dl[2], dl[3])}
                     : (u32x2){pack_f16(dl[0], dl[1]), pack_f16(dl[2], dl[3])};
        }
      }
      if (hh == 0 && p.lse_full) p.lse_full[qrow * p.H + head] = lse;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[qb]), __float_as_uint(l_part[qb]), false, false);
    const float l_tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const int64_t qrow = qrow0 + qb * 32;
    if (qrow >= p.n_q) continue;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t base = (qrow * p.H + head) * (int64_t)DH;
    const bool out16 = p.o16 != nullptr && job.group == 0;  // uniform over the workgroup
    const bool out_bf = p.o16_dt == ISPA_BF16;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + g4 * 8 + hh * 4;
        f32x4 v = {o[qb][dt][g4 * 4 + 0] * inv, o[qb][dt][g4 * 4 + 1] * inv, o[qb][dt][g4 * 4 + 2] * inv,
                   o[qb][dt][g4 * 4 + 3] * inv};
        if (out16)
          *(u32x2*)((uint16_t*)p.o16 + base + d0) = out_bf ? (u32x2){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}
                                                           : (u32x2){pack_f16(v[0], v[1]), pack_f16(v[2], v[3])};
        else
          *(f32x4*)(job.o + base + d0) = v;
      }
    }
    if (hh == 0) job.lse[qrow * p.H + head] = l_tot > 0.0f ? (m[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
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

// V vectors of 4 elements per thread.  Per row: m = max_k LSE_k, e_k = exp(LSE_k - m)
// (0 for an empty part), LSE = m + ln sum_k e_k and weight_k = e_k / sum_k e_k, which
// is exp(LSE_k - LSE); every thread of the row forms the same weights.
template <int V>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int tpr = p.d / (4 * V);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / tpr;
  const int c = (int)(gid - row * tpr);
  if (row >= p.n_rows) return;
  float m = -INFINITY;
  for (int k = 0; k < p.n_parts; ++k) m = fmaxf(m, p.lse[k][row]);
  float tot = 0.0f;
  if (m != -INFINITY)
    for (int k = 0; k < p.n_parts; ++k) tot += exp2f((p.lse[k][row] - m) * kLog2e);  // exp2(-inf) = 0
  const float L = m != -INFINITY ? m + log2f(tot) * kLn2 : -INFINITY;
  const float inv = m != -INFINITY ? 1.0f / tot : 0.0f;
  // the first n_first parts on their own (a0 and delta refer to their merge)
  const int nf = p.n_first > 1 ? p.n_first : 1;
  float m0 = -INFINITY;
  for (int k = 0; k < nf; ++k) m0 = fmaxf(m0, p.lse[k][row]);
  float tot0 = 0.0f;
  if (m0 != -INFINITY)
    for (int k = 0; k < nf; ++k) tot0 += exp2f((p.lse[k][row] - m0) * kLog2e);
  const float inv0 = m0 != -INFINITY ? 1.0f / tot0 : 0.0f;
  const int64_t off = row * p.d + (int64_t)c * 4 * V;
  f32x4 acc[V], o0[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = o0[v] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.n_parts; ++k) {
    const float lk = p.lse[k][row];
    const float w = m != -INFINITY ? exp2f((lk - m) * kLog2e) * inv : 0.0f;
    // weight in the first group's merge (exactly 1 for a single finite first part)
    const float w0 = k < nf && m0 != -INFINITY ? exp2f((lk - m0) * kLog2e) * inv0 : 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const f32x4 ok = *(const f32x4*)(p.o[k] + off + 4 * v);
      if (k == 0 && nf == 1) o0[v] = ok;
      else if (k < nf) o0[v] += w0 * ok;
      acc[v] += w * ok;
    }
  }
  if (p.lse_full && c == 0) p.lse_full[row] = L;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t o = off + 4 * v;
    if (p.o_full) *(f32x4*)(p.o_full + o) = acc[v];
    if (p.o16) {
      const bool bf = p.o16_dt == ISPA_BF16;
      auto pk = [&](float x, float y) { return bf ? pack_bf16(x, y) : pack_f16(x, y); };
      *(u32x2*)((uint16_t*)p.o16 + o) = (u32x2){pk(acc[v][0], acc[v][1]), pk(acc[v][2], acc[v][3])};
    }
    const f32x4 dl = acc[v] - o0[v];
    if (p.out_dt == ISPA_F32) {
      if (p.a0) *(f32x4*)((float*)p.a0 + o) = o0[v];
      if (p.delta) *(f32x4*)((float*)p.delta + o) = dl;
    } else {
      const bool bf = p.out_dt == ISPA_BF16;
      auto pk = [&](float x, float y) { return bf ? pack_bf16(x, y) : pack_f16(x, y); };
      if (p.a0) *(u32x2*)((uint16_t*)p.a0 + o) = (u32x2){pk(o0[v][0], o0[v][1]), pk(o0[v][2], o0[v][3])};
      if (p.delta) *(u32x2*)((uint16_t*)p.delta + o) = (u32x2){pk(dl[0], dl[1]), pk(dl[2], dl[3])};
    }
  }
}

// out[i .. i+3] = in[i .. i+3] rounded to 16-bit out_dt (n a multiple of 4)
__global__ __launch_bounds__(256) void to16_kernel(const float* in, int64_t n, uint16_t* out, int out_dt) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4 v = *(const f32x4*)(in + i);
  const bool bf = out_dt == ISPA_BF16;
  auto pk = [&](float x, float y) { return bf ? pack_bf16(x, y) : pack_f16(x, y); };
  *(u32x2*)(out + i) = (u32x2){pk(v[0], v[1]), pk(v[2], v[3])};
}

}  // namespace

ispa_status launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.n_rows == 0) return ISPA_OK;
  const int V = p.d % 8 == 0 ? 2 : 1;
  const int64_t threads = p.n_rows * (p.d / (4 * V));
  const int64_t blocks = (threads + 255) / 256;
  if (V == 2)
    hipLaunchKernelGGL(merge_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return check_launch("merge_kernel");
}

int attn_block_q(ispa_dtype dt, int32_t d) {
  if (dt == ISPA_BF16 && d == 128) return a5::BQ;
  return kBQ;
}

SplitPlan plan_splits(int bq, int64_t n_q, int32_t H, const HostGroup* groups, int n_groups, int max_jobs) {
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
    // One key set.  A launch that already gives at least half the CUs a
    // workgroup is not split: the CUs a split would add run at the clock the
    // chip then falls to, and the parts cost a merge (measured on MI355X at
    // 4680 queries x 12 heads, 228 workgroups: 93,600 keys whole 2569-2587 us,
    // in the 10 pieces the model below picks 2655-2662 us; 187,200 keys
    // 4848-4877 against 4917-4957 us).  Otherwise the piece count s minimises
    // the launch's estimated time, (waves of workgroups over the CUs) x (key
    // tiles per piece + a fixed cost of about kFillTiles tiles per workgroup:
    // pipeline fill, output store and the extra merge part), the fixed cost
    // fitted to 1-, 2-, 3- and 4-piece timings of a 9360-key group.
    constexpr int64_t kCUs = 256, kFillTiles = 10, kMinTiles = 4;
    if (2 * wgs >= kCUs) return plan;
    const int64_t tiles = (shortest + kBK - 1) / kBK;
    int64_t s = 1, best = INT64_MAX;
    for (int64_t c = 1; c <= 16 && (c == 1 || tiles / c >= kMinTiles); ++c) {
      const int64_t cost = (wgs * c + kCUs - 1) / kCUs * ((tiles + c - 1) / c + kFillTiles);
      if (cost < best) {
        best = cost;
        s = c;
      }
    }
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
    if (total - 1 + s > max_jobs) s = std::max(1, max_jobs - (total - 1));
    total += s - 1;
    plan.n_splits[g] = s;
    plan.split_len[g] = s > 1 ? (((n + s - 1) / s + kBK - 1) / kBK) * kBK : n;
  }
  return plan;
}

bool dual_single_pass(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, const HostGroup* groups, int out_dt) {
  if (dt != ISPA_BF16 || d != 128 || (out_dt != ISPA_BF16 && out_dt != ISPA_F16) || n_q <= 0) return false;
  for (int g = 0; g < 2; ++g) {
    int runs = 0;  // the two-run tile addressing, per group
    for (int s = 0; s < groups[g].n_segs; ++s) runs += groups[g].segs[s].n > 0;
    if (runs > 2) return false;
  }
  // one workgroup per (query tile, head): use it when that fills most of the
  // 256 CUs; fewer pairs are better served by splitting the keys
  const int64_t units = (n_q + a5::BQ - 1) / a5::BQ * H;
  return units >= 192;
}

ispa_status run_dual_single_pass(int64_t n_q, int32_t H, float scale, const void* q, int64_t q_stride,
                                 const HostGroup* groups, void* a_loc, void* delta, int out_dt, float* lse_full,
                                 void* ws, hipStream_t stream) {
  AttnParams p{};
  p.q = q;
  p.q_stride = q_stride;
  p.n_q = n_q;
  p.H = H;
  p.n_qtiles = (int)((n_q + a5::BQ - 1) / a5::BQ);
  p.c = scale * kLog2e;
  for (int g = 0; g < 2; ++g) {
    p.n_segs[g] = groups[g].n_segs;
    for (int s = 0; s < groups[g].n_segs; ++s) {
      const ispa_seg& sg = groups[g].segs[s];
      p.segs[g][s] = AttnSeg{sg.k, sg.v, sg.n, sg.k_stride, sg.v_stride};
    }
  }
  p.n_jobs = 1;
  p.jobs[0] = AttnJob{0, 0, 0, groups[0].n_keys(), nullptr, nullptr};
  p.a_loc = a_loc;
  p.delta = delta;
  p.lse_full = lse_full;
  p.out_dt = out_dt;
  p.o_stash = (float*)ws;
  const int64_t blocks = (int64_t)p.n_qtiles * H;
  hipLaunchKernelGGL((attn_bf16_d128_kernel<true, true>), dim3((unsigned)blocks), dim3(a5::WAVES * 64), 0, stream,
                     p);
  return check_launch("attention kernel (single-pass dual form)");
}

size_t merged_workspace_bytes(int64_t n_q, int32_t H, int32_t d, const SplitPlan& plan, int n_groups) {
  size_t total = 0;
  for (int g = 0; g < n_groups; ++g)
    total += plan.n_splits[g] * (align256((size_t)n_q * H * d * 4) + align256((size_t)n_q * H * 4));
  return total;
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
                                void* ws, size_t ws_bytes, hipStream_t stream, void* o16_g0, int o16_dt,
                                const MergeOut* merge_all) {
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
  const SplitPlan plan = plan_splits(bq, n_q, H, groups, n_groups, merge_all ? 16 : kMaxJobs);
  if ((merge_all ? merged_workspace_bytes(n_q, H, d, plan, n_groups)
                 : split_workspace_bytes(n_q, H, d, plan, n_groups)) > ws_bytes) {
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
  if (merge_all) {
    // every group's pieces become parts of one merge
    MergeParams mp{};
    mp.d = d;
    mp.n_rows = n_q * H;
    mp.a0 = merge_all->a0;
    mp.delta = merge_all->delta;
    mp.out_dt = merge_all->out_dt;
    mp.lse_full = merge_all->lse_full;
    mp.n_first = plan.n_splits[0];
    for (int g = 0; g < n_groups; ++g) {
      const int64_t n = groups[g].n_keys();
      for (int s = 0; s < plan.n_splits[g]; ++s) {
        float* po = (float*)wsp;
        wsp += align256((size_t)n_q * H * d * 4);
        float* pl = (float*)wsp;
        wsp += align256((size_t)n_q * H * 4);
        const int64_t kb = std::min<int64_t>(n, s * plan.split_len[g]);
        const int64_t ke = std::min<int64_t>(n, (s + 1) * plan.split_len[g]);
        pend[nj++] = Pending{g, kb, ke, po, pl};
        mp.o[mp.n_parts] = po;
        mp.lse[mp.n_parts] = pl;
        ++mp.n_parts;
      }
    }
    merges[n_merges++] = mp;
  }
  for (int g = 0; g < n_groups && !merge_all; ++g) {
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
    if (g == 0 && o16_g0) {  // the 16-bit output replaces the fp32 one
      mp.o16 = o16_g0;
      mp.o16_dt = o16_dt;
      mp.o_full = nullptr;
    }
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
  bool two_runs = true;  // every job overlaps at most two segments
  for (int j = 0; j < nj; ++j) {
    p.jobs[j] = AttnJob{pend[j].g, 0, pend[j].kb, pend[j].ke, pend[j].o, pend[j].lse};
    int runs = 0;
    int64_t st = 0;
    for (int sg = 0; sg < p.n_segs[pend[j].g]; ++sg) {
      const int64_t n = p.segs[pend[j].g][sg].n;
      if (std::max(pend[j].kb, st) < std::min(pend[j].ke, st + n)) ++runs;
      st += n;
    }
    two_runs = two_runs && runs <= 2;
  }
  // an unsplit group 0 asked for as 16-bit rows: the d = 128 kernel writes them
  // from its epilogue; the other kernels write fp32 and to16_kernel rounds it
  const bool direct16 = o16_g0 && plan.n_splits[0] == 1 && dt == ISPA_BF16 && d == 128;
  if (direct16) {
    p.o16 = o16_g0;
    p.o16_dt = o16_dt;
  }
  if (dt == ISPA_BF16) {
    const int64_t blocks = (int64_t)p.n_qtiles * H * nj;
    if (d == 128 && two_runs)
      hipLaunchKernelGGL(attn_bf16_d128_kernel<true>, dim3((unsigned)blocks), dim3(a5::WAVES * 64), 0, stream, p);
    else if (d == 128)
      hipLaunchKernelGGL(attn_bf16_d128_kernel<false>, dim3((unsigned)blocks), dim3(a5::WAVES * 64), 0, stream, p);
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
  if (o16_g0 && plan.n_splits[0] == 1 && !direct16) {  // unsplit group 0: its fp32 output, rounded
    const int64_t n = n_q * H * d;       // d is a multiple of 4
    hipLaunchKernelGGL(to16_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, o_out[0], n,
                       (uint16_t*)o16_g0, o16_dt);
    return check_launch("to16_kernel");
  }
  return ISPA_OK;
}

}  // namespace ispa
