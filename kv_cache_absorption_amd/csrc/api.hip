// C ABI of libispa: argument validation, workspace sizing and dispatch.
// Nothing here allocates device memory; every kernel runs on the caller's
// stream.
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "attn.hpp"
#include "attn8.hpp"
#include "gemm.hpp"
#include "gram.hpp"
#include "internal.hpp"

namespace ispa {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

ispa_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return ISPA_ERR_HIP;
  }
  return ISPA_OK;
}

namespace {

ispa_status fail(ispa_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// validate a key group; bf16 path needs 16-byte aligned rows
ispa_status check_group(const char* name, ispa_dtype dt, int32_t H, int32_t d, const ispa_seg* segs,
                        int32_t n) {
  if (n < 0 || n > ISPA_MAX_SEGS)
    return fail(ISPA_ERR_INVALID_ARG, std::string(name) + ": segment count out of range");
  if (n > 0 && !segs) return fail(ISPA_ERR_INVALID_ARG, std::string(name) + ": null segment table");
  const int64_t row = (int64_t)H * d;
  const size_t al = dt == ISPA_BF16 ? 16 : 4;
  for (int i = 0; i < n; ++i) {
    const ispa_seg& s = segs[i];
    if (s.n < 0) return fail(ISPA_ERR_INVALID_ARG, std::string(name) + ": negative segment length");
    if (s.n == 0) continue;
    if (!s.k || !s.v) return fail(ISPA_ERR_INVALID_ARG, std::string(name) + ": null k/v pointer");
    if (s.k_stride < row || s.v_stride < row)
      return fail(ISPA_ERR_INVALID_ARG, std::string(name) + ": row stride smaller than H*d");
    if (!aligned(s.k, al) || !aligned(s.v, al) || (dt == ISPA_BF16 && (s.k_stride % 8 || s.v_stride % 8)))
      return fail(ISPA_ERR_INVALID_ARG, std::string(name) + ": k/v rows must be 16-byte aligned");
  }
  return ISPA_OK;
}

ispa_status check_attn_common(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, const void* q,
                              int64_t q_stride) {
  if (dt != ISPA_BF16 && dt != ISPA_F32) return fail(ISPA_ERR_UNSUPPORTED, "attention dtype must be BF16 or F32");
  if (d != 64 && d != 128) return fail(ISPA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (n_q < 0 || H < 1) return fail(ISPA_ERR_INVALID_ARG, "n_q must be >= 0 and H >= 1");
  if (n_q > 0 && !q) return fail(ISPA_ERR_INVALID_ARG, "null q");
  if (q_stride < (int64_t)H * d) return fail(ISPA_ERR_INVALID_ARG, "q_stride smaller than H*d");
  if (dt == ISPA_BF16 && (!aligned(q, 16) || q_stride % 8))
    return fail(ISPA_ERR_INVALID_ARG, "q rows must be 16-byte aligned");
  if (dt == ISPA_F32 && !aligned(q, 4)) return fail(ISPA_ERR_INVALID_ARG, "q must be 4-byte aligned");
  return ISPA_OK;
}


}  // namespace

// ---------------------------------------------------------------- W8A8 product without allocation
// Scratch for ispa_w8a8_linear_noalloc: the activation codes and row scales
// of one call, in a fixed device array instead of a caller workspace.  Host
// code never uses the array's name as an address: the per-device address
// comes from hipGetSymbolAddress on the first call on that device.
static __device__ __align__(256) unsigned char scratch[ISPA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of this device's copy of `scratch` (looked up once per device).
ispa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ISPA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(ISPA_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ISPA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ISPA_OK;
}

}  // namespace
}  // namespace ispa

using namespace ispa;

extern "C" {

int32_t ispa_version(void) { return ISPA_VERSION; }

const char* ispa_status_str(ispa_status s) {
  switch (s) {
    case ISPA_OK: return "ok";
    case ISPA_ERR_INVALID_ARG: return "invalid argument";
    case ISPA_ERR_UNSUPPORTED: return "unsupported";
    case ISPA_ERR_WORKSPACE: return "workspace too small";
    case ISPA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* ispa_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------- dual_attn
size_t ispa_dual_attn_workspace_bytes(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, const ispa_seg* loc,
                                      int32_t n_loc, const ispa_seg* hist, int32_t n_hist) {
  if (n_q <= 0 || H < 1 || n_loc < 0 || n_hist < 0 || n_loc > ISPA_MAX_SEGS || n_hist > ISPA_MAX_SEGS)
    return 0;
  HostGroup g[2] = {{loc, n_loc}, {hist, n_hist}};
  const SplitPlan plan = plan_splits(attn_block_q(dt, d), n_q, H, g, 2);
  return split_workspace_bytes(n_q, H, d, plan, 2);
}

ispa_status ispa_dual_attn(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale, const void* q,
                           int64_t q_stride, const ispa_seg* loc, int32_t n_loc, const ispa_seg* hist,
                           int32_t n_hist, float* o_loc, float* lse_loc, float* o_hist, float* lse_hist,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  ispa_status st = check_attn_common(dt, n_q, H, d, q, q_stride);
  if (st) return st;
  if ((st = check_group("loc", dt, H, d, loc, n_loc))) return st;
  if ((st = check_group("hist", dt, H, d, hist, n_hist))) return st;
  if (n_q > 0 && (!o_loc || !lse_loc || !o_hist || !lse_hist))
    return fail(ISPA_ERR_INVALID_ARG, "null output pointer");
  if (!aligned(o_loc, 16) || !aligned(o_hist, 16)) return fail(ISPA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(ISPA_ERR_INVALID_ARG, "scale must be finite");
  const size_t need = ispa_dual_attn_workspace_bytes(dt, n_q, H, d, loc, n_loc, hist, n_hist);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(ISPA_ERR_WORKSPACE, "dual_attn workspace too small or misaligned");
  if (n_q == 0) return ISPA_OK;
  HostGroup g[2] = {{loc, n_loc}, {hist, n_hist}};
  float* o[2] = {o_loc, o_hist};
  float* l[2] = {lse_loc, lse_hist};
  return run_group_attention(dt, n_q, H, d, scale, q, q_stride, g, 2, o, l, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- dual_attn_merge
size_t ispa_dual_attn_merge_workspace_bytes(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d,
                                            const ispa_seg* loc, int32_t n_loc, const ispa_seg* hist,
                                            int32_t n_hist) {
  if (n_q <= 0 || H < 1 || n_loc < 0 || n_hist < 0 || n_loc > ISPA_MAX_SEGS || n_hist > ISPA_MAX_SEGS)
    return 0;
  HostGroup g[2] = {{loc, n_loc}, {hist, n_hist}};
  const SplitPlan plan = plan_splits(attn_block_q(dt, d), n_q, H, g, 2, 16);
  return merged_workspace_bytes(n_q, H, d, plan, 2);
}

ispa_status ispa_dual_attn_merge(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale, const void* q,
                                 int64_t q_stride, const ispa_seg* loc, int32_t n_loc, const ispa_seg* hist,
                                 int32_t n_hist, void* a_loc, void* delta, ispa_dtype out_dt, float* lse_full,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  ispa_status st = check_attn_common(dt, n_q, H, d, q, q_stride);
  if (st) return st;
  if ((st = check_group("loc", dt, H, d, loc, n_loc))) return st;
  if ((st = check_group("hist", dt, H, d, hist, n_hist))) return st;
  if (!valid_dtype(out_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad out_dt");
  if (n_q > 0 && (!a_loc || !delta)) return fail(ISPA_ERR_INVALID_ARG, "null output pointer");
  const size_t oal = out_dt == ISPA_F32 ? 16 : 8;
  if (!aligned(a_loc, oal) || !aligned(delta, oal))
    return fail(ISPA_ERR_INVALID_ARG, "a_loc and delta must be 16-byte (fp32) or 8-byte (16-bit) aligned");
  if (!std::isfinite(scale)) return fail(ISPA_ERR_INVALID_ARG, "scale must be finite");
  const size_t need = ispa_dual_attn_merge_workspace_bytes(dt, n_q, H, d, loc, n_loc, hist, n_hist);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(ISPA_ERR_WORKSPACE, "dual_attn_merge workspace too small or misaligned");
  if (n_q == 0) return ISPA_OK;
  HostGroup g[2] = {{loc, n_loc}, {hist, n_hist}};
  if (dual_single_pass(dt, n_q, H, d, g, out_dt))
    return run_dual_single_pass(n_q, H, scale, q, q_stride, g, a_loc, delta, out_dt, lse_full, ws, stream);
  float* o[2] = {nullptr, nullptr};
  float* l[2] = {nullptr, nullptr};
  const MergeOut mo{a_loc, delta, out_dt, lse_full};
  return run_group_attention(dt, n_q, H, d, scale, q, q_stride, g, 2, o, l, ws, ws_bytes, stream, nullptr,
                             ISPA_BF16, &mo);
}

// ---------------------------------------------------------------- lse_merge
ispa_status ispa_lse_merge(int32_t n_parts, const float* const* o_parts, const float* const* lse_parts,
                           int64_t n_q, int32_t H, int32_t d, float* o_full, float* lse_full, void* a0_out,
                           void* delta_out, ispa_dtype out_dt, hipStream_t stream) {
  if (n_parts < 1 || n_parts > 16) return fail(ISPA_ERR_INVALID_ARG, "n_parts must be 1..16");
  if (!o_parts || !lse_parts) return fail(ISPA_ERR_INVALID_ARG, "null part table");
  if (n_q < 0 || H < 1 || d < 4 || d % 4) return fail(ISPA_ERR_INVALID_ARG, "bad shape (d must be a multiple of 4)");
  if (!valid_dtype(out_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad out_dt");
  for (int i = 0; i < n_parts; ++i) {
    if (n_q > 0 && (!o_parts[i] || !lse_parts[i])) return fail(ISPA_ERR_INVALID_ARG, "null part pointer");
    if (!aligned(o_parts[i], 16)) return fail(ISPA_ERR_INVALID_ARG, "parts must be 16-byte aligned");
  }
  if (!aligned(o_full, 16) || !aligned(a0_out, 16) || !aligned(delta_out, 16))
    return fail(ISPA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  MergeParams p{};
  p.n_parts = n_parts;
  p.d = d;
  p.n_rows = n_q * H;
  for (int i = 0; i < n_parts; ++i) {
    p.o[i] = o_parts[i];
    p.lse[i] = lse_parts[i];
  }
  p.o_full = o_full;
  p.lse_full = lse_full;
  p.a0 = a0_out;
  p.delta = delta_out;
  p.out_dt = out_dt;
  return launch_merge(p, stream);
}

// ---------------------------------------------------------------- accum_stats
size_t ispa_accum_stats_workspace_bytes(ispa_dtype a_dt, int64_t n, int32_t D) {
  if (n <= 0 || D <= 0) return 0;
  if (a_dt == ISPA_F32) return align256((size_t)n * D * 4) + align256(64 * 8);
  const int64_t np = (n + kNtBK - 1) / kNtBK * kNtBK;
  const size_t rblocks = (size_t)((D + kNtBM - 1) / kNtBM) * (size_t)((np + 127) / 128);
  const int64_t split = nt_stats_split(D, np);
  const size_t part = split > 1 ? align256((size_t)split * 2 * D * D * 4) : 0;
  return align256((size_t)D * D * 2) + 2 * align256((size_t)D * np * 2) + align256(rblocks * 8) + part;
}

ispa_status ispa_accum_stats(ispa_dtype a_dt, ispa_dtype w_dt, int64_t n, int32_t D, const void* a_loc,
                             const void* delta_a, const void* w, float* G, float* C, double* r2, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(a_dt) || !valid_dtype(w_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad dtype");
  if (a_dt == ISPA_F32 && w_dt != ISPA_F32) return fail(ISPA_ERR_UNSUPPORTED, "F32 statistics need F32 W");
  if (a_dt != ISPA_F32 && w_dt == ISPA_F32) return fail(ISPA_ERR_UNSUPPORTED, "16-bit statistics need 16-bit W");
  if (D <= 0 || D % 64) return fail(ISPA_ERR_INVALID_ARG, "D must be a positive multiple of 64");
  if (n < 0) return fail(ISPA_ERR_INVALID_ARG, "n must be >= 0");
  if (!G || !C || !r2 || !w) return fail(ISPA_ERR_INVALID_ARG, "null G/C/r2/w");
  if (n > 0 && (!a_loc || !delta_a)) return fail(ISPA_ERR_INVALID_ARG, "null activations");
  const size_t al = a_dt == ISPA_F32 ? 4 : 16;
  if (!aligned(a_loc, al) || !aligned(delta_a, al) || !aligned(w, a_dt == ISPA_F32 ? 4 : 8))
    return fail(ISPA_ERR_INVALID_ARG, "misaligned activations or W");
  if (!aligned(G, 16) || !aligned(C, 16)) return fail(ISPA_ERR_INVALID_ARG, "G and C must be 16-byte aligned");
  if (n == 0) return ISPA_OK;
  const size_t need = ispa_accum_stats_workspace_bytes(a_dt, n, D);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "accum_stats workspace too small or misaligned");
  if (a_dt == ISPA_F32)
    return launch_stats_f32(n, D, (const float*)a_loc, (const float*)delta_a, (const float*)w, G, C, r2, ws,
                            stream);
  // Workspace: W^T (in the operand type), A_loc^T and R^T with the
  // token dimension zero-padded to a multiple of the GEMM's K stage, per-workgroup
  // ||R||^2, and (when the token range is split) the partial G and C sums.
  const int64_t np = (n + kNtBK - 1) / kNtBK * kNtBK;
  char* wp = (char*)ws;
  uint16_t* Wt = (uint16_t*)wp;
  wp += align256((size_t)D * D * 2);
  uint16_t* At = (uint16_t*)wp;
  wp += align256((size_t)D * np * 2);
  uint16_t* Rt = (uint16_t*)wp;
  wp += align256((size_t)D * np * 2);
  double* partials = (double*)wp;
  const size_t rblocks_bytes = (size_t)((D + kNtBM - 1) / kNtBM) * (size_t)((np + 127) / 128) * 8;
  ispa_status st;
  {
    // W^T (converted to the operand type) and A_loc^T in one launch
    const Transpose16 tj[2] = {{w, Wt, D, D, D, D, D, w_dt, a_dt}, {a_loc, At, D, n, D, np, np, a_dt, a_dt}};
    if ((st = launch_transpose16(tj, 2, stream))) return st;
  }
  // R^T = W^T dA^T, stored with zero padding, and per-workgroup ||R||^2
  NtGemmParams r{};
  r.M = D;
  r.N = np;
  r.K = D;
  r.x = Wt;
  r.ldx = D;
  r.y = delta_a;
  r.ldy = D;
  r.y_rows = n;
  r.epi = kNtStoreT;
  r.out = Rt;
  r.ld_out = np;
  r.n_valid = n;
  r.bn = 128;  // narrower tiles: R has no K split, so fill the CUs with tiles
  r.tiles_m = (D + kNtBM - 1) / kNtBM;
  r.tiles_n = (int)((np + r.bn - 1) / r.bn);
  r.ksplit = 1;
  r.kchunk = D;
  r.sq_partials = partials;
  int nblk = 0;
  if ((st = launch_nt_gemm(r, a_dt, stream, &nblk))) return st;
  // G += A^T A (upper-triangle tiles) and C += A^T R (all tiles) in one launch
  NtGemmParams g{};
  g.M = D;
  g.N = D;
  g.K = np;
  g.x = At;
  g.ldx = np;
  g.y = At;
  g.y2 = Rt;
  g.ldy = np;
  g.y_rows = D;
  g.epi = kNtAccum;
  g.out = G;
  g.out2 = C;
  g.ld_out = D;
  g.bn = kNtBM;
  g.tiles_m = g.tiles_n = (D + kNtBM - 1) / kNtBM;
  g.tri = 1;
  g.two_kinds = 1;
  const int64_t stages = np / kNtBK;
  g.ksplit = (int)nt_stats_split(D, np);
  g.kchunk = (stages + g.ksplit - 1) / g.ksplit * kNtBK;
  g.part = g.ksplit > 1 ? (float*)(wp + align256(rblocks_bytes)) : nullptr;
  if ((st = launch_nt_gemm(g, a_dt, stream, nullptr))) return st;
  return launch_nt_split_reduce(g, partials, nblk, r2, stream);
}

// ---------------------------------------------------------------- grouped statistics
size_t ispa_gram_state_bytes(int32_t D) {
  if (D <= 0 || D % 64) return 0;
  return (size_t)gram_splits(D) * 3 * (size_t)D * D * 4;
}

ispa_status ispa_accum_gram(ispa_dtype a_dt, int64_t n, int32_t D, const void* a_loc, const void* delta_a,
                            void* state, hipStream_t stream) {
  if (a_dt != ISPA_BF16 && a_dt != ISPA_F16) return fail(ISPA_ERR_UNSUPPORTED, "activations must be BF16 or F16");
  if (D <= 0 || D % 64) return fail(ISPA_ERR_INVALID_ARG, "D must be a positive multiple of 64");
  if (n < 0) return fail(ISPA_ERR_INVALID_ARG, "n must be >= 0");
  if (!state) return fail(ISPA_ERR_INVALID_ARG, "null state");
  if (n > 0 && (!a_loc || !delta_a)) return fail(ISPA_ERR_INVALID_ARG, "null activations");
  if (!aligned(a_loc, 16) || !aligned(delta_a, 16) || !aligned(state, 16))
    return fail(ISPA_ERR_INVALID_ARG, "activations and state must be 16-byte aligned");
  if (n == 0) return ISPA_OK;
  const int S = gram_splits(D);
  const int64_t stages = (n + 31) / 32;
  const int64_t kchunk = (stages + S - 1) / S * 32;
  if (kchunk * D * 2 >= ((int64_t)1 << 31))
    return fail(ISPA_ERR_UNSUPPORTED, "too many token rows in one call for this width: split the call");
  SyrkParams p{};
  p.a = a_loc;
  p.b = delta_a;
  p.n = n;
  p.lda = D;
  p.D = D;
  p.nbh = (D + 255) / 256;
  p.n_tiles = p.nbh * (2 * p.nbh + 1);  // upper triangle of the 2 nbh x 2 nbh block grid
  p.ksplit = S;
  p.kchunk = kchunk;
  p.state = (float*)state;
  p.split_stride = 3 * (int64_t)D * D;
  return launch_syrk(p, a_dt, stream);
}

size_t ispa_gram_finalize_workspace_bytes(int32_t D) {
  if (D <= 0 || D % 64) return 0;
  return gram_finalize_ws_bytes(D);
}

ispa_status ispa_gram_finalize(int32_t n_layers, int32_t D, const void* state, int64_t state_stride, const void* w,
                               ispa_dtype w_dt, int64_t w_stride, float* G, float* C, double* r2,
                               int64_t mat_stride, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_layers < 1) return fail(ISPA_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (D <= 0 || D % 64) return fail(ISPA_ERR_INVALID_ARG, "D must be a positive multiple of 64");
  if (w_dt != ISPA_BF16) return fail(ISPA_ERR_UNSUPPORTED, "W must be BF16");
  if (!state || !w || !G || !C || !r2) return fail(ISPA_ERR_INVALID_ARG, "null pointer");
  const int64_t dd = (int64_t)D * D;
  const int64_t st_floats = (int64_t)(ispa_gram_state_bytes(D) / 4);
  if (state_stride < st_floats || w_stride < dd || mat_stride < dd)
    return fail(ISPA_ERR_INVALID_ARG, "state_stride, w_stride or mat_stride too small");
  if (!aligned(state, 16) || !aligned(G, 16) || !aligned(C, 16) || !aligned(w, 16) || state_stride % 4 ||
      w_stride % 8 || mat_stride % 4)
    return fail(ISPA_ERR_INVALID_ARG, "state, W, G and C (and their layer strides) must be 16-byte aligned");
  const size_t need = ispa_gram_finalize_workspace_bytes(D);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "gram_finalize workspace too small or misaligned");
  const int S = gram_splits(D);
  for (int l = 0; l < n_layers; ++l) {
    const ispa_status st = launch_gram_finalize(D, (const float*)state + l * state_stride, 3 * dd, S,
                                                (const uint16_t*)w + l * w_stride, G + l * mat_stride,
                                                C + l * mat_stride, r2 + l, ws, stream);
    if (st) return st;
  }
  return ISPA_OK;
}

// ---------------------------------------------------------------- solve_dw
size_t ispa_solve_dw_workspace_bytes(int32_t n_layers, int32_t D) {
  if (n_layers <= 0 || D <= 0) return 0;
  return solve_ws_bytes(n_layers, D);
}

ispa_status ispa_solve_dw(int32_t n_layers, int32_t D, const float* G, const float* C, const double* r2,
                          int64_t mat_stride, double lambda_abs, double lambda_rel, float* dW, double* eps,
                          int32_t* info, const void* w, ispa_dtype w_dt, void* w_eff, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  if (n_layers < 1) return fail(ISPA_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (D <= 0 || D % 64) return fail(ISPA_ERR_INVALID_ARG, "D must be a positive multiple of 64");
  if (mat_stride < (int64_t)D * D) return fail(ISPA_ERR_INVALID_ARG, "mat_stride smaller than D*D");
  if (!G || !C || !r2 || !dW || !eps || !info) return fail(ISPA_ERR_INVALID_ARG, "null pointer");
  if ((w == nullptr) != (w_eff == nullptr)) return fail(ISPA_ERR_INVALID_ARG, "w and w_eff must both be set or null");
  if (w && !valid_dtype(w_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad w_dt");
  if (!std::isfinite(lambda_abs) || !std::isfinite(lambda_rel) || lambda_abs < 0 || lambda_rel < 0)
    return fail(ISPA_ERR_INVALID_ARG, "lambda must be finite and >= 0");
  const size_t need = ispa_solve_dw_workspace_bytes(n_layers, D);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "solve_dw workspace too small or misaligned");
  return run_solve(n_layers, D, G, C, r2, mat_stride, lambda_abs, lambda_rel, dW, eps, info, w, w_dt, w_eff,
                   ws, stream);
}

// ---------------------------------------------------------------- select
ispa_status ispa_select_layers(int32_t n_layers, int32_t K, const double* eps, int32_t* selected,
                               uint8_t* is_local, int32_t* status, hipStream_t stream) {
  if (n_layers < 1 || n_layers > 1024) return fail(ISPA_ERR_INVALID_ARG, "n_layers must be 1..1024");
  if (K < 0 || K > n_layers) return fail(ISPA_ERR_INVALID_ARG, "K must be in 0..n_layers");
  if (!eps || !is_local || !status || (K > 0 && !selected)) return fail(ISPA_ERR_INVALID_ARG, "null pointer");
  return launch_select(n_layers, K, eps, selected, is_local, status, stream);
}

// ---------------------------------------------------------------- local_attn_proj
size_t ispa_local_attn_proj_workspace_bytes(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d,
                                            const ispa_seg* segs, int32_t n_segs) {
  if (n_q <= 0 || H < 1 || n_segs < 0 || n_segs > ISPA_MAX_SEGS) return 0;
  HostGroup g[1] = {{segs, n_segs}};
  const SplitPlan plan = plan_splits(attn_block_q(dt, d), n_q, H, g, 1);
  const size_t D = (size_t)H * d;
  // fp32 attention output and LSE, its 16-bit copy and W^T for the projection GEMM, split parts
  const size_t proj = dt == ISPA_F32 ? 0 : align256((size_t)n_q * D * 2) + align256(D * D * 2);
  return align256((size_t)n_q * D * 4) + align256((size_t)n_q * H * 4) + proj +
         split_workspace_bytes(n_q, H, d, plan, 1);
}

// Width of the projection GEMM's tiles: the one whose last wave of workgroups
// leaves the fewest CU-tiles idle (256 CUs, one workgroup each).
static int proj_tile_n(int64_t n_q, int32_t D) {
  const int64_t tm = (n_q + kNtBM - 1) / kNtBM;
  int best = 128;
  int64_t best_cost = -1;
  for (int bn : {256, 128}) {
    const int64_t tiles = tm * ((D + bn - 1) / bn);
    const int64_t cost = (tiles + 255) / 256 * bn;  // waves x tile width
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = bn;
    }
  }
  return best;
}

ispa_status ispa_local_attn_proj(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale, const void* q,
                                 int64_t q_stride, const ispa_seg* segs, int32_t n_segs, const void* w_proj,
                                 ispa_dtype w_dt, void* y, ispa_dtype y_dt, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  ispa_status st = check_attn_common(dt, n_q, H, d, q, q_stride);
  if (st) return st;
  if (n_segs < 1) return fail(ISPA_ERR_INVALID_ARG, "n_segs must be >= 1");
  if ((st = check_group("segs", dt, H, d, segs, n_segs))) return st;
  if (!valid_dtype(w_dt) || !valid_dtype(y_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad w_dt or y_dt");
  if (dt == ISPA_F32 && w_dt != ISPA_F32) return fail(ISPA_ERR_UNSUPPORTED, "F32 attention needs F32 W");
  if (dt == ISPA_BF16 && w_dt == ISPA_F32) return fail(ISPA_ERR_UNSUPPORTED, "BF16 attention needs 16-bit W");
  if (!w_proj || (n_q > 0 && !y)) return fail(ISPA_ERR_INVALID_ARG, "null w_proj or y");
  if (!aligned(w_proj, 4) || !aligned(y, 4)) return fail(ISPA_ERR_INVALID_ARG, "misaligned w_proj or y");
  if (!std::isfinite(scale)) return fail(ISPA_ERR_INVALID_ARG, "scale must be finite");
  if (n_q == 0) return ISPA_OK;
  const size_t need = ispa_local_attn_proj_workspace_bytes(dt, n_q, H, d, segs, n_segs);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "local_attn_proj workspace too small or misaligned");
  const int32_t D = H * d;
  float* O = (float*)ws;
  float* lse = (float*)((char*)ws + align256((size_t)n_q * D * 4));
  char* rest = (char*)lse + align256((size_t)n_q * H * 4);
  uint16_t* O16 = nullptr;
  uint16_t* Wt = nullptr;
  if (dt != ISPA_F32) {
    O16 = (uint16_t*)rest;
    rest += align256((size_t)n_q * D * 2);
    Wt = (uint16_t*)rest;
    rest += align256((size_t)D * D * 2);
  }
  // The NT GEMM stores 4 consecutive outputs per lane and reads W in 8-byte pieces.
  const bool nt = dt != ISPA_F32 && aligned(y, y_dt == ISPA_F32 ? 16 : 8) && aligned(w_proj, 8);
  HostGroup g[1] = {{segs, n_segs}};
  float* oo[1] = {O};
  float* ll[1] = {lse};
  st = run_group_attention(dt, n_q, H, d, scale, q, q_stride, g, 1, oo, ll, rest,
                           ws_bytes - (size_t)(rest - (char*)ws), stream, nt ? O16 : nullptr, ISPA_BF16);
  if (st) return st;
  if (dt == ISPA_F32) return launch_proj_f32(n_q, D, O, (const float*)w_proj, y, y_dt, stream);
  if (nt) {
    // y = O W: W^T (bf16) once, then the K-contiguous GEMM over the bf16 attention output
    if ((st = launch_transpose16(w_proj, D, D, D, Wt, D, D, w_dt, ISPA_BF16, stream))) return st;
    NtGemmParams p{};
    p.M = n_q;
    p.N = D;
    p.K = D;
    p.x = O16;
    p.ldx = D;
    p.y = Wt;
    p.ldy = D;
    p.y_rows = D;
    p.epi = kNtStore;
    p.out = y;
    p.out_dt = y_dt;
    p.ld_out = D;
    p.bn = proj_tile_n(n_q, D);
    p.tiles_m = (int)((n_q + kNtBM - 1) / kNtBM);
    p.tiles_n = (int)((D + p.bn - 1) / p.bn);
    p.ksplit = 1;
    p.kchunk = D;
    return launch_nt_gemm(p, ISPA_BF16, stream, nullptr);
  }
  GemmParams p{};
  p.M = n_q;
  p.N = D;
  p.K = D;
  p.x = GemmOperand{O, D, ISPA_F32, kDirect};
  p.y = GemmOperand{w_proj, D, w_dt, kTrans};
  p.epi = kStore;
  p.out_dt = y_dt;
  p.out = y;
  p.ld_out = D;
  p.tiles_m = (int)((n_q + kGemmBM - 1) / kGemmBM);
  p.tiles_n = (int)((D + kGemmBN - 1) / kGemmBN);
  p.ksplit = 1;
  p.kchunk = (D + kGemmBK - 1) / kGemmBK * kGemmBK;
  return launch_gemm(p, ISPA_BF16, stream, nullptr);
}

// ---------------------------------------------------------------- W8A8 projection
// The fp8 product of quantised rows (codes xq, scales sx) with the quantised
// weight: the NT GEMM on the fp8 matrix core, dequantised in its store.
static ispa_status run_w8a8_gemm(int64_t n, int32_t d_in, int32_t d_out, const uint8_t* xq, const float* sx,
                                 const uint8_t* w_codes, const float* w_scales, void* y, ispa_dtype y_dt,
                                 hipStream_t stream) {
  NtGemmParams p{};
  p.M = n;
  p.N = d_out;
  p.K = d_in;
  p.x = xq;
  p.ldx = d_in;
  p.y = w_codes;
  p.ldy = d_in;
  p.y_rows = d_out;
  p.epi = kNtStoreScaled;
  p.sx = sx;
  p.sy = w_scales;
  p.out = y;
  p.out_dt = y_dt;
  p.ld_out = d_out;
  p.bn = proj_tile_n(n, d_out);
  p.tiles_m = (int)((n + kNtBM - 1) / kNtBM);
  p.tiles_n = (int)((d_out + p.bn - 1) / p.bn);
  p.ksplit = 1;
  p.kchunk = d_in;
  return launch_nt_gemm(p, kMtE4M3, stream, nullptr);
}

size_t ispa_quantize_w_fp8_workspace_bytes(int32_t d_in, int32_t d_out) {
  if (d_in <= 0 || d_out <= 0) return 0;
  return align256((size_t)d_in * d_out * 2);  // W^T in its 16-bit type
}

ispa_status ispa_quantize_w_fp8(ispa_dtype w_dt, int32_t d_in, int32_t d_out, const void* w, uint8_t* w_codes,
                                float* w_scales, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (w_dt != ISPA_BF16 && w_dt != ISPA_F16) return fail(ISPA_ERR_UNSUPPORTED, "W must be BF16 or F16");
  if (d_in <= 0 || d_out <= 0 || d_in % 4 || d_out % 4)
    return fail(ISPA_ERR_INVALID_ARG, "d_in and d_out must be positive multiples of 4");
  if (!w || !w_codes || !w_scales) return fail(ISPA_ERR_INVALID_ARG, "null w, w_codes or w_scales");
  if (!aligned(w, 8) || !aligned(w_codes, 4) || !aligned(w_scales, 4))
    return fail(ISPA_ERR_INVALID_ARG, "misaligned w, w_codes or w_scales");
  const size_t need = ispa_quantize_w_fp8_workspace_bytes(d_in, d_out);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "quantize_w_fp8 workspace too small or misaligned");
  // W^T [d_out][d_in] (an output column per row), then per-row codes
  const Transpose16 t{w, ws, d_out, d_in, d_out, d_in, d_in, w_dt, w_dt};
  ispa_status st = launch_transpose16(&t, 1, stream);
  if (st) return st;
  return launch_quant_rows_e4m3(ws, w_dt, d_in, d_out, d_in, w_codes, d_in, w_scales, stream);
}

size_t ispa_w8a8_linear_workspace_bytes(int64_t n, int32_t d_in) {
  if (n <= 0 || d_in <= 0) return 0;
  return align256((size_t)n * d_in) + align256((size_t)n * 4);  // activation codes and scales
}

static ispa_status check_w8a8(int32_t d_in, int32_t d_out, const uint8_t* w_codes, const float* w_scales, void* y,
                              ispa_dtype y_dt, bool any_rows) {
  if (!valid_dtype(y_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad y_dt");
  if (d_in <= 0 || d_in % 64 || d_out <= 0 || d_out % 4)
    return fail(ISPA_ERR_INVALID_ARG, "d_in must be a positive multiple of 64 and d_out of 4");
  if (!w_codes || !w_scales || (any_rows && !y)) return fail(ISPA_ERR_INVALID_ARG, "null w_codes, w_scales or y");
  if (!aligned(w_codes, 16) || !aligned(w_scales, 16) || !aligned(y, y_dt == ISPA_F32 ? 16 : 8))
    return fail(ISPA_ERR_INVALID_ARG, "misaligned w_codes, w_scales or y");
  return ISPA_OK;
}

ispa_status ispa_w8a8_linear(ispa_dtype x_dt, int64_t n, int32_t d_in, int32_t d_out, const void* x, int64_t ld_x,
                             const uint8_t* w_codes, const float* w_scales, void* y, ispa_dtype y_dt, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(x_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad x_dt");
  if (n < 0) return fail(ISPA_ERR_INVALID_ARG, "n must be >= 0");
  ispa_status st = check_w8a8(d_in, d_out, w_codes, w_scales, y, y_dt, n > 0);
  if (st) return st;
  if (ld_x < d_in || ld_x % 4) return fail(ISPA_ERR_INVALID_ARG, "ld_x must be >= d_in and a multiple of 4");
  if (n > 0 && !x) return fail(ISPA_ERR_INVALID_ARG, "null x");
  if (!aligned(x, x_dt == ISPA_F32 ? 16 : 8)) return fail(ISPA_ERR_INVALID_ARG, "misaligned x");
  if (n == 0) return ISPA_OK;
  const size_t need = ispa_w8a8_linear_workspace_bytes(n, d_in);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "w8a8_linear workspace too small or misaligned");
  uint8_t* xq = (uint8_t*)ws;
  float* sx = (float*)((char*)ws + align256((size_t)n * d_in));
  if ((st = launch_quant_rows_e4m3(x, x_dt, ld_x, n, d_in, xq, d_in, sx, stream))) return st;
  return run_w8a8_gemm(n, d_in, d_out, xq, sx, w_codes, w_scales, y, y_dt, stream);
}

ispa_status ispa_w8a8_linear_noalloc(ispa_dtype x_dt, int64_t n, int32_t d_in, int32_t d_out, const void* x,
                                     int64_t ld_x, const uint8_t* w_codes, const float* w_scales, void* y,
                                     ispa_dtype y_dt, hipStream_t stream) {
  if (!valid_dtype(x_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad x_dt");
  if (n < 0) return fail(ISPA_ERR_INVALID_ARG, "n must be >= 0");
  ispa_status st = check_w8a8(d_in, d_out, w_codes, w_scales, y, y_dt, n > 0);
  if (st) return st;
  if (ld_x < d_in || ld_x % 4) return fail(ISPA_ERR_INVALID_ARG, "ld_x must be >= d_in and a multiple of 4");
  if (n > 0 && !x) return fail(ISPA_ERR_INVALID_ARG, "null x");
  if (!aligned(x, x_dt == ISPA_F32 ? 16 : 8)) return fail(ISPA_ERR_INVALID_ARG, "misaligned x");
  if (n == 0) return ISPA_OK;
  if (ispa_w8a8_linear_workspace_bytes(n, d_in) > (size_t)ISPA_NOALLOC_SCRATCH_BYTES)
    return fail(ISPA_ERR_INVALID_ARG, "n * d_in + 4 n (each rounded up to 256) exceeds the fixed scratch of "
                                      "ISPA_NOALLOC_SCRATCH_BYTES");
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  // the quantiser writes every code and scale the product reads: nothing to clear
  uint8_t* xq = (uint8_t*)ws;
  float* sx = (float*)((char*)ws + align256((size_t)n * d_in));
  if ((st = launch_quant_rows_e4m3(x, x_dt, ld_x, n, d_in, xq, d_in, sx, stream))) return st;
  return run_w8a8_gemm(n, d_in, d_out, xq, sx, w_codes, w_scales, y, y_dt, stream);
}

size_t ispa_local_attn_proj_fp8_workspace_bytes(int64_t n_q, int32_t H, int32_t d, const ispa_seg* segs,
                                                int32_t n_segs) {
  if (n_q <= 0 || H < 1 || n_segs < 0 || n_segs > ISPA_MAX_SEGS) return 0;
  HostGroup g[1] = {{segs, n_segs}};
  const SplitPlan plan = plan_splits(attn_block_q(ISPA_BF16, d), n_q, H, g, 1);
  const size_t D = (size_t)H * d;
  // fp32 attention output and LSE, its codes and row scales, split parts
  return align256((size_t)n_q * D * 4) + align256((size_t)n_q * H * 4) + align256((size_t)n_q * D) +
         align256((size_t)n_q * 4) + split_workspace_bytes(n_q, H, d, plan, 1);
}

ispa_status ispa_local_attn_proj_fp8(int64_t n_q, int32_t H, int32_t d, float scale, const void* q,
                                     int64_t q_stride, const ispa_seg* segs, int32_t n_segs,
                                     const uint8_t* w_codes, const float* w_scales, void* y, ispa_dtype y_dt,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  ispa_status st = check_attn_common(ISPA_BF16, n_q, H, d, q, q_stride);
  if (st) return st;
  if (n_segs < 1) return fail(ISPA_ERR_INVALID_ARG, "n_segs must be >= 1");
  if ((st = check_group("segs", ISPA_BF16, H, d, segs, n_segs))) return st;
  const int32_t D = H * d;
  if ((st = check_w8a8(D, D, w_codes, w_scales, y, y_dt, n_q > 0))) return st;
  if (!std::isfinite(scale)) return fail(ISPA_ERR_INVALID_ARG, "scale must be finite");
  if (n_q == 0) return ISPA_OK;
  const size_t need = ispa_local_attn_proj_fp8_workspace_bytes(n_q, H, d, segs, n_segs);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "local_attn_proj_fp8 workspace too small or misaligned");
  char* wp = (char*)ws;
  float* O = (float*)wp;
  wp += align256((size_t)n_q * D * 4);
  float* lse = (float*)wp;
  wp += align256((size_t)n_q * H * 4);
  uint8_t* xq = (uint8_t*)wp;
  wp += align256((size_t)n_q * D);
  float* sx = (float*)wp;
  wp += align256((size_t)n_q * 4);
  HostGroup g[1] = {{segs, n_segs}};
  float* oo[1] = {O};
  float* ll[1] = {lse};
  st = run_group_attention(ISPA_BF16, n_q, H, d, scale, q, q_stride, g, 1, oo, ll, wp,
                           ws_bytes - (size_t)(wp - (char*)ws), stream);
  if (st) return st;
  if ((st = launch_quant_rows_e4m3(O, ISPA_F32, D, n_q, D, xq, D, sx, stream))) return st;
  return run_w8a8_gemm(n_q, D, D, xq, sx, w_codes, w_scales, y, y_dt, stream);
}

// ---------------------------------------------------------------- quantised local attention
static ispa_status check_rows_in(ispa_dtype dt, const void* x, int64_t stride, int64_t min_stride, bool any,
                                 const char* what) {
  if (!valid_dtype(dt)) return fail(ISPA_ERR_UNSUPPORTED, std::string(what) + ": dtype must be F32, BF16 or F16");
  if (stride < min_stride || stride % 4)
    return fail(ISPA_ERR_INVALID_ARG, std::string(what) + ": row stride must be >= H*d and a multiple of 4");
  if (any && !x) return fail(ISPA_ERR_INVALID_ARG, std::string(what) + ": null pointer");
  if (!aligned(x, dt == ISPA_F32 ? 16 : 8)) return fail(ISPA_ERR_INVALID_ARG, std::string(what) + ": misaligned rows");
  return ISPA_OK;
}

size_t ispa_kv_fp8_bytes(int64_t n, int32_t H, int32_t d) {
  if (n <= 0 || H < 1 || d != kF8D) return 0;
  return (size_t)H * f8_tiles(n) * kF8TileBytes;
}

size_t ispa_quantize_kv_fp8_workspace_bytes(int64_t n, int32_t H, int32_t d) {
  if (d != kF8D) return 0;
  return quant_kv_ws_bytes(n, H);
}

ispa_status ispa_quantize_kv_fp8(ispa_dtype dt, int64_t n, int32_t H, int32_t d, const void* k, int64_t k_stride,
                                 const void* v, int64_t v_stride, uint8_t* k_codes, uint8_t* v_codes,
                                 float* k_scales, float* v_scales, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (d != kF8D) return fail(ISPA_ERR_UNSUPPORTED, "the fp8 path takes head_dim 128");
  if (n < 0 || H < 1) return fail(ISPA_ERR_INVALID_ARG, "n must be >= 0 and H >= 1");
  const int64_t row = (int64_t)H * d;
  ispa_status st;
  if ((st = check_rows_in(dt, k, k_stride, row, n > 0, "k"))) return st;
  if ((st = check_rows_in(dt, v, v_stride, row, n > 0, "v"))) return st;
  if (n == 0) return ISPA_OK;
  if (!k_codes || !v_codes || !k_scales || !v_scales)
    return fail(ISPA_ERR_INVALID_ARG, "null k_codes, v_codes, k_scales or v_scales");
  if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 4) || !aligned(v_scales, 4))
    return fail(ISPA_ERR_INVALID_ARG, "misaligned codes or scales");
  if (!ws || ws_bytes < quant_kv_ws_bytes(n, H) || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "quantize_kv_fp8 workspace too small or misaligned");
  return launch_quant_kv_fp8(dt, n, H, k, k_stride, v, v_stride, k_codes, v_codes, k_scales, v_scales, ws, stream);
}

ispa_status ispa_quantize_q_fp8(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, const void* q, int64_t q_stride,
                                uint8_t* q_codes, float* q_scales, hipStream_t stream) {
  if (d != kF8D) return fail(ISPA_ERR_UNSUPPORTED, "the fp8 path takes head_dim 128");
  if (n_q < 0 || H < 1) return fail(ISPA_ERR_INVALID_ARG, "n_q must be >= 0 and H >= 1");
  ispa_status st;
  if ((st = check_rows_in(dt, q, q_stride, (int64_t)H * d, n_q > 0, "q"))) return st;
  if (n_q == 0) return ISPA_OK;
  if (!q_codes || !q_scales) return fail(ISPA_ERR_INVALID_ARG, "null q_codes or q_scales");
  if (!aligned(q_codes, 4) || !aligned(q_scales, 4)) return fail(ISPA_ERR_INVALID_ARG, "misaligned q_codes or q_scales");
  return launch_quant_q_fp8(dt, n_q, H, q, q_stride, q_codes, q_scales, stream);
}

static ispa_status check_attn_fp8(int64_t n_q, int32_t H, int32_t d, float scale, const uint8_t* q_codes,
                                  const float* q_scales, const ispa_seg_fp8* segs, int32_t n_segs,
                                  Attn8Seg* out, bool check_q = true) {
  if (d != kF8D) return fail(ISPA_ERR_UNSUPPORTED, "the fp8 path takes head_dim 128");
  if (n_q < 0 || H < 1) return fail(ISPA_ERR_INVALID_ARG, "n_q must be >= 0 and H >= 1");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(ISPA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (n_segs < 0 || n_segs > ISPA_MAX_SEGS_FP8) return fail(ISPA_ERR_INVALID_ARG, "segment count out of range");
  if (n_segs > 0 && !segs) return fail(ISPA_ERR_INVALID_ARG, "null segment table");
  for (int i = 0; i < n_segs; ++i) {
    const ispa_seg_fp8& s = segs[i];
    if (s.n < 0) return fail(ISPA_ERR_INVALID_ARG, "negative segment length");
    if (s.n > 0 && (!s.k_codes || !s.v_codes || !s.k_scales || !s.v_scales))
      return fail(ISPA_ERR_INVALID_ARG, "null codes or scales in a segment");
    if (!aligned(s.k_codes, 16) || !aligned(s.v_codes, 16) || !aligned(s.k_scales, 4) || !aligned(s.v_scales, 4))
      return fail(ISPA_ERR_INVALID_ARG, "misaligned codes or scales in a segment");
    out[i] = Attn8Seg{s.k_codes, s.v_codes, s.k_scales, s.v_scales, s.n};
  }
  if (!check_q) return ISPA_OK;
  if (n_q > 0 && (!q_codes || !q_scales)) return fail(ISPA_ERR_INVALID_ARG, "null q_codes or q_scales");
  if (!aligned(q_codes, 16) || !aligned(q_scales, 4)) return fail(ISPA_ERR_INVALID_ARG, "misaligned q_codes or q_scales");
  return ISPA_OK;
}

ispa_status ispa_local_attn_fp8(int64_t n_q, int32_t H, int32_t d, float scale, const uint8_t* q_codes,
                                const float* q_scales, const ispa_seg_fp8* segs, int32_t n_segs, void* o,
                                ispa_dtype o_dt, float* lse, hipStream_t stream) {
  Attn8Seg s8[ISPA_MAX_SEGS_FP8];
  ispa_status st = check_attn_fp8(n_q, H, d, scale, q_codes, q_scales, segs, n_segs, s8);
  if (st) return st;
  if (!valid_dtype(o_dt)) return fail(ISPA_ERR_UNSUPPORTED, "bad o_dt");
  if (n_q > 0 && !o) return fail(ISPA_ERR_INVALID_ARG, "null o");
  if (!aligned(o, o_dt == ISPA_F32 ? 16 : 8) || !aligned(lse, 4)) return fail(ISPA_ERR_INVALID_ARG, "misaligned o or lse");
  if (n_q == 0) return ISPA_OK;
  return launch_attn_fp8(n_q, H, scale, q_codes, q_scales, s8, n_segs, o, o_dt, lse, stream);
}

size_t ispa_local_attn_fp8_proj_workspace_bytes(int64_t n_q, int32_t H, int32_t d) {
  if (n_q <= 0 || H < 1 || d != kF8D) return 0;
  const size_t D = (size_t)H * d;
  // Q codes and scales, the fp32 attention output, its codes and row scales
  return align256((size_t)n_q * D) + align256((size_t)n_q * H * 4) + align256((size_t)n_q * D * 4) +
         align256((size_t)n_q * D) + align256((size_t)n_q * 4);
}

ispa_status ispa_local_attn_fp8_proj(int64_t n_q, int32_t H, int32_t d, float scale, ispa_dtype q_dt, const void* q,
                                     int64_t q_stride, const ispa_seg_fp8* segs, int32_t n_segs,
                                     const uint8_t* w_codes, const float* w_scales, void* y, ispa_dtype y_dt,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  Attn8Seg s8[ISPA_MAX_SEGS_FP8];
  ispa_status st = check_attn_fp8(n_q, H, d, scale, nullptr, nullptr, segs, n_segs, s8, false);
  if (st) return st;
  if ((st = check_rows_in(q_dt, q, q_stride, (int64_t)H * d, n_q > 0, "q"))) return st;
  const int32_t D = H * d;
  if ((st = check_w8a8(D, D, w_codes, w_scales, y, y_dt, n_q > 0))) return st;
  if (n_q == 0) return ISPA_OK;
  const size_t need = ispa_local_attn_fp8_proj_workspace_bytes(n_q, H, d);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(ISPA_ERR_WORKSPACE, "local_attn_fp8_proj workspace too small or misaligned");
  char* wp = (char*)ws;
  uint8_t* qc = (uint8_t*)wp;
  wp += align256((size_t)n_q * D);
  float* qsc = (float*)wp;
  wp += align256((size_t)n_q * H * 4);
  float* O = (float*)wp;
  wp += align256((size_t)n_q * D * 4);
  uint8_t* xq = (uint8_t*)wp;
  wp += align256((size_t)n_q * D);
  float* sx = (float*)wp;
  if ((st = launch_quant_q_fp8(q_dt, n_q, H, q, q_stride, qc, qsc, stream))) return st;
  if ((st = launch_attn_fp8(n_q, H, scale, qc, qsc, s8, n_segs, O, ISPA_F32, nullptr, stream))) return st;
  if ((st = launch_quant_rows_e4m3(O, ISPA_F32, D, n_q, D, xq, D, sx, stream))) return st;
  return run_w8a8_gemm(n_q, D, D, xq, sx, w_codes, w_scales, y, y_dt, stream);
}

}  // extern "C"
