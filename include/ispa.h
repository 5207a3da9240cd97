/*
 * libispa -- the data-parallel hot path of Instance-Specific Parametric
 * Absorption (ISPA) for AMD Instinct MI355X (gfx950).
 *
 * Pages cited below (all about arXiv 2607.00712, "Towards Memory-Efficient
 * Autoregressive Video Generation via Instance-Specific Parametric
 * Absorption"):
 *   EN review  -- English papernotes review: "Key Designs" 1-3.
 *   DE summary -- gist.science technical summary, section 2 "Methodik":
 *                 the objective and the closed form for Delta W.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument that names a tensor is DEVICE memory owned by
 *    the caller; the library never allocates, frees or keeps a pointer after
 *    the call returns.  Host arrays (segment tables, part lists) are read
 *    during the call only.
 *  - Calls are asynchronous and ordered on the caller's stream; none of them
 *    synchronises.  A null stream is the legacy default stream.
 *  - Layouts are row-major.  A token row holds all heads: Q and O are
 *    [n_q, H, d] = [n_q, D] with D = H*d; a key/value segment is [n, H, d]
 *    with a row stride in elements (>= H*d).  LSE is [n_q, H], natural log.
 *    W is [D_in, D_out] acting on row vectors (y = a W): pass the transpose of
 *    a torch.nn.Linear weight.  G, C, dW are [D, D].
 *  - Return codes: ISPA_OK, or an error detected on the host before anything
 *    was launched (ISPA_ERR_INVALID_ARG, ISPA_ERR_UNSUPPORTED,
 *    ISPA_ERR_WORKSPACE), or ISPA_ERR_HIP when a launch failed.  On error
 *    ispa_last_error() (thread-local) holds a message.  Numeric failures found
 *    on the device are reported through device outputs (info, status).
 *  - Workspace: calls that need scratch take (ws, ws_bytes), device memory
 *    of at least the size returned by the matching *_workspace_bytes query
 *    with the same shape arguments, aligned to 256 bytes.  Calls sharing a
 *    workspace must not overlap in time.
 *  - Stateless and thread-safe: no global flags, no hidden caches.  The one
 *    exception is ispa_w8a8_linear_noalloc, which keeps a fixed scratch
 *    array per device (see there).
 *  - The header is C as well as C++: a C program compiles it with the ROCm
 *    include directory and -D__HIP_PLATFORM_AMD__ (for hipStream_t) and links
 *    -lispa.
 */
#ifndef ISPA_H
#define ISPA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISPA_VERSION 10000 /* 1.0.0 */

typedef int32_t ispa_status;
enum {
  ISPA_OK = 0,
  ISPA_ERR_INVALID_ARG = 1, /* null pointer, bad size, K > N, stride < row */
  ISPA_ERR_UNSUPPORTED = 2, /* head_dim or dtype combination not built    */
  ISPA_ERR_WORKSPACE = 3,   /* workspace missing or too small             */
  ISPA_ERR_HIP = 4          /* launch or runtime error                    */
};

typedef int32_t ispa_dtype;
enum { ISPA_F32 = 0, ISPA_BF16 = 1, ISPA_F16 = 2 };

/* Maximum segments in one key group. */
#define ISPA_MAX_SEGS 8

/* One contiguous run of keys and values: rows [0, n) of k and v, each row
 * [H, d] of the call's dtype, rows k_stride / v_stride elements apart. */
typedef struct {
  const void* k;
  const void* v;
  int64_t n;
  int64_t k_stride;
  int64_t v_stride;
} ispa_seg;

int32_t ispa_version(void);
const char* ispa_status_str(ispa_status s);
const char* ispa_last_error(void);

/*
 * ispa_dual_attn -- dual-stream attention (EN review, Key Design 1: the
 * same query attends to the disjoint local and history groups, and each
 * group returns its value-weighted output and its log-sum-exp).
 *
 * For every query row i and head h, and each group g in {loc, hist} (the
 * concatenation of that group's segments):
 *   s_j = scale * <q_ih, k_jh>,  lse_g = ln sum_j exp(s_j),
 *   o_g = sum_j exp(s_j - lse_g) v_jh.
 * No mask inside a group.  An empty group (no keys) writes o = 0 and
 * lse = -inf.
 *   dt        ISPA_BF16 (MFMA path, d in {64,128}) or ISPA_F32 (d in {64,128}).
 *   q         [n_q, H, d] of dt, rows q_stride elements apart.
 *   loc,hist  host arrays of n_loc / n_hist segments (0 <= n <= ISPA_MAX_SEGS).
 *   o_loc,o_hist     fp32 [n_q, H, d] (dense, D per row).
 *   lse_loc,lse_hist fp32 [n_q, H].
 */
size_t ispa_dual_attn_workspace_bytes(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d,
                                      const ispa_seg* loc, int32_t n_loc,
                                      const ispa_seg* hist, int32_t n_hist);
ispa_status ispa_dual_attn(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale,
                           const void* q, int64_t q_stride,
                           const ispa_seg* loc, int32_t n_loc,
                           const ispa_seg* hist, int32_t n_hist,
                           float* o_loc, float* lse_loc, float* o_hist, float* lse_hist,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ispa_lse_merge -- n-way log-sum-exp merge (EN review, Key Design 1: the
 * full activation is recovered from the groups' outputs weighted by their
 * normalisation constants; a plain average would be wrong).
 *   lse = m + ln sum_p exp(lse_p - m), m = max_p lse_p,
 *   o   = sum_p exp(lse_p - lse) o_p.
 * Parts with lse = -inf get weight 0; if every part is -inf, o = 0 and
 * lse = -inf.
 *   o_parts, lse_parts  host arrays of n_parts (1..16) device pointers to
 *                       fp32 [n_q, H, d] and fp32 [n_q, H].
 *   o_full   fp32 [n_q, H, d] or NULL;  lse_full fp32 [n_q, H] or NULL.
 *   a0_out   part 0 converted to out_dt, [n_q, D], or NULL (A_loc when part
 *            0 is the local group).
 *   delta_out  (o - o_parts[0]) computed in fp32, converted to out_dt, or
 *            NULL (A_full - A_loc).
 *   out_dt   ISPA_F32, ISPA_BF16 or ISPA_F16 (round to nearest even).
 */
ispa_status ispa_lse_merge(int32_t n_parts, const float* const* o_parts,
                           const float* const* lse_parts, int64_t n_q, int32_t H, int32_t d,
                           float* o_full, float* lse_full, void* a0_out, void* delta_out,
                           ispa_dtype out_dt, hipStream_t stream);

/*
 * ispa_dual_attn_merge -- dual-stream attention followed by the LSE merge in
 * one call, for the warmup path (EN review, Key Design 1: the local and
 * history groups are attended separately and their outputs combined by
 * their log-sum-exp weights; the same review's Key Design 2 regresses
 * A_full - A_loc on A_loc).
 * Same inputs and grouping as ispa_dual_attn; the outputs are those that
 * ispa_lse_merge would give on its (o_loc, o_hist) results:
 *   a_loc    o_loc converted to out_dt, [n_q, D]   (A_loc)
 *   delta    o - o_loc in fp32, converted to out_dt, [n_q, D], where o is the
 *            merge of both groups                     (A_full - A_loc)
 *   lse_full fp32 [n_q, H] LSE of both groups, or NULL.
 * The groups' pieces are merged once, without materialising o_loc and o_hist
 * in fp32.  out_dt: ISPA_F32, ISPA_BF16 or ISPA_F16.  a_loc and delta must be
 * 16-byte aligned (8-byte for 16-bit out_dt).
 */
size_t ispa_dual_attn_merge_workspace_bytes(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d,
                                            const ispa_seg* loc, int32_t n_loc,
                                            const ispa_seg* hist, int32_t n_hist);
ispa_status ispa_dual_attn_merge(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale,
                                 const void* q, int64_t q_stride,
                                 const ispa_seg* loc, int32_t n_loc,
                                 const ispa_seg* hist, int32_t n_hist,
                                 void* a_loc, void* delta, ispa_dtype out_dt, float* lse_full,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ispa_accum_stats -- in-place accumulation of the regression statistics
 * (EN review, Key Design 2: activation outer products and activation-residual
 * cross statistics are accumulated over the warmup forward passes).
 *   R  = delta_a W                  (fp32 accumulation)
 *   r2 += ||R||_F^2                 (from the fp32 R, summed in fp64)
 *   G  += a_loc^T a_loc             (UPPER triangle i <= j only; entries
 *                                    below the diagonal are not touched)
 *   C  += a_loc^T R                 (R rounded to a_dt before this product)
 *   a_dt   type of a_loc and delta_a: ISPA_F32, ISPA_BF16 or ISPA_F16.  With
 *          BF16/F16 the products run on MFMA in that type; W is converted to
 *          a_dt on load (w_dt may differ).  ISPA_F32 requires w_dt = F32.
 *   a_loc, delta_a  [n, D] row-major; w [D, D]; G, C fp32 [D, D]; r2 one fp64.
 *   D must be a multiple of 64; n >= 0 (n = 0 is a no-op).
 * The caller zeroes G, C and r2 when a warmup starts.
 */
size_t ispa_accum_stats_workspace_bytes(ispa_dtype a_dt, int64_t n, int32_t D);
ispa_status ispa_accum_stats(ispa_dtype a_dt, ispa_dtype w_dt, int64_t n, int32_t D,
                             const void* a_loc, const void* delta_a, const void* w,
                             float* G, float* C, double* r2,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Statistics in the grouping of the printed closed form (DE summary,
 * Methodik: dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W;
 * EN review, Key Design 2: the statistics are accumulated over the warmup
 * forward passes).  The factor A_loc^T dA (dA = A_full - A_loc) does not
 * involve W, and ||dA W||^2 = <dA^T dA, W W^T>, so each warmup chunk adds
 * one symmetric rank-k update of X = [A_loc | dA]:
 *   G += A_loc^T A_loc,  M += A_loc^T dA,  H += dA^T dA
 * (4 n D^2 multiply-adds counted as flops, against 5 n D^2 for
 * ispa_accum_stats, and no R = dA W), and the switch forms C = M W and
 * r2 = <H, W W^T> once.  The accumulator is a per-layer state whose layout
 * is private to the library: ispa_gram_state_bytes(D) bytes, 16-byte
 * aligned, all-zero bytes meaning "no rows yet" (the caller zeroes it when
 * a warmup starts).
 *
 * ispa_accum_gram -- one chunk's rows into the state.
 *   a_dt     ISPA_F16 or ISPA_BF16 (the products run on MFMA in that type,
 *            exact, with fp32 sums).
 *   a_loc, delta_a  [n, D] row-major (D elements per row), 16-byte aligned.
 *   D a positive multiple of 64; n >= 0 (n = 0 is a no-op).
 * ispa_gram_finalize -- G, C and r2 of n_layers states (layer l at
 *   state + l*state_stride floats, its W at w + l*w_stride elements, its G
 *   and C at + l*mat_stride floats, its r2 at r2[l]), for ispa_solve_dw:
 *   G   the upper triangle of sum A_loc^T A_loc (entries below the diagonal
 *       are not touched), fp32 [D, D];
 *   C   M W, fp32 [D, D] (M split into three bf16 planes, so the product
 *       runs on the bf16 matrix core to fp32 accuracy);
 *   r2  <H, W W^T> summed in fp64.
 *   Written, not accumulated; the state is left as it was.  W: ISPA_BF16
 *   [D, D] (y = a W).  Needs ispa_gram_finalize_workspace_bytes(D) of
 *   workspace (reused layer by layer).
 */
size_t ispa_gram_state_bytes(int32_t D);
ispa_status ispa_accum_gram(ispa_dtype a_dt, int64_t n, int32_t D, const void* a_loc, const void* delta_a,
                            void* state, hipStream_t stream);
size_t ispa_gram_finalize_workspace_bytes(int32_t D);
ispa_status ispa_gram_finalize(int32_t n_layers, int32_t D, const void* state, int64_t state_stride,
                               const void* w, ispa_dtype w_dt, int64_t w_stride, float* G, float* C,
                               double* r2, int64_t mat_stride, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * ispa_solve_dw -- closed-form ridge absorption and reconstruction error,
 * batched over layers (DE summary, Methodik: Delta W minimises
 * ||A_loc (W + dW) - A_full W||^2 + lambda ||dW||^2, closed form
 * dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W; EN review,
 * Key Design 2 for eps).  Per layer l (matrices mat_stride elements apart):
 *   lambda = lambda_abs + lambda_rel * tr(G) / D
 *   G + lambda I = L L^T (fp64 Cholesky, G read from its upper triangle)
 *   dW  = L^-T L^-1 C                    (fp64, stored fp32)
 *   eps = r2 - <dW, C> - lambda ||dW||^2 (= ||A_loc dW - R||^2 at the ridge
 *                                         optimum, penalty excluded)
 *   info = 0, or the 1-based index of the first non-positive pivot (then dW
 *          and eps are NaN).
 *   w, w_eff  optional (both NULL or both set): w_eff = w + dW rounded once
 *          to w_dt (BF16, F16 or F32), same layout as w.
 *   D must be a multiple of 64.
 */
size_t ispa_solve_dw_workspace_bytes(int32_t n_layers, int32_t D);
ispa_status ispa_solve_dw(int32_t n_layers, int32_t D, const float* G, const float* C,
                          const double* r2, int64_t mat_stride, double lambda_abs,
                          double lambda_rel, float* dW, double* eps, int32_t* info,
                          const void* w, ispa_dtype w_dt, void* w_eff,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ispa_select_layers -- instance-specific layer selection (EN review, Key
 * Design 3: sort layers by increasing eps and take the K lowest as L-Layers;
 * K = x N for ISPA-x).  Stable: equal eps go to the lower layer index.
 *   eps       fp64 [n_layers] (device), 1 <= n_layers <= 1024, 0 <= K <= n.
 *   selected  int32 [K]: layer indices in ascending-eps order.
 *   is_local  uint8 [n_layers]: 1 for selected layers.
 *   status    int32 [1]: 0, or 1 if any eps is NaN (outputs then zero).
 */
ispa_status ispa_select_layers(int32_t n_layers, int32_t K, const double* eps,
                               int32_t* selected, uint8_t* is_local, int32_t* status,
                               hipStream_t stream);

/*
 * ispa_local_attn_proj -- post-switch layer (EN review, Key Designs 2-3: an
 * L-Layer attends to its retained sink and current keys only and projects
 * with W + dW; an F-Layer keeps full attention over its history with W).
 *   y = softmax(scale q k^T) v  over all keys of the segments, then y W.
 * When the launch would leave most CUs idle (fewer than 128 workgroups, one
 * per query tile and head), a long key set is split into blocks whose
 * partial (o, lse) are merged by the LSE rule before the projection;
 * otherwise it runs whole.
 *   dt      ISPA_BF16 (d in {64,128}) or ISPA_F32.
 *   w_proj  [D, D] of w_dt (W + dW for L-Layers, W for F-Layers); with
 *           dt = BF16, w_dt must be BF16 or F16 (products on MFMA in bf16);
 *           with dt = F32, w_dt must be F32.
 *   y       [n_q, D] of y_dt (ISPA_F32 or ISPA_BF16).
 *   n_segs  1..ISPA_MAX_SEGS; an empty key set gives y = 0.
 */
size_t ispa_local_attn_proj_workspace_bytes(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d,
                                            const ispa_seg* segs, int32_t n_segs);
ispa_status ispa_local_attn_proj(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d,
                                 float scale, const void* q, int64_t q_stride,
                                 const ispa_seg* segs, int32_t n_segs,
                                 const void* w_proj, ispa_dtype w_dt,
                                 void* y, ispa_dtype y_dt,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * W8A8 post-switch projection.  The pages report a 1.86x overall speed-up of
 * ISPA combined with W8A8 post-training quantisation (EN review, Key
 * Findings, the Figure 7 item; DE summary, section 4 "Experimentelle
 * Ergebnisse") and give no scheme.  The scheme here, our reading: OCP FP8
 * E4M3 codes for both operands of y = O W, one symmetric scale per activation
 * row (token) and per weight output column, fp32 accumulation on the fp8
 * matrix core.  For a row x: scale = max|x| / 448 and
 * code = E4M3(clamp(x / scale, -448, 448)), both divisions IEEE fp32, round
 * to nearest even, a zero magnitude stored as code 0x00; a zero row has
 * scale 0 and zero codes.
 *
 * ispa_quantize_w_fp8 -- the weight step, once per switch for each layer.
 *   w         [d_in, d_out] of w_dt (ISPA_BF16 or ISPA_F16), 8-byte aligned
 *             (W + dW of an L-Layer, or W of an F-Layer).
 *   w_codes   uint8 [d_out, d_in]: output column j's codes as row j.
 *   w_scales  fp32 [d_out].
 *   d_in, d_out positive multiples of 4.  Needs the workspace below.
 */
size_t ispa_quantize_w_fp8_workspace_bytes(int32_t d_in, int32_t d_out);
ispa_status ispa_quantize_w_fp8(ispa_dtype w_dt, int32_t d_in, int32_t d_out, const void* w,
                                uint8_t* w_codes, float* w_scales,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ispa_w8a8_linear -- y = Q(x) Q(W): x quantised per row here, W given as
 * ispa_quantize_w_fp8 left it;  y_ij = sx_i sw_j sum_k dec(qx_ik) dec(qw_jk).
 *   x         [n, d_in] of x_dt (ISPA_F32, ISPA_BF16 or ISPA_F16), rows ld_x
 *             elements apart (ld_x >= d_in, a multiple of 4); 16-byte aligned
 *             for F32, 8-byte for 16-bit types.
 *   w_codes   uint8 [d_out, d_in], 16-byte aligned; w_scales fp32 [d_out],
 *             16-byte aligned.
 *   y         [n, d_out] of y_dt (F32 16-byte aligned, BF16 or F16 8-byte).
 *   d_in a positive multiple of 64, d_out of 4.
 */
size_t ispa_w8a8_linear_workspace_bytes(int64_t n, int32_t d_in);
ispa_status ispa_w8a8_linear(ispa_dtype x_dt, int64_t n, int32_t d_in, int32_t d_out,
                             const void* x, int64_t ld_x, const uint8_t* w_codes,
                             const float* w_scales, void* y, ispa_dtype y_dt,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ispa_w8a8_linear_noalloc -- ispa_w8a8_linear for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * layouts, results and kernels as ispa_w8a8_linear, without (ws, ws_bytes):
 * the activation codes and row scales go to a fixed scratch array of
 * ISPA_NOALLOC_SCRATCH_BYTES in the library, one per device, held until the
 * process ends.  Its device address is looked up on the first call on each
 * device.  Limit: ispa_w8a8_linear_workspace_bytes(n, d_in) must not exceed
 * ISPA_NOALLOC_SCRATCH_BYTES (n <= 6548 rows at d_in = 5120); larger
 * calls return ISPA_ERR_INVALID_ARG before anything is launched.  The call
 * allocates nothing.  Every call on one device shares that device's
 * scratch: calls that overlap in time on one device (different streams or
 * threads without ordering) race and give wrong results; calls ordered on
 * one stream are safe.
 */
#define ISPA_NOALLOC_SCRATCH_BYTES (32u << 20)
ispa_status ispa_w8a8_linear_noalloc(ispa_dtype x_dt, int64_t n, int32_t d_in, int32_t d_out, const void* x,
                                     int64_t ld_x, const uint8_t* w_codes, const float* w_scales, void* y,
                                     ispa_dtype y_dt, hipStream_t stream);

/*
 * ispa_local_attn_proj_fp8 -- ispa_local_attn_proj with the W8A8 projection:
 * bf16 attention over the segments (as ispa_local_attn_proj, fp32 output),
 * then ispa_w8a8_linear of that output with (w_codes, w_scales) of
 * [D, D] (D = H d).  Arguments as the two calls it combines.
 */
size_t ispa_local_attn_proj_fp8_workspace_bytes(int64_t n_q, int32_t H, int32_t d,
                                                const ispa_seg* segs, int32_t n_segs);
ispa_status ispa_local_attn_proj_fp8(int64_t n_q, int32_t H, int32_t d, float scale,
                                     const void* q, int64_t q_stride,
                                     const ispa_seg* segs, int32_t n_segs,
                                     const uint8_t* w_codes, const float* w_scales,
                                     void* y, ispa_dtype y_dt,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Quantised local attention: the post-switch L-Layer's attention on the fp8
 * matrix core.  The pages report the W8A8 speed-up of ISPA (EN review, Key
 * Findings, the Figure 7 item; DE summary, section 4) and give no scheme;
 * the scheme here, our reading: the three operands as OCP FP8 E4M3 codes
 * with power-of-two scales, K and V once per cache chunk and head (when the
 * chunk is written), Q per query row and head.  A group's scale is the least
 * 2^e (e >= -126) with max|x| <= 448 * 2^e (1 for a group of zeros); a code is
 * the round-to-nearest-even E4M3 value of x / scale (exact division), a
 * magnitude that rounds to zero stored as 0x00.  The attention is then the
 * softmax attention of the dequantised operands; the kernel rounds its
 * probabilities to E4M3 as well (relative step 2^-4) and accumulates in fp32.
 * Head dimension 128 only.
 *
 * fp8 cache of one chunk of n keys: T = ceil(n / 64) tiles per head, each an
 * 8 KB block of K codes (64 keys x 128) and one of V codes (V transposed,
 * 128 x 64 key positions), both in the kernel's own row order and swizzle;
 * keys past n are zero codes.  k_codes and v_codes are each
 * ispa_kv_fp8_bytes(n, H, 128) bytes, 16-byte aligned; the scales are fp32 [H].
 *
 * ispa_quantize_kv_fp8 -- a chunk's K and V ([n, H, 128] rows k_stride /
 *   v_stride elements apart, dt ISPA_F32, ISPA_BF16 or ISPA_F16; 16-bit rows
 *   8-byte aligned, fp32 rows 16-byte aligned, strides multiples of 4) into the
 *   cache format.  Workspace: ispa_quantize_kv_fp8_workspace_bytes.
 * ispa_quantize_q_fp8 -- queries [n_q, H, 128] (rows q_stride elements apart,
 *   same dtypes and alignment) -> q_codes uint8 [n_q, H, 128] (4-byte aligned)
 *   and q_scales fp32 [n_q, H].
 * ispa_local_attn_fp8 -- for every query row and head, attention over the
 *   keys of the n_segs (0..ISPA_MAX_SEGS_FP8) chunks in order:
 *     o = sum_j softmax_j(scale <q^, k^_j>) v^_j,  lse = ln sum_j exp(s_j)
 *   (^ = dequantised).  q_codes 16-byte aligned; scale > 0 and finite;
 *   o [n_q, H, 128] of o_dt (fp32 16-byte, 16-bit types 8-byte aligned); lse
 *   fp32 [n_q, H] or NULL.  No keys at all: o = 0, lse = -inf.
 * ispa_local_attn_fp8_proj -- the post-switch L-Layer output with both stages
 *   quantised: q (q_dt) quantised as ispa_quantize_q_fp8, ispa_local_attn_fp8
 *   into an fp32 workspace, then ispa_w8a8_linear of that output with
 *   (w_codes, w_scales) of [D, D], D = 128 H.  y [n_q, D] of y_dt.
 */
#define ISPA_FP8_TILE_KEYS 64
/* Maximum chunks (segments) in one quantised attention call. */
#define ISPA_MAX_SEGS_FP8 64
size_t ispa_kv_fp8_bytes(int64_t n, int32_t H, int32_t d);
size_t ispa_quantize_kv_fp8_workspace_bytes(int64_t n, int32_t H, int32_t d);
ispa_status ispa_quantize_kv_fp8(ispa_dtype dt, int64_t n, int32_t H, int32_t d,
                                 const void* k, int64_t k_stride, const void* v, int64_t v_stride,
                                 uint8_t* k_codes, uint8_t* v_codes, float* k_scales, float* v_scales,
                                 void* ws, size_t ws_bytes, hipStream_t stream);
ispa_status ispa_quantize_q_fp8(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, const void* q,
                                int64_t q_stride, uint8_t* q_codes, float* q_scales, hipStream_t stream);

/* One chunk of the fp8 cache as ispa_quantize_kv_fp8 wrote it. */
typedef struct {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_scales;
  const float* v_scales;
  int64_t n;
} ispa_seg_fp8;

ispa_status ispa_local_attn_fp8(int64_t n_q, int32_t H, int32_t d, float scale,
                                const uint8_t* q_codes, const float* q_scales,
                                const ispa_seg_fp8* segs, int32_t n_segs,
                                void* o, ispa_dtype o_dt, float* lse, hipStream_t stream);
size_t ispa_local_attn_fp8_proj_workspace_bytes(int64_t n_q, int32_t H, int32_t d);
ispa_status ispa_local_attn_fp8_proj(int64_t n_q, int32_t H, int32_t d, float scale,
                                     ispa_dtype q_dt, const void* q, int64_t q_stride,
                                     const ispa_seg_fp8* segs, int32_t n_segs,
                                     const uint8_t* w_codes, const float* w_scales,
                                     void* y, ispa_dtype y_dt,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ISPA_H */
