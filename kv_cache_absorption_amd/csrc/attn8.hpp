// Quantised (OCP FP8 E4M3) local attention: the fp8 key/value cache format,
// its quantisers and the attention kernel.
#pragma once

#include "common.hpp"

namespace ispa {

constexpr int kF8Keys = 64;                   // keys per cache tile
constexpr int kF8D = 128;                     // head dimension of the fp8 path
constexpr int kF8TileBytes = kF8Keys * kF8D;  // 8 KB: one K tile or one V^T tile
constexpr int kF8MaxSegs = ISPA_MAX_SEGS_FP8;

inline int64_t f8_tiles(int64_t n) { return (n + kF8Keys - 1) / kF8Keys; }

// Per-(tile, head) maxima of |K| and |V| of a chunk, fp32 [2][H][tiles].
size_t quant_kv_ws_bytes(int64_t n, int32_t H);
// One chunk of n keys (rows k_stride / v_stride elements apart, H heads of
// 128 of dt) into the cache format: per head a power-of-two scale for K and
// one for V, and the codes as tiles of 64 keys (the layout is stated where the
// kernels are defined).
ispa_status launch_quant_kv_fp8(int dt, int64_t n, int32_t H, const void* k, int64_t k_stride, const void* v,
                                int64_t v_stride, uint8_t* k_codes, uint8_t* v_codes, float* k_scales,
                                float* v_scales, void* ws, hipStream_t stream);
// Queries [n_q][q_stride] of dt (H heads of 128) -> codes [n_q][H][128] and
// power-of-two scales [n_q][H], one per row and head.
ispa_status launch_quant_q_fp8(int dt, int64_t n_q, int32_t H, const void* q, int64_t q_stride, uint8_t* q_codes,
                               float* q_scales, hipStream_t stream);

struct Attn8Seg {
  const uint8_t* k;  // [H][tiles][64][128] codes
  const uint8_t* v;  // [H][tiles][128][64] codes (V^T per tile)
  const float* ks;   // [H]
  const float* vs;   // [H]
  int64_t n;         // keys
};
// o [n_q][H][128] of o_dt (fp32, bf16 or f16), lse [n_q][H] (optional)
ispa_status launch_attn_fp8(int64_t n_q, int32_t H, float scale, const uint8_t* q_codes, const float* q_scales,
                            const Attn8Seg* segs, int n_segs, void* o, int o_dt, float* lse, hipStream_t stream);

}  // namespace ispa
