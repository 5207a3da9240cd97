// Shared device/host helpers for libispa (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "ispa.h"

namespace ispa {

// ---- vector types used by the MFMA builtins ------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- scalar conversions (round to nearest even) ---------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
  return (float)h;
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  f32x2 v = {x, 0.0f};
  bf16x2 p = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, p) & 0xffffu;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// two floats -> packed pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// load one element of a matrix of runtime dtype as float
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, int dt) {
  if (dt == ISPA_F32) return ((const float*)p)[i];
  uint32_t b = ((const uint16_t*)p)[i];
  return dt == ISPA_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float x, int dt) {
  if (dt == ISPA_F32) {
    ((float*)p)[i] = x;
  } else {
    ((uint16_t*)p)[i] = (uint16_t)(dt == ISPA_BF16 ? f32_to_bf16_bits(x) : f32_to_f16_bits(x));
  }
}

// ---- wave helpers ----------------------------------------------------------
// The larger of the values of lane l and lane l ^ 32, in every lane.  After
// v_permlane32_swap of a register with a copy of itself, one result holds the
// lane's own value and the other its partner's (which is which depends on the
// half), so the maximum of the two results is the pair's maximum.
__device__ __forceinline__ float pair_max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Map a linear workgroup id so that the workgroups the hardware places on
// one XCD (ids b, b+8, b+16, ...) get a contiguous range of logical ids.
// Bijective for any n.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t n) {
  const uint32_t x = b & 7u, k = b >> 3;
  const uint32_t q = n >> 3, r = n & 7u;
  return x * q + (x < r ? x : r) + k;
}

// ---- host helpers -----------------------------------------------------------
void set_error(const std::string& msg);
inline int elem_bytes(int dt) { return dt == ISPA_F32 ? 4 : 2; }
inline bool valid_dtype(int dt) { return dt == ISPA_F32 || dt == ISPA_BF16 || dt == ISPA_F16; }
ispa_status check_launch(const char* what);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace ispa
