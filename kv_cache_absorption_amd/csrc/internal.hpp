// Internal entry points shared between the translation units of libispa.
#pragma once

#include "common.hpp"

namespace ispa {

size_t solve_ws_bytes(int32_t n_layers, int32_t D);
ispa_status run_solve(int32_t L, int32_t D, const float* G, const float* C, const double* r2,
                      int64_t ms, double la, double lr, float* dW, double* eps, int32_t* info,
                      const void* w, int w_dt, void* w_eff, void* ws, hipStream_t stream);
ispa_status launch_select(int32_t N, int32_t K, const double* eps, int32_t* selected, uint8_t* is_local,
                          int32_t* status, hipStream_t stream);

}  // namespace ispa
