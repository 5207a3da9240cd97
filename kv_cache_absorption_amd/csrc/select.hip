// Layer selection: the K layers with the lowest eps become L-Layers (EN review,
// Key Design 3).  One workgroup; the rank of layer i is the number of layers
// ordered before it (lower eps, or equal eps and lower index), which is the
// position a stable ascending sort gives it.
#include "common.hpp"

namespace ispa {

namespace {

__global__ __launch_bounds__(1024) void select_kernel(int N, int K, const double* eps, int32_t* selected,
                                                      uint8_t* is_local, int32_t* status) {
  __shared__ double e[1024];
  __shared__ int bad;
  const int i = threadIdx.x;
  if (i == 0) bad = 0;
  __syncthreads();
  if (i < N) {
    e[i] = eps[i];
    if (isnan(e[i])) bad = 1;
  }
  __syncthreads();
  if (bad) {
    if (i < N) is_local[i] = 0;
    if (i < K) selected[i] = 0;
    if (i == 0) *status = 1;
    return;
  }
  if (i < N) {
    const double x = e[i];
    int rank = 0;
    for (int j = 0; j < N; ++j) rank += (e[j] < x) || (e[j] == x && j < i);
    is_local[i] = rank < K ? 1 : 0;
    if (rank < K) selected[rank] = i;
  }
  if (i == 0) *status = 0;
}

}  // namespace

ispa_status launch_select(int32_t N, int32_t K, const double* eps, int32_t* selected, uint8_t* is_local,
                          int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(1), dim3(1024), 0, stream, N, K, eps, selected, is_local, status);
  return check_launch("select_kernel");
}

}  // namespace ispa
