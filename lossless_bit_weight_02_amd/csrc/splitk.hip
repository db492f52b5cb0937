// Sum of the partial outputs of a split-k GEMM (the GEMV and matrix-core kernels write one
// [m][n] slice per k range to a workspace): y[i] = part[0][i] + part[1][i] + ..., added in range
// order, so the result does not depend on which range finished first.
#include <hip/hip_runtime.h>

#include "w12_launch.hpp"

namespace w12 {

__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int splits,
                                                      int64_t cnt, float* __restrict__ y) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += step) {
    float s = part[i];
    for (int j = 1; j < splits; ++j) s += part[j * cnt + i];
    y[i] = s;
  }
}

hipError_t launch_split_reduce(const float* part, int splits, int64_t cnt, float* y, hipStream_t s) {
  int64_t blocks = (cnt + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)blocks), dim3(256), 0, s, part, splits, cnt, y);
  return hipGetLastError();
}

}  // namespace w12
