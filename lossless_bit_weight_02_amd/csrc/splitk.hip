// Sum of the partial outputs of a split-k GEMM (the GEMV and matrix-core kernels write one
// [m][n] slice per k range to a workspace): y[i] = part[0][i] + part[1][i] + ..., added in range
// order, so the result does not depend on which range finished first.
#include <hip/hip_runtime.h>

#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

// The partial slices arrive from memory (written by the previous kernel): every thread issues
// the loads of up to 16 slices at once -- buffer loads, which return 0 past the last slice
// instead of needing a branch -- and then adds them in order.
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int splits,
                                                      int64_t cnt, float* __restrict__ y) {
  const Rsrc rp = make_rsrc(part, (uint32_t)((int64_t)splits * cnt * 4));
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += step) {
    float s = 0.0f;
    for (int j0 = 0; j0 < splits; j0 += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rp, (uint32_t)(((int64_t)(j0 + j) * cnt + i) * 4), 0, 0));
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < splits) s = (j0 + j == 0) ? v[j] : s + v[j];
    }
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
