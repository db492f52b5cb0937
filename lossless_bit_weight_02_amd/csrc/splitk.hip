// Sum of the partial outputs of a split-k GEMM (the GEMV and matrix-core kernels write one
// [m][n] slice per k range to a workspace): y[i] = part[0][i] + part[1][i] + ..., added in range
// order, so the result does not depend on which range finished first.
#include <hip/hip_runtime.h>

#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

// x [m][k] (bfloat16 bits) -> xt [k][16][8]: xt[c][r][t] = x[16 t + r][c] (0 past m), so the
// eight-tile matrix-core kernel's lane r16 finds the x values of rows r16, 16 + r16, ..., 112 + r16
// at one escape column in a single 16-byte load.
// A workgroup takes 16 columns: thread t reads 8 of them of x row t / 2 as one 16-byte load into
// LDS, then writes the 8 entries of run t % 16 at column t / 16 as one 16-byte store.  (x and the
// output are 16-byte aligned and k is a multiple of 128.)
__global__ __launch_bounds__(256) void k_x_transpose(const uint16_t* __restrict__ x, int m, int64_t k,
                                                     uint16_t* __restrict__ xt) {
  __shared__ uint16_t tile[128][18];
  const int64_t c0 = (int64_t)blockIdx.x * 16;
  const int t = threadIdx.x;
  {
    const int j = t >> 1, h = t & 1;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < m) v = *reinterpret_cast<const u32x4*>(x + (int64_t)j * k + c0 + 8 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[j][8 * h + 2 * i] = (uint16_t)(v[i] & 0xFFFFu);
      tile[j][8 * h + 2 * i + 1] = (uint16_t)(v[i] >> 16);
    }
  }
  __syncthreads();
  {
    const int c = t >> 4, r = t & 15;
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)tile[16 * (2 * i) + r][c] | (uint32_t)tile[16 * (2 * i + 1) + r][c] << 16;
    *reinterpret_cast<u32x4*>(xt + (c0 + c) * 128 + 8 * r) = o;
  }
}

hipError_t launch_x_transpose(const uint16_t* x, int m, int64_t k, uint16_t* xt, hipStream_t s) {
  if (k % 16 != 0 || m > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_x_transpose, dim3((unsigned)(k / 16)), dim3(256), 0, s, x, m, k, xt);
  return hipGetLastError();
}

// The partial slices arrive from memory (written by the previous kernel): every thread issues
// the loads of up to 16 slices at once -- buffer loads, which return 0 past the last slice
// instead of needing a branch -- and then adds them in order.
// The ordered sum over the k ranges of element i of the [rows][cols] partial slices.
__device__ __forceinline__ float range_sum(const Rsrc& rp, int splits, int64_t cnt, int64_t i) {
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
  return s;
}

// silu: the gate and up sums of output i (row r, column c of h [rows][cols / 2]) are the slices'
// columns 16 (c / 8) + c % 8 and that + 8; h = silu(gate) * up goes to r * (ldy / 2) + c.
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int splits,
                                                      int64_t rows, int64_t cols,
                                                      float* __restrict__ y, uint16_t* __restrict__ y16,
                                                      int64_t ldy, int silu_pairs) {
  const int64_t cnt = rows * cols;
  const Rsrc rp = make_rsrc(part, (uint32_t)((int64_t)splits * cnt * 4));
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int64_t oc = silu_pairs ? cols / 2 : cols, ld = silu_pairs ? ldy / 2 : ldy;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * oc; i += step) {
    const int64_t r = i / oc, c = i - r * oc;
    float v;
    if (silu_pairs) {
      const int64_t gc = 16 * (c / 8) + c % 8;
      const float gate = range_sum(rp, splits, cnt, r * cols + gc);
      const float up = range_sum(rp, splits, cnt, r * cols + gc + 8);
      v = silu(gate) * up;
    } else {
      v = range_sum(rp, splits, cnt, i);
    }
    if (y16) y16[r * ld + c] = float_to_bf16_rne(v);
    else y[r * ld + c] = v;
  }
}

// Top-1 over the workgroups' keys (see MfmaArgs::top1): row j's winner is the largest of
// part[g * 32 + j], g < groups; its row index and value are decoded from the key.
__global__ __launch_bounds__(64) void k_top1_final(const uint64_t* __restrict__ part, int groups,
                                                   int32_t* __restrict__ idx, float* __restrict__ val) {
  const int j = blockIdx.x, t = threadIdx.x;
  uint64_t b = 0;
  for (int g = t; g < groups; g += 64) {
    const uint64_t v = part[(int64_t)g * 32 + j];
    b = v > b ? v : b;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh /= 2) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)b, sh, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(b >> 32), sh, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    b = o > b ? o : b;
  }
  if (t == 0) {
    const uint32_t ord = (uint32_t)(b >> 32);
    const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    idx[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)b);
    val[j] = __builtin_bit_cast(float, u);
  }
}

// The best key over columns c0 .. c1 - 1 of one row of outputs (value order of the float bits,
// NaN above +Inf; ties to the lowest index row0 + column), reduced over the 256 threads of the
// workgroup (thread 0 returns it).
__device__ __forceinline__ uint64_t block_best_key(const float* __restrict__ yr, int64_t c0, int64_t c1,
                                                   int64_t row0) {
  __shared__ uint64_t s_b[4];
  const int t = threadIdx.x;
  uint64_t b = 0;
  for (int64_t c = c0 + t; c < c1; c += 256) {
    const uint32_t u = __builtin_bit_cast(uint32_t, yr[c]);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const uint64_t key = ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(row0 + c));
    b = key > b ? key : b;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh /= 2) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)b, sh, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(b >> 32), sh, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    b = o > b ? o : b;
  }
  if ((t & 63) == 0) s_b[t >> 6] = b;
  __syncthreads();
  if (t == 0)
    for (int i = 0; i < 4; ++i) b = s_b[i] > b ? s_b[i] : b;
  return b;
}

// Best key of each row j < m of y [m][cols] (row index = row0 + column), into keys[j].
__global__ __launch_bounds__(256) void k_top1_rows(const float* __restrict__ y, int64_t cols, int64_t row0,
                                                   uint64_t* __restrict__ keys) {
  const int j = blockIdx.x;
  const uint64_t b = block_best_key(y + (int64_t)j * cols, 0, cols, row0);
  if (threadIdx.x == 0) keys[j] = b;
}

hipError_t launch_top1_rows(const float* y, int m, int64_t cols, int64_t row0, uint64_t* keys, hipStream_t s) {
  hipLaunchKernelGGL(k_top1_rows, dim3((unsigned)m), dim3(256), 0, s, y, cols, row0, keys);
  return hipGetLastError();
}

hipError_t launch_top1_final(const uint64_t* part, int groups, int m, int32_t* idx, float* val,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_top1_final, dim3((unsigned)m), dim3(64), 0, s, part, groups, idx, val);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* part, int splits, int64_t rows, int64_t cols, YOut y,
                               int64_t ldy, hipStream_t s) {
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)blocks), dim3(256), 0, s, part, splits, rows, cols,
                     y.f, y.h, ldy, y.silu ? 1 : 0);
  return hipGetLastError();
}

}  // namespace w12
