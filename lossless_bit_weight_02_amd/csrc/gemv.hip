// Skinny GEMM for 1..8 activation rows: y[m][n] = sum_k x[m][k] * W[n][k].
//
// W12 records are decoded in registers (SpecPilot, arXiv 2611.02501, figure-captions page,
// Fig. 5(b): the GEMM decodes W12 records in registers) -- here into bfloat16 pairs for
// v_dot2_f32_bf16 instead of a matrix-unit operand, because at this many rows the product is a
// bandwidth-bound matrix-vector stream, not a dense contraction.
//
// Work split: persistent workgroups of 4 waves.  A workgroup first copies its k-slice of x into
// LDS, then every wave takes whole rows n (round robin over all waves of the grid).  Lane l
// owns 16 consecutive k per 1024-wide step, so one wave-wide 128-bit load covers 1 KiB of the
// AE plane and a 64-bit load 512 B of the B plane, fully coalesced.  Partial sums are reduced
// across the wave with DPP.  Escapes are applied after the k loop by the lanes in parallel.
//
// Window trick: a decoded pair is w' = w / 2^(base - 112), with the exponent field 112 + E
// (see w12_device.hpp), so the row's dot product sum_k x w' is scaled once by 2^(base - 112)
// at the end.  An escaped slot decodes to w' = 2^-15; its contribution x * 2^-15 is removed and
// x * (exact value) added.
#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

struct GemvArgs {
  const uint16_t* x;      // x[m][ldx] (bfloat16), the slice starts at column k0
  int64_t ldx;
  const uint8_t* base;
  const uint8_t* ae;
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc_col;
  const uint16_t* esc_val;
  const uint16_t* w;      // dense bfloat16 W for the baseline
  float* y;               // y[m][ldy]
  int64_t ldy;
  int64_t n, k;           // rows of W, row length (stride of every plane)
  int64_t k0;             // first column of this slice
  int kn;                 // slice length, multiple of 16
  int accumulate;         // add to y instead of overwriting (second and later slices)
};

constexpr int kStep = 1024;  // k per wave per step: 64 lanes x 16

// R rows per wave task (their loads interleave, so a wave keeps 2*U*R loads in flight), U steps
// of 1024 k issued together.
template <int FMT, int M, int R, int U>
__global__ __launch_bounds__(kBlock) void k_gemv(GemvArgs a) {
  extern __shared__ u32x4 xs[];  // [M][kn / 8] in 16-byte words
  const int tid = threadIdx.x, lane = tid & 63;
  const int kn = a.kn, kn8 = kn >> 3;

  for (int i = tid; i < M * kn8; i += kBlock) {
    const int m = i / kn8, j = i - m * kn8;
    xs[i] = *reinterpret_cast<const u32x4*>(a.x + m * a.ldx + a.k0 + 8 * j);
  }
  __syncthreads();
  const uint16_t* xs16 = reinterpret_cast<const uint16_t*>(xs);

  const uint32_t e112 = exp112_pair();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t tasks = (a.n + R - 1) / R;

  for (int64_t task = (int64_t)blockIdx.x * 4 + wave; task < tasks; task += nwaves) {
    const int64_t row0 = task * R;
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    // rows past the end of W (last task only) read the last row; their results are dropped
    const uint8_t* aer[R];
    const uint8_t* lor[R];
    const uint16_t* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r < a.n ? row0 + r : a.n - 1;
      aer[r] = nullptr; lor[r] = nullptr; wr[r] = nullptr;
      if constexpr (FMT == kFmtBF16) {
        wr[r] = a.w + row * a.k + a.k0;
      } else {
        aer[r] = a.ae + row * a.k + a.k0;
        if constexpr (FMT == kFmtW12) lor[r] = a.lo + row * (a.k >> 1) + (a.k0 >> 1);
      }
    }

    for (int kb = lane * 16; kb < kn; kb += kStep * U) {
      u32x4 A[R][U], A2[R][U];
      u32x2 L[R][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = kb + u * kStep;
        if (kk < kn) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if constexpr (FMT == kFmtBF16) {
              A[r][u] = load_nt(reinterpret_cast<const u32x4*>(wr[r] + kk));
              A2[r][u] = load_nt(reinterpret_cast<const u32x4*>(wr[r] + kk + 8));
            } else {
              A[r][u] = load_nt(reinterpret_cast<const u32x4*>(aer[r] + kk));
              if constexpr (FMT == kFmtW12) L[r][u] = load_nt(reinterpret_cast<const u32x2*>(lor[r] + (kk >> 1)));
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = kb + u * kStep;
        if (kk < kn) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            uint32_t p[8];
            if constexpr (FMT == kFmtBF16) {
              p[0] = A[r][u].x; p[1] = A[r][u].y; p[2] = A[r][u].z; p[3] = A[r][u].w;
              p[4] = A2[r][u].x; p[5] = A2[r][u].y; p[6] = A2[r][u].z; p[7] = A2[r][u].w;
            } else if constexpr (FMT == kFmtW12) {
              window_group8(A[r][u].x, A[r][u].y, L[r][u].x, e112, p);
              window_group8(A[r][u].z, A[r][u].w, L[r][u].y, e112, p + 4);
            } else {
              window_group8_q(A[r][u].x, A[r][u].y, e112, p);
              window_group8_q(A[r][u].z, A[r][u].w, e112, p + 4);
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const u32x4 x0 = xs[m * kn8 + (kk >> 3)];
              const u32x4 x1 = xs[m * kn8 + (kk >> 3) + 1];
              float s = acc[r][m];
              s = dot2_bf16(p[0], x0.x, s);
              s = dot2_bf16(p[1], x0.y, s);
              s = dot2_bf16(p[2], x0.z, s);
              s = dot2_bf16(p[3], x0.w, s);
              s = dot2_bf16(p[4], x1.x, s);
              s = dot2_bf16(p[5], x1.y, s);
              s = dot2_bf16(p[6], x1.z, s);
              s = dot2_bf16(p[7], x1.w, s);
              acc[r][m] = s;
            }
          }
        }
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r;
      if (row >= a.n) break;
      float* acr = acc[r];
      if constexpr (FMT != kFmtBF16) {
        // Escapes of this row inside the slice: remove the placeholder x * 2^-15 from the dense
        // sum P and collect the exact part Q = sum x * v separately, so that
        // y = 2^(base-112) P + Q rounds only once per reduction (a one-hot x then returns every
        // weight exactly).
        const uint32_t e0 = a.esc_ptr[row], e1 = a.esc_ptr[row + 1];
        const bool has_esc = e1 > e0;
        float q[M];
#pragma unroll
        for (int m = 0; m < M; ++m) q[m] = 0.0f;
        if (has_esc) {
          for (uint32_t e = e0 + lane; e < e1; e += 64) {
            const int64_t c = (int64_t)a.esc_col[e] - a.k0;
            if (c >= 0 && c < kn) {
              const float v = bf16_to_float(a.esc_val[e]);
#pragma unroll
              for (int m = 0; m < M; ++m) {
                const float xv = bf16_to_float(xs16[m * kn + c]);
                acr[m] = fmaf(-xv, kPlaceholder, acr[m]);
                q[m] = fmaf(xv, v, q[m]);
              }
            }
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) acr[m] = wave_sum_to_lane63(acr[m]);
        if (has_esc) {
#pragma unroll
          for (int m = 0; m < M; ++m) q[m] = wave_sum_to_lane63(q[m]);
        }
        const float sc = window_scale(a.base[row]);
#pragma unroll
        for (int m = 0; m < M; ++m) acr[m] = fmaf(sc, acr[m], q[m]);
      } else {
#pragma unroll
        for (int m = 0; m < M; ++m) acr[m] = wave_sum_to_lane63(acr[m]);
      }
      if (lane == 63) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float* yp = a.y + m * a.ldy + row;
          *yp = a.accumulate ? *yp + acr[m] : acr[m];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
typedef void (*GemvKernel)(GemvArgs);

// Steps of 1024 k issued together: all of a row when it has at most 6 steps.
static int unroll_for(int64_t kn) {
  const int64_t steps = (kn + kStep - 1) / kStep;
  return steps <= 2 ? 2 : steps <= 4 ? 4 : steps == 5 ? 5 : 6;
}

// Rows per wave task: two for the W12 and Q8 streams while the x reads stay cheap (m <= 4); the
// dense bf16 stream already moves 32 B per lane per step and runs best with one.
template <int FMT>
constexpr int rows_for(int m) { return FMT != kFmtBF16 && m <= 4 ? 2 : 1; }

template <int FMT, int M>
static GemvKernel pick_u(int u) {
  constexpr int R = rows_for<FMT>(M);
  switch (u) {
    case 2: return k_gemv<FMT, M, R, 2>;
    case 4: return k_gemv<FMT, M, R, 4>;
    case 5: return k_gemv<FMT, M, R, 5>;
    default: return k_gemv<FMT, M, R, 6>;
  }
}

template <int FMT>
static GemvKernel pick(int m, int u) {
  switch (m) {
    case 1: return pick_u<FMT, 1>(u);
    case 2: return pick_u<FMT, 2>(u);
    case 3: return pick_u<FMT, 3>(u);
    case 4: return pick_u<FMT, 4>(u);
    case 5: return pick_u<FMT, 5>(u);
    case 6: return pick_u<FMT, 6>(u);
    case 7: return pick_u<FMT, 7>(u);
    default: return pick_u<FMT, 8>(u);
  }
}

static GemvKernel pick_kernel(Fmt f, int m, int u) {
  if (f == kFmtW12) return pick<kFmtW12>(m, u);
  if (f == kFmtQ8) return pick<kFmtQ8>(m, u);
  return pick<kFmtBF16>(m, u);
}

static int rows_per_task(Fmt f, int m) {
  return f == kFmtW12 ? rows_for<kFmtW12>(m) : f == kFmtQ8 ? rows_for<kFmtQ8>(m) : rows_for<kFmtBF16>(m);
}

hipError_t launch_gemv(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                       float* y, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  for (int64_t m0 = 0; m0 < m; m0 += 8) {
    const int mb = (int)((m - m0) < 8 ? (m - m0) : 8);
    // k-slices whose x copy fits the LDS budget (one slice for every shape with 2*m*k <= 64 KiB)
    const int64_t lds_budget = di.max_lds < 65536 ? di.max_lds : 65536;
    int64_t slice = (lds_budget / (2 * mb)) & ~(int64_t)(kStep - 1);
    if (slice <= 0) slice = kStep;
    if (slice > k) slice = k;
    for (int64_t k0 = 0; k0 < k; k0 += slice) {
      const int kn = (int)((k - k0) < slice ? (k - k0) : slice);
      GemvKernel kern = pick_kernel(f, mb, unroll_for(kn));
      const size_t lds = (size_t)2 * mb * kn;
      int occ = 0;
      err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern),
                                                         kBlock, lds);
      if (err != hipSuccess) return err;
      if (occ < 1) occ = 1;
      const int64_t tasks = (n + rows_per_task(f, mb) - 1) / rows_per_task(f, mb);
      int64_t blocks = (tasks + 3) / 4;
      const int64_t cap = (int64_t)di.cus * occ;
      if (blocks > cap) blocks = cap;
      GemvArgs a;
      a.x = x + m0 * k;
      a.ldx = k;
      a.base = p.base; a.ae = p.ae; a.lo = p.lo;
      a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
      a.w = p.w;
      a.y = y + m0 * n;
      a.ldy = n;
      a.n = n; a.k = k; a.k0 = k0; a.kn = kn;
      a.accumulate = k0 > 0;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), lds, s, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace w12
