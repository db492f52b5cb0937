// Skinny GEMM for 9..64 activation rows on the matrix cores: y[m][n] = sum_k x[m][k] W[n][k].
//
// From about 16 rows the product is a dense contraction again (SpecPilot, arXiv 2611.02501,
// summary page, "Main Findings": the W12 GEMM is measured at 1 and at 32 rows), so the decoded
// weights feed v_mfma_f32_16x16x32_bf16 as its A operand, the register operand of the pages'
// design (figure-captions page, Fig. 5(b), there for wgmma).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 8 bfloat16 of the k-group (l / 16); the 16x16 fp32 result gives
// lane l rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.  A = 16 weight rows, B = 16 activation
// rows, so the result is y^T for a 16 x 16 tile.
//
// Work split: a wave owns RT tiles of 16 weight rows and all NT tiles of 16 activation rows,
// and walks k in blocks of 128.  Within a block, lane group g (= l / 16) owns the 32
// consecutive k starting at 32*g: two 128-bit loads of the AE plane and one of the B plane per
// weight row, four 128-bit loads of x per activation row.  MFMA step t (0..3) then takes k
// 32*g + 8t .. +7 from every group -- the same k on the A and the B side, which is all the
// instruction needs.  Weight rows are decoded straight into the A operand registers.
//
// Epilogue per (row n, column m): y = 2^(base-112) * (acc - 2^-15 * sum_esc x) + sum_esc x*v,
// the escape list of row n walked by the lane that owns (n, m).
#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

struct MfmaArgs {
  const uint16_t* x;   // x[m][ldx]
  int64_t ldx;
  int m;               // activation rows in this launch (<= 16 * NT)
  const uint8_t* base;
  const uint8_t* ae;
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc_col;
  const uint16_t* esc_val;
  const uint16_t* w;
  float* y;            // y[m][ldy]
  int64_t ldy;
  int64_t n, k;
};

constexpr int kKBlock = 128;

template <int FMT, int NT, int RT>
__global__ __launch_bounds__(kBlock) void k_mfma(MfmaArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t tasks = (a.n + 16 * RT - 1) / (16 * RT);
  const uint32_t e112 = exp112_pair();

  for (int64_t task = (int64_t)blockIdx.x * 4 + wave; task < tasks; task += nwaves) {
    const int64_t n0 = task * 16 * RT;
    floatx4 acc[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[rt][c] = (floatx4){0.f, 0.f, 0.f, 0.f};

    int64_t wrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t r = n0 + 16 * rt + r16;
      wrow[rt] = r < a.n ? r : a.n - 1;  // rows past the end read a valid row; results are dropped
    }

    for (int64_t kb = 0; kb < a.k; kb += kKBlock) {
      const int64_t kl = kb + 32 * g;
      const bool kin = kl < a.k;  // k % 32 == 0: a lane's 32-run is wholly inside or outside
      uint32_t A[RT][16];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (!kin) {
#pragma unroll
          for (int j = 0; j < 16; ++j) A[rt][j] = 0u;
          continue;
        }
        if constexpr (FMT == kFmtBF16) {
          const u32x4* src = reinterpret_cast<const u32x4*>(a.w + wrow[rt] * a.k + kl);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 v = load_nt(src + q);
            A[rt][4 * q] = v.x; A[rt][4 * q + 1] = v.y; A[rt][4 * q + 2] = v.z; A[rt][4 * q + 3] = v.w;
          }
        } else {
          const u32x4* src = reinterpret_cast<const u32x4*>(a.ae + wrow[rt] * a.k + kl);
          const u32x4 a0 = load_nt(src), a1 = load_nt(src + 1);
          if constexpr (FMT == kFmtW12) {
            const u32x4 l = load_nt(reinterpret_cast<const u32x4*>(a.lo + wrow[rt] * (a.k >> 1) + (kl >> 1)));
            window_group8(a0.x, a0.y, l.x, e112, &A[rt][0]);
            window_group8(a0.z, a0.w, l.y, e112, &A[rt][4]);
            window_group8(a1.x, a1.y, l.z, e112, &A[rt][8]);
            window_group8(a1.z, a1.w, l.w, e112, &A[rt][12]);
          } else {
            window_group8_q(a0.x, a0.y, e112, &A[rt][0]);
            window_group8_q(a0.z, a0.w, e112, &A[rt][4]);
            window_group8_q(a1.x, a1.y, e112, &A[rt][8]);
            window_group8_q(a1.z, a1.w, e112, &A[rt][12]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int mrow = 16 * c + r16;
        u32x4 B[4];
        if (kin && mrow < a.m) {
          const u32x4* src = reinterpret_cast<const u32x4*>(a.x + mrow * a.ldx + kl);
#pragma unroll
          for (int t = 0; t < 4; ++t) B[t] = src[t];
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) B[t] = (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const u32x4 av = {A[rt][4 * t], A[rt][4 * t + 1], A[rt][4 * t + 2], A[rt][4 * t + 3]};
            acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                 __builtin_bit_cast(bf16x8, B[t]),
                                                                 acc[rt][c], 0, 0, 0);
          }
        }
      }
    }

    // epilogue
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t nrow = n0 + 16 * rt + 4 * g + r;
        if (nrow >= a.n) continue;
        float sc = 1.0f;
        uint32_t e0 = 0, e1 = 0;
        if constexpr (FMT != kFmtBF16) {
          sc = window_scale(a.base[nrow]);
          e0 = a.esc_ptr[nrow];
          e1 = a.esc_ptr[nrow + 1];
        }
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const int mcol = 16 * c + r16;
          if (mcol >= a.m) continue;
          float v = acc[rt][c][r];
          if constexpr (FMT != kFmtBF16) {
            float sub = 0.0f, q = 0.0f;
            for (uint32_t e = e0; e < e1; ++e) {
              const float xv = bf16_to_float(a.x[mcol * a.ldx + a.esc_col[e]]);
              sub += xv;
              q = fmaf(xv, bf16_to_float(a.esc_val[e]), q);
            }
            v = fmaf(sc, fmaf(-kPlaceholder, sub, v), q);
          }
          a.y[mcol * a.ldy + nrow] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
typedef void (*MfmaKernel)(MfmaArgs);
constexpr int kRT = 2;

template <int FMT>
static MfmaKernel pick(int nt) {
  switch (nt) {
    case 1: return k_mfma<FMT, 1, kRT>;
    case 2: return k_mfma<FMT, 2, kRT>;
    case 3: return k_mfma<FMT, 3, kRT>;
    default: return k_mfma<FMT, 4, kRT>;
  }
}

static MfmaKernel pick_kernel(Fmt f, int nt) {
  if (f == kFmtW12) return pick<kFmtW12>(nt);
  if (f == kFmtQ8) return pick<kFmtQ8>(nt);
  return pick<kFmtBF16>(nt);
}

hipError_t launch_mfma(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                       float* y, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  for (int64_t m0 = 0; m0 < m; m0 += 64) {
    const int mb = (int)((m - m0) < 64 ? (m - m0) : 64);
    const int nt = (mb + 15) / 16;
    MfmaKernel kern = pick_kernel(f, nt);
    int occ = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern), kBlock, 0);
    if (err != hipSuccess) return err;
    if (occ < 1) occ = 1;
    const int64_t tasks = (n + 16 * kRT - 1) / (16 * kRT);
    int64_t blocks = (tasks + 3) / 4;
    const int64_t cap = (int64_t)di.cus * occ;
    if (blocks > cap) blocks = cap;
    MfmaArgs a;
    a.x = x + m0 * k;
    a.ldx = k;
    a.m = mb;
    a.base = p.base; a.ae = p.ae; a.lo = p.lo;
    a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
    a.w = p.w;
    a.y = y + m0 * n;
    a.ldy = n;
    a.n = n; a.k = k;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace w12
