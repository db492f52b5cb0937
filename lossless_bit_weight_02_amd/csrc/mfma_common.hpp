// Shared by the two matrix-core GEMM kernels (mfma.hip: up to two activation tiles, x staged
// with global-to-LDS loads; mfma_wide.hip: three and four tiles, x staged through registers).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 8 bfloat16 of the k-group (l / 16); the 16x16 fp32 result gives
// lane l rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.  A = 16 weight rows, B = 16 activation
// rows, so the result is y^T for a 16 x 16 tile.  The weight lanes decode row r = l % 16,
// columns 32 g .. 32 g + 31 (g = l / 16) of each 128-column block, so MFMA step t of a block
// pairs A columns 32 g + 8 t .. +7 with the same columns of x.
#pragma once

#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

struct MfmaArgs {
  const uint16_t* x;   // x[m][k] (this launch's rows)
  int m;               // activation rows in this launch (<= 16 * NT)
  const uint8_t* base;
  const uint8_t* ae;   // tiled storage
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc_col;
  const uint16_t* esc_val;
  const uint16_t* w;   // dense bfloat16 W (baseline), tiled storage
  const float* scale;  // per-row scale of the 8-bit copy (its codes are in `ae`)
  float* y;            // y[m][ldy]; with splits > 1, split j writes y + j * ysplit
  int64_t ldy;
  int64_t n, k;
  int rounds;          // tiles per wave (the last ones may be empty)
  int splits;          // k ranges (workgroup b takes range b % splits); 1: the whole row
  int cps;             // x chunks per k range (the last range may be shorter)
  int64_t ysplit;      // floats between the partial outputs of consecutive k ranges
  // top-1 mode (non-null; one k range only): no y is written; for each x row j < m the largest
  // output of the workgroup's tiles goes to top1[blockIdx.x * 32 + j] as an ordered key
  // (top1_key below), and a second kernel picks the largest key over the workgroups
  uint64_t* top1;
  // y (or the range's workspace slice) is 16-byte aligned and ldy % 4 == 0: the epilogue stores
  // 16-byte vectors of 4 consecutive outputs (transposed through LDS)
  int yvec;
  // with y16 set (a single k range), the outputs go there as bfloat16 (nearest even) instead of y
  uint16_t* y16;
  // eight activation tiles (W12 and Q8): x transposed, [k][128] bfloat16 (rows past m zero); the
  // epilogue reads the escapes' x values from it
  const uint16_t* xt;
};

// Ordered key of output v of row n: larger v gives a larger key, and for equal v the smaller n.
// (A NaN output compares above +Inf.)
__device__ __forceinline__ uint64_t top1_key(float v, int64_t n) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
}

constexpr int kWaves = 12;                  // waves per workgroup, one workgroup per CU
constexpr int kEscCap = 128;                // escapes of one tile copied to LDS

template <int FMT>
struct ABlock {
  u32x4 v[FMT == kFmtBF16 ? 4 : FMT == kFmtW12 ? 3 : 2];
};

// Block kb of the wave's tile; offsets past the tile's range read zeros.
template <int FMT>
__device__ __forceinline__ void load_ablock(Rsrc r0, Rsrc r1, uint32_t kb, uint32_t lane16,
                                            ABlock<FMT>& b) {
  if constexpr (FMT == kFmtBF16) {
    const uint32_t off = kb * kTileBF + lane16;
#pragma unroll
    for (int q = 0; q < 4; ++q) b.v[q] = __builtin_amdgcn_raw_buffer_load_b128(r0, off + 1024 * q, 0, kAuxNT);
  } else {
    const uint32_t off = kb * kTileAE + lane16;
    b.v[0] = __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, kAuxNT);
    b.v[1] = __builtin_amdgcn_raw_buffer_load_b128(r0, off + 1024, 0, kAuxNT);
    if constexpr (FMT == kFmtW12)
      b.v[2] = __builtin_amdgcn_raw_buffer_load_b128(r1, kb * kTileLO + lane16, 0, kAuxNT);
  }
}

template <int FMT>
__device__ __forceinline__ void ablock_pairs(const ABlock<FMT>& r, uint32_t e112, uint32_t p[16]) {
  if constexpr (FMT == kFmtBF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p[4 * q] = r.v[q].x; p[4 * q + 1] = r.v[q].y; p[4 * q + 2] = r.v[q].z; p[4 * q + 3] = r.v[q].w;
    }
  } else if constexpr (FMT == kFmtW12) {
    window_group8(r.v[0].x, r.v[0].y, r.v[2].x, e112, p);
    window_group8(r.v[0].z, r.v[0].w, r.v[2].y, e112, p + 4);
    window_group8(r.v[1].x, r.v[1].y, r.v[2].z, e112, p + 8);
    window_group8(r.v[1].z, r.v[1].w, r.v[2].w, e112, p + 12);
  } else if constexpr (FMT == kFmtI8) {
    i8_group16(r.v[0], p);
    i8_group16(r.v[1], p + 8);
  } else {
    window_group8_q(r.v[0].x, r.v[0].y, e112, p);
    window_group8_q(r.v[0].z, r.v[0].w, e112, p + 4);
    window_group8_q(r.v[1].x, r.v[1].y, e112, p + 8);
    window_group8_q(r.v[1].z, r.v[1].w, e112, p + 12);
    if constexpr (FMT == kFmtQ8M) midpoint16(p);
  }
}

// The scales of a lane's four output rows rg .. rg + 3: the window bottoms of the W12 record
// (packed bytes; the scale is 2^(base - 112)) or the float scales of the 8-bit copy.  Rows past
// n read 0.
template <int FMT>
struct RowScales {
  uint32_t bases = 0;
  float f[FMT == kFmtI8 ? 4 : 1] = {};
  __device__ __forceinline__ void load(const MfmaArgs& a, int64_t rg) {
    if constexpr (FMT == kFmtI8) {
      const Rsrc rs = make_rsrc(a.scale, (uint32_t)a.n * 4u);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(rg + r) * 4u, 0, 0));
    } else {
      const Rsrc rb = make_rsrc(a.base, (uint32_t)a.n);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        bases |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rb, (uint32_t)(rg + r), 0, 0) << (8 * r);
    }
  }
  __device__ __forceinline__ float get(int r) const {
    if constexpr (FMT == kFmtI8) return f[r];
    else return window_scale((bases >> (8 * r)) & 0xFFu);
  }
};

typedef void (*MfmaKernel)(MfmaArgs);

// The register-staged kernel for nt = 3 or 4 activation tiles (mfma_wide.hip); silu: the exact
// pass with the SiLU(gate) * up epilogue on row-interleaved gate+up weights (y / y16 then hold
// h [m][ldy / 2], 8 outputs per 16-row tile).
MfmaKernel mfma_wide_kernel(Fmt f, int nt, bool silu = false);

}  // namespace w12
