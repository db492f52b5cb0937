// Per-block helpers of the streaming GEMM kernels (GEMV and CU-streaming): the raw loads of
// one 128-column block of a lane's row, their decode to bfloat16 pairs, and the row sum over
// a row's four column-group lanes.
#pragma once

#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

// One 128-column block of the lane's row: the raw 128-bit words it loads.
template <int FMT>
struct BlockRegs {
  u32x4 v[FMT == kFmtBF16 ? 4 : FMT == kFmtW12 ? 3 : 2];
};

// Buffers over one tile's blocks of the planes (or the dense baseline); an absent tile reads zeros.
template <int FMT>
struct TileRsrc {
  Rsrc r0, r1;
};


// Block `kb` of the tile (kb = ~0: nothing) into the lane's registers.
template <int FMT>
__device__ __forceinline__ void load_block(const TileRsrc<FMT>& t, uint32_t kb, uint32_t lane16,
                                           BlockRegs<FMT>& r) {
  if constexpr (FMT == kFmtBF16) {
    const uint32_t off = kb == ~0u ? kOOB : kb * kTileBF + lane16;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = __builtin_amdgcn_raw_buffer_load_b128(t.r0, off + 1024 * q, 0, kAuxNT);
  } else {
    const uint32_t off = kb == ~0u ? kOOB : kb * kTileAE + lane16;
    r.v[0] = __builtin_amdgcn_raw_buffer_load_b128(t.r0, off, 0, kAuxNT);
    r.v[1] = __builtin_amdgcn_raw_buffer_load_b128(t.r0, off + 1024, 0, kAuxNT);
    if constexpr (FMT == kFmtW12)
      r.v[2] = __builtin_amdgcn_raw_buffer_load_b128(t.r1, kb == ~0u ? kOOB : kb * kTileLO + lane16, 0, kAuxNT);
  }
}

// The 16 dwords of bfloat16 pairs (w' for W12/Q8, w for the baseline) of columns 32g..32g+31.
template <int FMT>
__device__ __forceinline__ void block_pairs(const BlockRegs<FMT>& r, uint32_t e112, uint32_t p[16]) {
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

// Sum over the 4 lanes r, r+16, r+32, r+48 (the column groups of one row).
__device__ __forceinline__ float group_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace w12
