// The separate 8-bit copy of a W12 record for the Q pass (SpecPilot, arXiv 2611.02501, summary
// page, Main Findings: the RTX PRO 6000 port reads an INT6/INT8 copy in the Q pass instead of the
// zero-copy 8-bit view).  The pages give no quantiser; this one is linear, per output row:
//   M_n = the largest magnitude among the row's in-window weights (the window's smallest value
//         2^(base - 127) when it has none), s_n = M_n / 127 in float32,
//   q   = round-half-even(w / s_n) in float32 for in-window weights, clamped to +-127,
//   q   = 0 at escaped slots, which stay exact through the record's own escape list.
// The codes go to the same tiled storage order as the record's AE plane (one byte per weight), so
// the Q-pass GEMM kernels stream them exactly like the 8-bit view.
//
// Built from the record alone: every slot of a row is decoded (the window trick of the GEMMs:
// w = w' * 2^(base - 112) with w' the bfloat16 of exponent 112 + E), which includes the escaped
// slots' placeholder 2^(base - 127).  That placeholder is the window's smallest magnitude, so it
// never raises the maximum of a row that has an in-window weight, and it is the floor above for
// a row that has none; a second kernel then writes 0 over every escaped slot's code.
#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

// One workgroup per 16-row tile row: thread u takes row r = u / 16 of the tile row and, of each
// pair of 128-column blocks, the 16-column piece j = u % 16 (block 2 i + j / 8, column group
// g = (j % 8) / 2, half h = j % 2): its 16 AE bytes at 1024 h + 16 (r + 16 g) of the block and
// their B nibbles in the 8 bytes at 16 (r + 16 g) + 8 h.  The 16 threads of a row are 16
// consecutive lanes of one wave, so the row maximum is four shuffles.
__global__ __launch_bounds__(kBlock) void k_i8_build(const uint8_t* __restrict__ base,
                                                     const uint8_t* __restrict__ ae,
                                                     const uint8_t* __restrict__ lo, int64_t n,
                                                     int64_t k, int8_t* __restrict__ q,
                                                     float* __restrict__ scale) {
  const int64_t ktiles = k / kTileCols;
  const int64_t trows = (n + kTileRows - 1) / kTileRows;
  const uint32_t e112 = exp112_pair();
  const int u = threadIdx.x, r = u >> 4, j = u & 15;
  const int jb = j >> 3, g = (j & 7) >> 1, h = j & 1;
  const uint32_t ae_off = 1024u * h + 16u * (r + 16 * g);
  const uint32_t lo_off = 16u * (r + 16 * g) + 8u * h;
  for (int64_t tr = blockIdx.x; tr < trows; tr += gridDim.x) {
    const int64_t row = tr * kTileRows + r;
    const bool live = row < n;
    const uint32_t bs = live ? base[row] : 112u;
    // pass 1: the largest |w'| (bfloat16 bits without the sign: larger bits, larger magnitude)
    uint32_t big = 0;
    for (int64_t kb = jb; kb < ktiles; kb += 2) {
      const int64_t t = tr * ktiles + kb;
      const u32x4 a = *reinterpret_cast<const u32x4*>(ae + t * kTileAE + ae_off);
      const u32x2 l = *reinterpret_cast<const u32x2*>(lo + t * kTileLO + lo_off);
      uint32_t p[8];
      window_group8(a.x, a.y, l.x, e112, p);
      window_group8(a.z, a.w, l.y, e112, p + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo16 = p[i] & 0x7FFFu, hi16 = (p[i] >> 16) & 0x7FFFu;
        big = big > lo16 ? big : lo16;
        big = big > hi16 ? big : hi16;
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)big, off, 16);
      big = big > o ? big : o;
    }
    const float wsc = window_scale(bs);
    // the row maximum is a window value (at least the placeholder), never zero
    const float m_n = bf16_to_float(big) * wsc;
    const float s_n = m_n / 127.0f;
    if (live && j == 0) scale[row] = s_n;
    // pass 2: the codes, written where the AE bytes were read
    for (int64_t kb = jb; kb < ktiles; kb += 2) {
      const int64_t t = tr * ktiles + kb;
      const u32x4 a = *reinterpret_cast<const u32x4*>(ae + t * kTileAE + ae_off);
      const u32x2 l = *reinterpret_cast<const u32x2*>(lo + t * kTileLO + lo_off);
      uint32_t p[8];
      window_group8(a.x, a.y, l.x, e112, p);
      window_group8(a.z, a.w, l.y, e112, p + 4);
      uint32_t out[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t pair = p[2 * i + b / 2];
          const float w = bf16_to_float((b & 1) ? pair >> 16 : pair & 0xFFFFu) * wsc;
          float c = rintf(w / s_n);
          c = c > 127.0f ? 127.0f : c < -127.0f ? -127.0f : c;
          const int32_t ci = live ? (int32_t)c : 0;
          word |= ((uint32_t)ci & 0xFFu) << (8 * b);
        }
        out[i] = word;
      }
      *reinterpret_cast<u32x4*>(q + t * kTileAE + ae_off) = (u32x4){out[0], out[1], out[2], out[3]};
    }
  }
}

// Code 0 at every escaped slot: escape e of row `row` at column c sits in tile
// (row / 16) * ktiles + c / 128 at 1024 ((c % 32) / 16) + 16 (row % 16 + 16 ((c % 128) / 32)) + c % 16.
__global__ __launch_bounds__(kBlock) void k_i8_zero_escapes(const uint32_t* __restrict__ esc_ptr,
                                                            const uint32_t* __restrict__ esc_col,
                                                            int64_t n, int64_t k,
                                                            int8_t* __restrict__ q) {
  const int lane = threadIdx.x & 63;
  const int64_t ktiles = k / kTileCols;
  const int64_t nw = (int64_t)gridDim.x * (kBlock / 64);
  for (int64_t row = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); row < n; row += nw) {
    const uint32_t e1 = esc_ptr[row + 1];
    const int64_t r = row % kTileRows;
    for (uint32_t e = esc_ptr[row] + lane; e < e1; e += 64) {
      const int64_t c = esc_col[e], cc = c % kTileCols;
      const int64_t t = (row / kTileRows) * ktiles + c / kTileCols;
      q[t * kTileAE + 1024 * ((cc % 32) / 16) + 16 * (r + 16 * (cc / 32)) + cc % 16] = 0;
    }
  }
}

hipError_t launch_i8_build(const Planes& p, int64_t n, int64_t k, int8_t* q, float* scale, hipStream_t s) {
  const int64_t trows = (n + kTileRows - 1) / kTileRows;
  const int64_t cap = 1 << 20;
  hipLaunchKernelGGL(k_i8_build, dim3((unsigned)(trows < cap ? trows : cap)), dim3(kBlock), 0, s, p.base,
                     p.ae, p.lo, n, k, q, scale);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(k_i8_zero_escapes, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(kBlock), 0, s,
                     p.esc_ptr, p.esc_col, n, k, q);
  return hipGetLastError();
}

}  // namespace w12
