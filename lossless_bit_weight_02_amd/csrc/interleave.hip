// The record of row-interleaved gate+up weights, built from the gate and up records without
// decoding: output rows 16 t .. 16 t + 7 are gate rows 8 t .. 8 t + 7 and rows 16 t + 8 ..
// 16 t + 15 are up rows 8 t .. 8 t + 7, so both inputs of one SiLU(gate) * up output sit in one
// 16-row tile (summary page, Main Findings: W12 in plain decoding, where gate and up feed
// SiLU(gate) * up).  Windows and escape lists are per row, so the result is the parts' rows in
// the new order: byte-identical to encoding the interleaved matrix.
#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

// Part and row of output row R (the part's rows: 0 = gate, 1 = up).
__device__ __forceinline__ int64_t src_row(int64_t R, int& part) {
  const int64_t t = R >> 4, r = R & 15;
  part = r >= 8;
  return 8 * t + (r & 7);
}

// One thread per 16-byte piece of the output planes: per output tile and 128-column block, 128
// AE pieces (16 rows x 4 column groups x 2 halves) and 64 B pieces; each is one row's piece of a
// part's tile.  Also the window bottoms and escape counts (into esc_ptr[R + 1]) of every row.
__global__ __launch_bounds__(kBlock) void k_interleave_planes(Planes g, Planes u, int64_t rows, int64_t k,
                                                              uint8_t* __restrict__ base, uint8_t* __restrict__ ae,
                                                              uint8_t* __restrict__ lo,
                                                              uint32_t* __restrict__ esc_ptr) {
  const int64_t ktiles = k / kTileCols;
  const int64_t pieces = rows / kTileRows * ktiles * 192;
  const int64_t step = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < pieces; i += step) {
    const int64_t blk = i / 192;                 // output tile T = blk / ktiles, block kb = blk % ktiles
    const int c = (int)(i - blk * 192);
    const int64_t T = blk / ktiles, kb = blk - T * ktiles;
    const bool is_ae = c < 128;
    const int l = is_ae ? (c & 63) : c - 128, h = is_ae ? c >> 6 : 0;
    const int r = l & 15, cg = l >> 4;
    int part;
    const int64_t sr = src_row(T * kTileRows + r, part);
    const int64_t st = sr >> 4, rr = sr & 15;
    const Planes& p = part ? u : g;
    if (is_ae) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.ae + (st * ktiles + kb) * kTileAE + 1024 * h + 16 * (rr + 16 * cg));
      *reinterpret_cast<u32x4*>(ae + (T * ktiles + kb) * kTileAE + 1024 * h + 16 * l) = v;
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.lo + (st * ktiles + kb) * kTileLO + 16 * (rr + 16 * cg));
      *reinterpret_cast<u32x4*>(lo + (T * ktiles + kb) * kTileLO + 16 * l) = v;
    }
  }
  for (int64_t R = (int64_t)blockIdx.x * kBlock + threadIdx.x; R < rows; R += step) {
    int part;
    const int64_t sr = src_row(R, part);
    const Planes& p = part ? u : g;
    base[R] = p.base[sr];
    esc_ptr[R + 1] = p.esc_ptr[sr + 1] - p.esc_ptr[sr];
  }
}

// One wave per output row: its escapes copied from the part's row, in order.
__global__ __launch_bounds__(kBlock) void k_interleave_escapes(Planes g, Planes u, int64_t rows,
                                                               const uint32_t* __restrict__ esc_ptr,
                                                               uint32_t* __restrict__ esc_col,
                                                               uint16_t* __restrict__ esc_val) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kBlock / 64);
  for (int64_t R = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); R < rows; R += nw) {
    int part;
    const int64_t sr = src_row(R, part);
    const Planes& p = part ? u : g;
    const uint32_t s0 = p.esc_ptr[sr], s1 = p.esc_ptr[sr + 1], d0 = esc_ptr[R];
    for (uint32_t e = lane; s0 + e < s1; e += 64) {
      esc_col[d0 + e] = p.esc_col[s0 + e];
      esc_val[d0 + e] = p.esc_val[s0 + e];
    }
  }
}

hipError_t launch_interleave(const Planes& gate, const Planes& up, int64_t rows, int64_t k, uint8_t* base,
                             uint8_t* ae, uint8_t* lo, uint32_t* esc_ptr, uint32_t* esc_col, uint16_t* esc_val,
                             hipStream_t s) {
  const int64_t pieces = rows / kTileRows * (k / kTileCols) * 192;
  int64_t blocks = (pieces + kBlock - 1) / kBlock;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_interleave_planes, dim3((unsigned)blocks), dim3(kBlock), 0, s, gate, up, rows, k,
                     base, ae, lo, esc_ptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_scan(esc_ptr, rows, s);
  if (err != hipSuccess) return err;
  int64_t eblocks = (rows + 3) / 4;
  if (eblocks > 8192) eblocks = 8192;
  hipLaunchKernelGGL(k_interleave_escapes, dim3((unsigned)eblocks), dim3(kBlock), 0, s, gate, up, rows,
                     esc_ptr, esc_col, esc_val);
  return hipGetLastError();
}

}  // namespace w12
