// W12 encoder, decoder and the HBM read probe (gfx950).
//
// Format: SpecPilot (arXiv 2611.02501), figure-captions page, Fig. 5(a) -- three 4-bit planes
// per bfloat16 weight (A = sign + mantissa[6:4], E = exponent offset inside a 16-binade window
// chosen per output channel, B = mantissa[3:0]) and an exact escape list for the weights
// outside the window.  Byte layout and window rule: see include/w12.h.
#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

// ---------------------------------------------------------------------------------------------
// Encoder step 1: per-row window choice.
// One workgroup per row.  Each wave keeps its own 256-bin exponent histogram in LDS (exponent
// fields 0 and 255 are not counted: zeros, subnormals, Inf and NaN never sit in a window).
// Coverage of window b is the sum of bins b..b+15 for b = 1..239; the row's base is the b of
// largest coverage, the smallest such b on ties, found with a max over the key
// (coverage << 32 | ~b).  A row with nothing counted gets base 1.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_analyze(const uint16_t* __restrict__ w, int64_t n,
                                                    int64_t k, uint8_t* __restrict__ base,
                                                    uint32_t* __restrict__ esc_ptr) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint64_t wave_best[4];
  const int tid = threadIdx.x, wid = tid >> 6;
  for (int64_t row = blockIdx.x; row < n; row += gridDim.x) {
    for (int i = tid; i < 4 * 256; i += kBlock) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint16_t* r = w + row * k;
    for (int64_t kk = 8 * (int64_t)tid; kk < k; kk += 8 * kBlock) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(r + kk);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t h = (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t e = (h >> 7) & 0xFFu;
        if (e != 0u && e != 255u) atomicAdd(&hist[wid][e], 1u);
      }
    }
    __syncthreads();
    const uint32_t total = hist[0][tid] + hist[1][tid] + hist[2][tid] + hist[3][tid];
    __syncthreads();
    hist[0][tid] = total;
    __syncthreads();
    uint64_t key = 0;
    const uint32_t b = (uint32_t)tid + 1u;
    if (b <= 239u) {
      uint32_t cov = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) cov += hist[0][b + j];
      key = ((uint64_t)cov << 32) | (uint64_t)(0xFFFFFFFFu - b);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
    if ((tid & 63) == 0) wave_best[wid] = key;
    __syncthreads();
    if (tid == 0) {
      uint64_t best = wave_best[0];
      for (int i = 1; i < 4; ++i) best = wave_best[i] > best ? wave_best[i] : best;
      const uint32_t bb = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
      const uint64_t cov = best >> 32;
      base[row] = (uint8_t)bb;
      esc_ptr[row + 1] = (uint32_t)((uint64_t)k - cov);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Encoder step 2: esc_ptr[1..n] (row escape counts) -> inclusive prefix sums, esc_ptr[0] = 0.
// One workgroup of 1024 threads walks the array in chunks; sums are kept in 64 bits and any
// offset that does not fit 32 bits is stored as 0xFFFFFFFF (the host reports W12_ERR_RANGE).
// ---------------------------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 4;

__global__ __launch_bounds__(kScanThreads) void k_scan(uint32_t* __restrict__ esc_ptr, int64_t n) {
  __shared__ uint64_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint64_t carry = 0;
  for (int64_t c0 = 0; c0 < n; c0 += (int64_t)kScanThreads * kScanPer) {
    uint64_t v[kScanPer];
    uint64_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t i = c0 + (int64_t)tid * kScanPer + j;
      v[j] = i < n ? esc_ptr[1 + i] : 0u;
      s += v[j];
    }
    uint64_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    uint64_t before = carry, chunk = 0;
    for (int i = 0; i < kScanThreads / 64; ++i) {
      if (i < wid) before += wave_tot[i];
      chunk += wave_tot[i];
    }
    uint64_t run = before + incl - s;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t i = c0 + (int64_t)tid * kScanPer + j;
      run += v[j];
      if (i < n) esc_ptr[1 + i] = run >= 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)run;
    }
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) esc_ptr[0] = 0u;
}

// ---------------------------------------------------------------------------------------------
// Encoder step 3: planes + escapes.  One workgroup per row (rows of the last row tile past n are
// padding and get zero planes); thread t of a pass owns the aligned group of 8 weights
// g = pass*256 + t, so escapes come out in ascending k after a workgroup exclusive scan of the
// per-thread escape counts.  The group's 8 AE bytes and 4 B bytes land at their tiled positions
// (see w12_device.hpp).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int64_t ae_offset(int64_t row, int64_t col, int64_t ktiles) {
  const int64_t tile = (row >> 4) * ktiles + (col >> 7);
  const int64_t c = col & 127;
  return tile * kTileAE + 1024 * ((c & 31) >> 4) + 16 * ((row & 15) + 16 * (c >> 5)) + (c & 15);
}

__device__ __forceinline__ int64_t lo_offset(int64_t row, int64_t col, int64_t ktiles) {
  // byte holding the B nibbles of the aligned group of 8 starting at col (col % 8 == 0)
  const int64_t tile = (row >> 4) * ktiles + (col >> 7);
  const int64_t c = col & 127;
  return tile * kTileLO + 16 * ((row & 15) + 16 * (c >> 5)) + ((c & 31) >> 1);
}

__global__ __launch_bounds__(kBlock) void k_pack(const uint16_t* __restrict__ w, int64_t n,
                                                 int64_t npad, int64_t k,
                                                 const uint8_t* __restrict__ base,
                                                 const uint32_t* __restrict__ esc_ptr,
                                                 uint8_t* __restrict__ ae, uint8_t* __restrict__ lo,
                                                 uint32_t* __restrict__ esc_col,
                                                 uint16_t* __restrict__ esc_val) {
  __shared__ uint32_t wave_cnt[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t groups = k >> 3;
  const int64_t ktiles = k / kTileCols;
  for (int64_t row = blockIdx.x; row < npad; row += gridDim.x) {
    if (row >= n) {  // padding row of the last tile: zero planes, no escapes
      for (int64_t g = tid; g < groups; g += kBlock) {
        *reinterpret_cast<u32x2*>(ae + ae_offset(row, 8 * g, ktiles)) = (u32x2){0u, 0u};
        *reinterpret_cast<uint32_t*>(lo + lo_offset(row, 8 * g, ktiles)) = 0u;
      }
      continue;  // uniform over the workgroup
    }
    const uint32_t b = base[row];
    const uint64_t out0 = esc_ptr[row];
    uint64_t running = 0;
    for (int64_t g0 = 0; g0 < groups; g0 += kBlock) {
      const int64_t g = g0 + tid;
      const bool act = g < groups;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (act) v = *reinterpret_cast<const u32x4*>(w + row * k + 8 * g);
      uint32_t a0 = 0, a1 = 0, nib = 0, escmask = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t h = (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t s = h >> 15, e = (h >> 7) & 0xFFu, m = h & 0x7Fu;
        const bool inside = e >= b && e <= b + 15u;
        const uint32_t code = inside ? (s << 7) | ((e - b) << 3) | (m >> 4) : 0u;
        const uint32_t nb = inside ? (m & 0xFu) : 0u;
        if (j < 4) a0 |= code << (8 * j);
        else a1 |= code << (8 * (j - 4));
        nib |= nb << (8 * (j & 3) + 4 * (j >> 2));
        if (act && !inside) escmask |= 1u << j;
      }
      const uint32_t c = __builtin_popcount(escmask);
      uint32_t incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (lane == 63) wave_cnt[wid] = incl;
      __syncthreads();
      uint32_t before = 0, pass_total = 0;
      for (int i = 0; i < 4; ++i) {
        if (i < wid) before += wave_cnt[i];
        pass_total += wave_cnt[i];
      }
      if (act) {
        *reinterpret_cast<u32x2*>(ae + ae_offset(row, 8 * g, ktiles)) = (u32x2){a0, a1};
        *reinterpret_cast<uint32_t*>(lo + lo_offset(row, 8 * g, ktiles)) = nib;
        if (escmask) {
          uint64_t idx = out0 + running + before + incl - c;
          const uint64_t row_end = esc_ptr[row + 1];  // never write past the row's CSR range
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (((escmask >> j) & 1u) && idx < row_end) {
              esc_col[idx] = (uint32_t)(8 * g + j);
              esc_val[idx] = (uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
              ++idx;
            }
          }
        }
      }
      running += pass_total;
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decoder: one thread per aligned group of 8 weights of a real row.  The group's w' pairs
// (exponent 112 + E) get (base - 112) added to both exponent fields at once:
// (base - 112) * 0x00800080 mod 2^32.  Neither half can carry or borrow into the other because
// base + E stays within 1..254.  Reads the tiled planes, writes row-major bf16.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_decode(const uint8_t* __restrict__ base,
                                                   const uint8_t* __restrict__ ae,
                                                   const uint8_t* __restrict__ lo, int64_t n,
                                                   int64_t k, uint16_t* __restrict__ out) {
  // One workgroup per tile; thread u reads AE bytes 8u..8u+7 of the tile (coalesced) =
  // row r = l % 16, columns 32g + 16h + 8s .. +7 with u = 128h + 2l + s, l = r + 16g.
  const int64_t ktiles = k / kTileCols;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows * ktiles;
  const uint32_t e112 = exp112_pair();
  const int u = threadIdx.x, h = u >> 7, l = (u & 127) >> 1, sh = u & 1;
  const int r = l & 15, g = l >> 4;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t row = (t / ktiles) * kTileRows + r;
    if (row >= n) continue;
    const int64_t col = (t % ktiles) * kTileCols + 32 * g + 16 * h + 8 * sh;
    const u32x2 a = load_nt(reinterpret_cast<const u32x2*>(ae + t * kTileAE) + u);
    const uint32_t lw = *reinterpret_cast<const uint32_t*>(lo + t * kTileLO + 16 * l + 8 * h + 4 * sh);
    const uint32_t shift = ((uint32_t)base[row] - 112u) * 0x00800080u;
    uint32_t p[4];
    window_group8(a.x, a.y, lw, e112, p);
    const u32x4 res = {p[0] + shift, p[1] + shift, p[2] + shift, p[3] + shift};
    *reinterpret_cast<u32x4*>(out + row * k + col) = res;
  }
}

// Dense bf16 W [n][k] (row-major) -> the tiled storage order of the baseline (npad rows; padding
// rows zero).  One thread per aligned group of 8 values.
__global__ __launch_bounds__(kBlock) void k_bf16_tile(const uint16_t* __restrict__ w, int64_t n,
                                                      int64_t npad, int64_t k,
                                                      uint16_t* __restrict__ out) {
  const int64_t groups_per_row = k >> 3;
  const int64_t total = npad * groups_per_row;
  const int64_t ktiles = k / kTileCols;
  for (int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * kBlock) {
    const int64_t row = g / groups_per_row;
    const int64_t col = 8 * (g - row * groups_per_row);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < n) v = *reinterpret_cast<const u32x4*>(w + row * k + col);
    const int64_t tile = (row >> 4) * ktiles + (col >> 7);
    const int64_t c = col & 127;
    const int64_t byte = tile * kTileBF + 1024 * ((c & 31) >> 3) + 16 * ((row & 15) + 16 * (c >> 5));
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(out) + byte) = v;
  }
}

// Escapes over their placeholder slots: one wave per row, lanes stride the row's escapes.
__global__ __launch_bounds__(kBlock) void k_escape_scatter(const uint32_t* __restrict__ esc_ptr,
                                                           const uint32_t* __restrict__ esc_col,
                                                           const uint16_t* __restrict__ esc_val,
                                                           int64_t n, int64_t k,
                                                           uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kBlock / 64);
  for (int64_t row = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); row < n; row += nw) {
    const uint32_t e1 = esc_ptr[row + 1];
    for (uint32_t e = esc_ptr[row] + lane; e < e1; e += 64)
      out[row * k + esc_col[e]] = esc_val[e];
  }
}

// ---------------------------------------------------------------------------------------------
// Read probe: every wave streams contiguous 1 KiB lines (one 128-bit word per lane), four lines
// in flight, and folds them with XOR; one word per workgroup goes to the sink.
// ---------------------------------------------------------------------------------------------
constexpr int kProbeLines = 4;

__global__ __launch_bounds__(kBlock) void k_read_probe(const u32x4* __restrict__ buf, uint64_t words,
                                                       uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint64_t nwaves = (uint64_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (uint64_t t = wave * 64 * kProbeLines; t < words; t += nwaves * 64 * kProbeLines) {
    u32x4 v[kProbeLines];
#pragma unroll
    for (int u = 0; u < kProbeLines; ++u) {
      const uint64_t i = t + (uint64_t)u * 64 + lane;
      v[u] = i < words ? load_nt(buf + i) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeLines; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) atomicXor(&sink[blockIdx.x & 4095], acc);
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
static int grid_rows(int64_t n) {
  return (int)(n < 1048576 ? n : 1048576);
}

hipError_t launch_analyze(const uint16_t* w, int64_t n, int64_t k, uint8_t* base, uint32_t* esc_ptr,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_analyze, dim3(grid_rows(n)), dim3(kBlock), 0, s, w, n, k, base, esc_ptr);
  return hipGetLastError();
}

hipError_t launch_scan(uint32_t* esc_ptr, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, esc_ptr, n);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* base,
                       const uint32_t* esc_ptr, uint8_t* ae, uint8_t* lo, uint32_t* esc_col,
                       uint16_t* esc_val, hipStream_t s) {
  const int64_t npad = padded_rows(n);
  hipLaunchKernelGGL(k_pack, dim3(grid_rows(npad)), dim3(kBlock), 0, s, w, n, npad, k, base, esc_ptr,
                     ae, lo, esc_col, esc_val);
  return hipGetLastError();
}

hipError_t launch_bf16_tile(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  const int64_t npad = padded_rows(n);
  int64_t blocks = (npad * (k >> 3) + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)di.cus * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_bf16_tile, dim3((unsigned)blocks), dim3(kBlock), 0, s, w, n, npad, k, out);
  return hipGetLastError();
}

hipError_t launch_decode(const Planes& p, int64_t n, int64_t k, uint16_t* out, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows * (k / kTileCols);
  const int64_t cap = (int64_t)di.cus * 8;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)(tiles < cap ? tiles : cap)), dim3(kBlock), 0, s, p.base,
                     p.ae, p.lo, n, k, out);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int64_t sblocks = (n + 3) / 4;
  if (sblocks > cap) sblocks = cap;
  hipLaunchKernelGGL(k_escape_scatter, dim3((unsigned)sblocks), dim3(kBlock), 0, s, p.esc_ptr,
                     p.esc_col, p.esc_val, n, k, out);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  const int blocks = di.cus * 8 < 4096 ? di.cus * 8 : 4096;
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(kBlock), 0, s,
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace w12
