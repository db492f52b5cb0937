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
// One workgroup per group of 16 rows (a row of tiles): wave w owns rows 4w..4w+3, and lane q of
// row r (16 lanes per row) reads columns 8q..8q+7 of every 128-column block, so a wave reads
// four 256-byte row segments per block; kEncU blocks are loaded together.  Each row keeps a
// 256-bin exponent histogram in LDS (exponent fields 0 and 255 are not counted: zeros,
// subnormals, Inf and NaN never sit in a window).  Coverage of window b is the sum of bins
// b..b+15 for b = 1..239; the row's base is the b of largest coverage, the smallest such b on
// ties, found with a max over the key (coverage << 32 | ~b).  A row with nothing counted gets
// base 1.  A row's lanes are all in one wave, so no workgroup barrier is needed.
// ---------------------------------------------------------------------------------------------
constexpr int kEncU = 4;   // 128-column blocks per loop pass of the encoder kernels

__global__ __launch_bounds__(kBlock) void k_analyze(const uint16_t* __restrict__ w, int64_t n,
                                                    int64_t k, uint8_t* __restrict__ base,
                                                    uint32_t* __restrict__ esc_ptr) {
  // rows 264 words apart: the four rows of a wave start 8 banks apart, so the bins they hit
  // (a few neighbouring exponents) do not share LDS banks across rows
  __shared__ uint32_t hist[16][264];
  const int tid = threadIdx.x, r = tid >> 4, q = tid & 15;
  const int64_t groups = (n + kTileRows - 1) / kTileRows;
  const int64_t ktiles = k / kTileCols;
  uint32_t* const hr = hist[r];
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t row = grp * kTileRows + r;
    const bool real = row < n;
    for (int i = q; i < 256; i += 16) hr[i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    const uint16_t* src = w + (real ? row : 0) * k + 8 * q;
    for (int64_t j0 = 0; j0 < ktiles; j0 += kEncU) {
      u32x4 v[kEncU];
#pragma unroll
      for (int i = 0; i < kEncU; ++i) {
        const bool ok = real && j0 + i < ktiles;
        v[i] = ok ? load_nt(reinterpret_cast<const u32x4*>(src + (j0 + i) * kTileCols))
                  : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kEncU; ++i) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint32_t e = (v[i][jj >> 1] >> (16 * (jj & 1) + 7)) & 0xFFu;
          if (e != 0u && e != 255u) atomicAdd(&hr[e], 1u);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
    // windows b = 16q .. 16q + 15 from a running sum over bins 16q .. 16q + 30
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) run += hr[16 * q + j];
    uint64_t key = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int b = 16 * q + j;
      run += b + 15 < 256 ? hr[b + 15] : 0u;   // run = bins b .. b + 15
      if (b >= 1 && b <= 239) {
        const uint64_t kb = ((uint64_t)run << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)b);
        key = kb > key ? kb : key;
      }
      run -= hr[b];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {   // max over the row's 16 lanes
      const uint64_t o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
    if (q == 0 && real) {
      base[row] = (uint8_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
      esc_ptr[row + 1] = (uint32_t)((uint64_t)k - (key >> 32));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");   // reads done before re-zeroing
  }
}

// ---------------------------------------------------------------------------------------------
// Encoder step 2: esc_ptr[1..n] (row escape counts) -> inclusive prefix sums, esc_ptr[0] = 0.
// One workgroup of 1024 threads walks the array in chunks of 20480.  A chunk goes through LDS:
// coalesced loads in, each thread scans a run of 20 consecutive counts, coalesced stores out.
// Sums are kept in 64 bits and any offset that does not fit 32 bits is stored as 0xFFFFFFFF (the
// host reports W12_ERR_RANGE).
// ---------------------------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 20;   // counts per thread and chunk

__global__ __launch_bounds__(kScanThreads) void k_scan(uint32_t* __restrict__ esc_ptr, int64_t n) {
  __shared__ uint32_t buf[kScanThreads * kScanPer];
  __shared__ uint64_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint64_t carry = 0;
  for (int64_t c0 = 0; c0 < n; c0 += (int64_t)kScanThreads * kScanPer) {
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t i = c0 + (int64_t)j * kScanThreads + tid;
      buf[j * kScanThreads + tid] = i < n ? esc_ptr[1 + i] : 0u;
    }
    __syncthreads();
    uint32_t v[kScanPer];
    uint64_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      v[j] = buf[tid * kScanPer + j];
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
      run += v[j];
      buf[tid * kScanPer + j] = run >= 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)run;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t i = c0 + (int64_t)j * kScanThreads + tid;
      if (i < n) esc_ptr[1 + i] = buf[j * kScanThreads + tid];
    }
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) esc_ptr[0] = 0u;
}

// ---------------------------------------------------------------------------------------------
// Encoder step 3: planes + escapes.
// One workgroup per group of 16 rows (npad / 16 groups; rows past n are padding and get zero
// planes).  Lane q of row r packs columns 8q..8q+7 of every 128-column block: its 8 AE bytes
// go to 1024 h + 16 (r + 16 g) + 8 (q % 2) and its 4 B-plane bytes to 16 (r + 16 g) + 4 (q % 4)
// of the tile (g = q / 4, h = (q / 2) % 2; see w12_device.hpp), so each tile's 2 KiB of AE and
// 1 KiB of B are written whole by one workgroup.  The row's escapes come out in ascending
// column order: within a block by an exclusive scan over the row's 16 lanes, across blocks by a
// running count those lanes keep.  A row's lanes are all in one wave: no workgroup barrier.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_pack(const uint16_t* __restrict__ w, int64_t n,
                                                 int64_t npad, int64_t k,
                                                 const uint8_t* __restrict__ base,
                                                 const uint32_t* __restrict__ esc_ptr,
                                                 uint8_t* __restrict__ ae, uint8_t* __restrict__ lo,
                                                 uint32_t* __restrict__ esc_col,
                                                 uint16_t* __restrict__ esc_val) {
  const int tid = threadIdx.x, r = tid >> 4, q = tid & 15;
  const int g = q >> 2, h = (q >> 1) & 1;
  const uint32_t ae_off = 1024u * h + 16u * (r + 16 * g) + 8u * (q & 1);
  const uint32_t lo_off = 16u * (r + 16 * g) + 4u * (q & 3);
  const int64_t groups = npad / kTileRows;
  const int64_t ktiles = k / kTileCols;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t row = grp * kTileRows + r;
    const bool real = row < n;
    const uint32_t b = real ? base[row] : 0u;
    const uint64_t out0 = real ? esc_ptr[row] : 0u;
    const uint64_t row_end = real ? esc_ptr[row + 1] : 0u;   // never write past the row's CSR range
    uint64_t running = 0;
    const uint16_t* src = w + (real ? row : 0) * k + 8 * q;
    for (int64_t j0 = 0; j0 < ktiles; j0 += kEncU) {
      u32x4 v[kEncU];
#pragma unroll
      for (int i = 0; i < kEncU; ++i) {
        const bool ok = real && j0 + i < ktiles;
        v[i] = ok ? load_nt(reinterpret_cast<const u32x4*>(src + (j0 + i) * kTileCols))
                  : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kEncU; ++i) {
        const int64_t j = j0 + i;
        if (j >= ktiles) break;   // uniform
        uint32_t a0 = 0, a1 = 0, nib = 0, escmask = 0;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint32_t hw = (v[i][jj >> 1] >> (16 * (jj & 1))) & 0xFFFFu;
          const uint32_t sg = hw >> 15, e = (hw >> 7) & 0xFFu, m = hw & 0x7Fu;
          const bool inside = e >= b && e <= b + 15u;
          const uint32_t code = inside ? (sg << 7) | ((e - b) << 3) | (m >> 4) : 0u;
          const uint32_t nb = inside ? (m & 0xFu) : 0u;
          if (jj < 4) a0 |= code << (8 * jj);
          else a1 |= code << (8 * (jj - 4));
          nib |= nb << (8 * (jj & 3) + 4 * (jj >> 2));
          if (real && !inside) escmask |= 1u << jj;
        }
        const int64_t tile = grp * ktiles + j;
        __builtin_nontemporal_store((u32x2){a0, a1}, reinterpret_cast<u32x2*>(ae + tile * kTileAE + ae_off));
        __builtin_nontemporal_store(nib, reinterpret_cast<uint32_t*>(lo + tile * kTileLO + lo_off));
        // escapes of this block: exclusive scan of the counts over the row's lanes q = 0..15
        const uint32_t c = __builtin_popcount(escmask);
        uint32_t incl = c;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const uint32_t o = __shfl_up(incl, off, 16);
          if (q >= off) incl += o;
        }
        const uint32_t block_total = __shfl(incl, 15, 16);
        if (escmask) {
          uint64_t idx = out0 + running + incl - c;
          const int64_t col0 = j * kTileCols + 8 * q;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            if (((escmask >> jj) & 1u) && idx < row_end) {
              esc_col[idx] = (uint32_t)(col0 + jj);
              esc_val[idx] = (uint16_t)((v[i][jj >> 1] >> (16 * (jj & 1))) & 0xFFFFu);
              ++idx;
            }
          }
        }
        running += block_total;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decoder: one thread per aligned group of 16 weights of a real row (as two groups of 8).  The group's w' pairs
// (exponent 112 + E) get (base - 112) added to both exponent fields at once:
// (base - 112) * 0x00800080 mod 2^32.  Neither half can carry or borrow into the other because
// base + E stays within 1..254.  Reads the tiled planes, writes row-major bf16.
// ---------------------------------------------------------------------------------------------
constexpr int kDecU = 4;   // units of two tiles per workgroup pass of the decoder (loads issued together)

__global__ __launch_bounds__(kBlock) void k_decode(const uint8_t* __restrict__ base,
                                                   const uint8_t* __restrict__ ae,
                                                   const uint8_t* __restrict__ lo, int64_t n,
                                                   int64_t k, uint16_t* __restrict__ out) {
  // A workgroup pass takes two tiles per unit; thread u works on tile 2 U + u / 128 of unit U,
  // row r = (u % 128) / 8 of it, columns 16 j .. 16 j + 15 with j = u % 8 (g = j / 2, h = j % 2).
  // Those 16 AE bytes sit at 1024 h + 16 (r + 16 g), their B nibbles in the 8 bytes at
  // 16 (r + 16 g) + 8 h of the tile's B plane (one 16-byte and one 8-byte load), and eight
  // lanes write one row's 256 output bytes.  A workgroup issues the loads of kDecU units before
  // decoding, so enough bytes are in flight per CU.
  const int64_t ktiles = k / kTileCols;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows * ktiles;
  const int64_t units = (tiles + 1) / 2;
  const uint32_t e112 = exp112_pair();
  const int u = threadIdx.x, sub = u >> 7, r = (u & 127) >> 3, j = u & 7;
  const int g = j >> 1, h = j & 1;
  const uint32_t ae_off = 1024u * h + 16u * (r + 16 * g);
  const uint32_t lo_off = 16u * (r + 16 * g) + 8u * h;
  const int64_t step = (int64_t)gridDim.x * kDecU;
  for (int64_t u0 = blockIdx.x; u0 < units; u0 += step) {
    u32x4 a[kDecU];
    u32x2 lw[kDecU];
    uint32_t bs[kDecU];
#pragma unroll
    for (int i = 0; i < kDecU; ++i) {
      const int64_t t = 2 * (u0 + (int64_t)i * gridDim.x) + sub;
      const bool ok = t < tiles;
      const int64_t tt = ok ? t : 0;
      const int64_t row = (tt / ktiles) * kTileRows + r;
      a[i] = load_nt(reinterpret_cast<const u32x4*>(ae + tt * kTileAE + ae_off));
      lw[i] = load_nt(reinterpret_cast<const u32x2*>(lo + tt * kTileLO + lo_off));
      bs[i] = base[row < n ? row : n - 1];
    }
#pragma unroll
    for (int i = 0; i < kDecU; ++i) {
      const int64_t t = 2 * (u0 + (int64_t)i * gridDim.x) + sub;
      const int64_t row = (t / ktiles) * kTileRows + r;
      if (t >= tiles || row >= n) continue;
      const int64_t col = (t % ktiles) * kTileCols + 16 * j;
      const uint32_t shift = (bs[i] - 112u) * 0x00800080u;
      uint32_t p[8];
      window_group8(a[i].x, a[i].y, lw[i].x, e112, p);
      window_group8(a[i].z, a[i].w, lw[i].y, e112, p + 4);
      const u32x4 r0 = {p[0] + shift, p[1] + shift, p[2] + shift, p[3] + shift};
      const u32x4 r1 = {p[4] + shift, p[5] + shift, p[6] + shift, p[7] + shift};
      // streaming stores: the decoded matrix is not read back by this kernel
      __builtin_nontemporal_store(r0, reinterpret_cast<u32x4*>(out + row * k + col));
      __builtin_nontemporal_store(r1, reinterpret_cast<u32x4*>(out + row * k + col + 8));
    }
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
// Workgroups for a loop over groups of 16 rows (each loop takes the groups blockIdx + i grid).
static int grid_groups(int64_t groups) {
  return (int)(groups < 1048576 ? groups : 1048576);
}

hipError_t launch_analyze(const uint16_t* w, int64_t n, int64_t k, uint8_t* base, uint32_t* esc_ptr,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_analyze, dim3(grid_groups((n + kTileRows - 1) / kTileRows)), dim3(kBlock), 0, s,
                     w, n, k, base, esc_ptr);
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
  hipLaunchKernelGGL(k_pack, dim3(grid_groups(npad / kTileRows)), dim3(kBlock), 0, s, w, n, npad, k, base, esc_ptr,
                     ae, lo, esc_col, esc_val);
  return hipGetLastError();
}

// Escape offsets of one part of a row-stacked record: its CSR shifted by the escapes of the parts
// before it.
__global__ __launch_bounds__(kBlock) void k_rebase(const uint32_t* __restrict__ src, int64_t cnt,
                                                   uint32_t add, uint32_t* __restrict__ dst) {
  const int64_t step = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < cnt; i += step) dst[i] = src[i] + add;
}

hipError_t launch_rebase(const uint32_t* src, int64_t cnt, uint32_t add, uint32_t* dst, hipStream_t s) {
  int64_t blocks = (cnt + kBlock - 1) / kBlock;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_rebase, dim3((unsigned)blocks), dim3(kBlock), 0, s, src, cnt, add, dst);
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
  const int64_t want = ((tiles + 1) / 2 + kDecU - 1) / kDecU;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)(want < cap ? want : cap)), dim3(kBlock), 0, s, p.base,
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
