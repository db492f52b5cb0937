// Skinny GEMM for 9..64 activation rows on the matrix cores: y[m][n] = sum_k x[m][k] W[n][k].
//
// From about 16 rows the product is a dense contraction again (SpecPilot, arXiv 2611.02501,
// summary page, "Main Findings": the W12 GEMM is measured at 1 and at 32 rows), so the decoded
// weights feed v_mfma_f32_16x16x32_bf16 as its A operand -- the register operand of the pages'
// design (figure-captions page, Fig. 5(b), there for wgmma).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 8 bfloat16 of the k-group (l / 16); the 16x16 fp32 result gives
// lane l rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.  A = 16 weight rows, B = 16 activation
// rows, so the result is y^T for a 16 x 16 tile.
//
// The tiled plane storage (w12_device.hpp) already holds each 16-row x 128-column block in this
// lane order: lane l = r + 16g loads row r, columns 32g..32g+31 with wave-wide 1 KiB reads and
// decodes them straight into four A operands (MFMA step t takes columns 32g + 8t .. +7 from
// group g; the B operand is built with the same column mapping).  Each wave owns one tile and
// keeps the next D blocks of it in flight.  The four waves of a workgroup share x: 256-column
// chunks of the m rows of x are staged in LDS (double buffered, the next chunk held in
// registers), and every wave reads its B operands from there.
//
// Epilogue per (row n, column m): y = 2^(base-112) * (acc - 2^-15 * sum_esc x) + sum_esc x*v,
// the escape lists of rows n walked by the lanes that own (n, m); the tile's escapes are copied
// to LDS at the start of the tile so the epilogue only waits for its x loads.
#include "w12_device.hpp"
#include "w12_launch.hpp"

namespace w12 {

struct MfmaArgs {
  const uint16_t* x;   // x[m][ldx]
  int64_t ldx;
  int m;               // activation rows in this launch (<= 16 * NT)
  const uint8_t* base;
  const uint8_t* ae;   // tiled storage
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc_col;
  const uint16_t* esc_val;
  const uint16_t* w;   // dense bfloat16 W (baseline), tiled storage
  float* y;            // y[m][ldy]
  int64_t ldy;
  int64_t n, k;
};

constexpr int kChunk = 256;           // columns of x staged per LDS buffer
constexpr int kXPitch = kChunk + 8;   // padded LDS row (bfloat16 elements)
constexpr int kEscCap = 256;          // escapes of one tile staged in LDS (more: read from memory)
constexpr int kEscBatch = 4;          // escapes per epilogue step

template <int FMT>
struct ABlock {
  u32x4 v[FMT == kFmtBF16 ? 4 : FMT == kFmtW12 ? 3 : 2];
};

template <int FMT>
__device__ __forceinline__ void load_ablock(const MfmaArgs& a, int64_t tile_block, int lane, ABlock<FMT>& r) {
  if constexpr (FMT == kFmtBF16) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.w) + tile_block * (kTileBF / 16) + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = load_nt(src + 64 * q);
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.ae) + tile_block * (kTileAE / 16) + lane;
    r.v[0] = load_nt(src);
    r.v[1] = load_nt(src + 64);
    if constexpr (FMT == kFmtW12)
      r.v[2] = load_nt(reinterpret_cast<const u32x4*>(a.lo) + tile_block * (kTileLO / 16) + lane);
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
  } else {
    window_group8_q(r.v[0].x, r.v[0].y, e112, p);
    window_group8_q(r.v[0].z, r.v[0].w, e112, p + 4);
    window_group8_q(r.v[1].x, r.v[1].y, e112, p + 8);
    window_group8_q(r.v[1].z, r.v[1].w, e112, p + 12);
  }
}

// Registers are capped so that three workgroups (12 waves) fit on a CU for up to 32 activation
// rows: the 544 tiles-of-4 of a 34816-row weight are then all resident at once, no second round.
template <int FMT, int NT, int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(NT <= 2 ? 3 : 2, 8)))
void k_mfma(MfmaArgs a) {
  constexpr int NX = 16 * NT * kChunk / 8 / kBlock;   // 16-byte words of x per thread per chunk
  static_assert(NX >= 1, "x chunk too small for the workgroup");
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][16 * NT * kXPitch];
  __shared__ uint32_t s_ecol[4][kEscCap];       // per wave: escapes of its tile (column, value)
  __shared__ uint16_t s_eval[4][kEscCap];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ktiles = a.k / kTileCols;
  const int KB = (int)ktiles;
  const int nch = (int)((a.k + kChunk - 1) / kChunk);
  const int64_t tiles = (a.n + kTileRows - 1) / kTileRows;
  const int64_t passes = (tiles + 3) / 4;
  const uint32_t e112 = exp112_pair();

  for (int64_t pass = blockIdx.x; pass < passes; pass += gridDim.x) {
    int64_t tile = pass * 4 + w;
    const bool valid = tile < tiles;
    tile = valid ? tile : tiles - 1;             // every wave stays in the barriers below
    const int64_t tb0 = tile * ktiles;

    floatx4 acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = (floatx4){0.f, 0.f, 0.f, 0.f};

    ABlock<FMT> buf[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < KB) load_ablock<FMT>(a, tb0 + d, lane, buf[d]);

    // The escapes of this lane's four rows 4g..4g+3 form one contiguous CSR range; the whole
    // tile's escapes are copied into LDS now, while the A blocks stream, so the epilogue only
    // waits for its x loads.
    uint32_t my_e0 = 0, my_b1 = 0, my_b2 = 0, my_b3 = 0, my_e1 = 0, t_e0 = 0, t_e1 = 0;
    if constexpr (FMT != kFmtBF16) {
      const int64_t row0 = tile * kTileRows;
      auto ptr_at = [&](int64_t r) { return a.esc_ptr[r < a.n ? r : a.n]; };
      t_e0 = ptr_at(row0);
      t_e1 = ptr_at(row0 + kTileRows);
      my_e0 = ptr_at(row0 + 4 * g);
      my_b1 = ptr_at(row0 + 4 * g + 1);
      my_b2 = ptr_at(row0 + 4 * g + 2);
      my_b3 = ptr_at(row0 + 4 * g + 3);
      my_e1 = ptr_at(row0 + 4 * g + 4);
      if (t_e1 - t_e0 <= (uint32_t)kEscCap) {
        for (uint32_t e = t_e0 + lane; e < t_e1; e += 64) {
          s_ecol[w][e - t_e0] = a.esc_col[e];
          s_eval[w][e - t_e0] = a.esc_val[e];
        }
      }
    }

    u32x4 rx[NX];
    auto load_x = [&](int c) {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int e = tid + i * kBlock, mr = e / (kChunk / 8), c8 = e % (kChunk / 8);
        const int64_t col = (int64_t)c * kChunk + 8 * c8;
        rx[i] = (mr < a.m && col < a.k) ? *reinterpret_cast<const u32x4*>(a.x + mr * a.ldx + col)
                                        : (u32x4){0u, 0u, 0u, 0u};
      }
    };
    auto store_x = [&](int b) {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int e = tid + i * kBlock, mr = e / (kChunk / 8), c8 = e % (kChunk / 8);
        *reinterpret_cast<u32x4*>(&s_x[b][mr * kXPitch + 8 * c8]) = rx[i];
      }
    };

    __syncthreads();                             // the previous pass no longer reads s_x
    load_x(0);
    store_x(0);
    if (nch > 1) load_x(1);
    __syncthreads();

    int kb = 0;
    for (int c = 0; c < nch; ++c) {
      const int b = c & 1;
#pragma unroll
      for (int qb = 0; qb < kChunk / kTileCols; ++qb) {
        if (kb < KB) {
          const int slot = kb % D;
          uint32_t p[16];
#pragma unroll
          for (int s = 0; s < D; ++s) {
            if (s == slot) {
              ablock_pairs<FMT>(buf[s], e112, p);
              if (kb + D < KB) load_ablock<FMT>(a, tb0 + kb + D, lane, buf[s]);
            }
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 av = {p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]};
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              const u32x4 bv = *reinterpret_cast<const u32x4*>(
                  &s_x[b][(16 * cc + r16) * kXPitch + kTileCols * qb + 32 * g + 8 * t]);
              acc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, bv), acc[cc],
                                                               0, 0, 0);
            }
          }
        }
        ++kb;
      }
      if (c + 1 < nch) {
        __syncthreads();
        store_x(b ^ 1);
        if (c + 2 < nch) load_x(c + 2);
        __syncthreads();
      }
    }

    if (!valid) continue;
    float q[NT][4];
#pragma unroll
    for (int cc = 0; cc < NT; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) q[cc][r] = 0.0f;
    if constexpr (FMT != kFmtBF16) {
      // Escapes of rows 4g..4g+3, kEscBatch at a time (their x loads are issued together).  The
      // placeholder x * 2^-15 comes off the accumulator, the exact x * v goes to q.
      const bool in_lds = t_e1 - t_e0 <= (uint32_t)kEscCap;
      for (uint32_t e = my_e0; e < my_e1; e += kEscBatch) {
        uint32_t col[kEscBatch];
        float val[kEscBatch];
        int rr[kEscBatch];
#pragma unroll
        for (int j = 0; j < kEscBatch; ++j) {
          const uint32_t ej = e + j;
          const bool ok = ej < my_e1;
          if (in_lds) {
            col[j] = ok ? s_ecol[w][ej - t_e0] : 0u;
            val[j] = ok ? bf16_to_float(s_eval[w][ej - t_e0]) : 0.0f;
          } else {
            col[j] = ok ? a.esc_col[ej] : 0u;
            val[j] = ok ? bf16_to_float(a.esc_val[ej]) : 0.0f;
          }
          rr[j] = ok ? (int)(ej >= my_b1) + (int)(ej >= my_b2) + (int)(ej >= my_b3) : -1;
        }
#pragma unroll
        for (int cc = 0; cc < NT; ++cc) {
          const int mcol = 16 * cc + r16;
          float xv[kEscBatch];
#pragma unroll
          for (int j = 0; j < kEscBatch; ++j)
            xv[j] = (rr[j] >= 0 && mcol < a.m) ? bf16_to_float(a.x[mcol * a.ldx + col[j]]) : 0.0f;
#pragma unroll
          for (int j = 0; j < kEscBatch; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (rr[j] == r) {
                acc[cc][r] = fmaf(-xv[j], kPlaceholder, acc[cc][r]);
                q[cc][r] = fmaf(xv[j], val[j], q[cc][r]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t nrow = tile * kTileRows + 4 * g + r;
      if (nrow >= a.n) continue;
      float sc = 1.0f;
      if constexpr (FMT != kFmtBF16) sc = window_scale(a.base[nrow]);
#pragma unroll
      for (int cc = 0; cc < NT; ++cc) {
        const int mcol = 16 * cc + r16;
        if (mcol >= a.m) continue;
        const float v = FMT != kFmtBF16 ? fmaf(sc, acc[cc][r], q[cc][r]) : acc[cc][r];
        a.y[mcol * a.ldy + nrow] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
typedef void (*MfmaKernel)(MfmaArgs);

// Blocks of A in flight per wave: fewer when more activation tiles (or the 4-word dense bf16
// blocks of the baseline) need registers.
template <int FMT>
static MfmaKernel pick(int nt) {
  constexpr int D2 = 3;
  switch (nt) {
    case 1: return k_mfma<FMT, 1, 4>;
    case 2: return k_mfma<FMT, 2, D2>;
    case 3: return k_mfma<FMT, 3, 3>;
    default: return k_mfma<FMT, 4, 3>;
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
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  for (int64_t m0 = 0; m0 < m; m0 += 64) {
    const int mb = (int)((m - m0) < 64 ? (m - m0) : 64);
    const int nt = (mb + 15) / 16;
    MfmaKernel kern = pick_kernel(f, nt);
    int occ = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern), kBlock, 0);
    if (err != hipSuccess) return err;
    if (occ < 1) occ = 1;
    int64_t blocks = (tiles + 3) / 4;
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
