// Skinny GEMM for 1..8 activation rows: y[m][n] = sum_k x[m][k] * W[n][k].
//
// The W12 planes are turned back into bfloat16 inside the kernel's registers, never through
// memory (SpecPilot, arXiv 2611.02501, figure-captions page, Fig. 5(b)).  Here the decoded pairs
// feed v_dot2_f32_bf16 rather than a matrix-unit operand: with this few rows of x the product is
// a bandwidth-bound matrix-vector stream, not a dense contraction.  Rows are summed across lanes
// with two cross-lane shuffles.
//
// Work split: workgroups of 4 waves, one per pass of tiles (a workgroup loops over several
// passes only in the split-k launch below, whose grid is the resident slots).  A workgroup copies
// its k-slice of x into LDS.  A wave owns one 16-row tile of the tiled plane storage (see
// w12_device.hpp) at a time
// and, with KS > 1, only every KS-th 128-column block of it (the KS waves of a tile are in the same
// workgroup and add their partial sums through LDS in a fixed order).  Lane l = r + 16g works on
// row r, columns 32g..32g+31 of each block: its AE (2 x 128-bit) and B (1 x 128-bit) loads are
// wave-wide 1 KiB contiguous reads.
//
// Split k: a shape with few tiles for the chip (the k and v projections of a 27B-class layer
// have 64) splits the slice into `splits` k ranges; workgroup b takes range b % splits and writes
// partial sums to its own slice of a workspace, which a second kernel adds in range order.
//
// Escapes: the part-0 wave of a tile patches them from x in LDS.  Their metadata is fetched one
// tile ahead so the patch never waits on memory: the row bounds of the wave's next tile at the
// start of a tile, that tile's first kEscPre escapes per row at its end (rows with more read the
// rest from memory).
//
// Pipeline: D blocks in flight per wave, through buffer loads whose offset is pushed past the
// range when there is nothing to load (w12_device.hpp), so the ring slots are static registers and
// each step waits only for the block it consumes.  The ring runs on across the wave's tiles: the
// last D refills of a tile already fetch the first blocks of the wave's next tile, so a tile's
// epilogue (escape patch, cross-wave sum, store) does not drain the stream.  Padding steps (when a
// wave has fewer blocks than the ring period) read zeros and skip their arithmetic.
//
// Window trick: a decoded pair is w' = w / 2^(base - 112), with the exponent field 112 + E
// (see w12_device.hpp), so the row's dot product sum_k x w' is scaled once by 2^(base - 112)
// at the end.  An escaped slot decodes to w' = 2^-15; its contribution x * 2^-15 is removed and
// x * (exact value) is added in a separate sum, so y = 2^(base-112) P + Q.
#include "block.hpp"

namespace w12 {

struct GemvArgs {
  const uint16_t* x;      // x[m][ldx] (bfloat16), the slice starts at column k0
  int64_t ldx;
  const uint8_t* base;
  const uint8_t* ae;      // tiled storage
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc_col;
  const uint16_t* esc_val;
  const uint16_t* w;      // dense bfloat16 W (baseline), tiled storage
  const float* scale;     // per-row scale of the 8-bit copy (its codes are in `ae`)
  float* y;               // y[m][ldy]; with splits > 1, range j writes y + j * ysplit
  int64_t ldy;
  int64_t n, k;           // rows of W, row length
  int64_t k0;             // first column of this launch's slice (multiple of 128)
  int kn;                 // length of one k range of the slice (multiple of 128)
  int accumulate;         // add to y instead of overwriting (second and later slices)
  int splits;             // k ranges of the slice: workgroup b takes range b % splits
  int64_t kend;           // end of the slice (the last range may be shorter)
  int64_t ysplit;         // floats between the partial outputs of consecutive ranges
  uint16_t* y16;          // set (one slice, one range): outputs as bfloat16 (nearest even) here
  int silu;               // (one slice, one range) y / y16 hold h = silu(gate) * up, [m][ldy / 2]
};

template <int FMT>
__device__ __forceinline__ TileRsrc<FMT> tile_rsrc(const GemvArgs& a, int64_t tile, bool valid,
                                                   uint32_t ktiles) {
  TileRsrc<FMT> t;
  const int64_t t0 = valid ? tile : 0;
  if constexpr (FMT == kFmtBF16) {
    t.r0 = make_rsrc(a.w + t0 * ktiles * (kTileBF / 2), valid ? ktiles * (uint32_t)kTileBF : 0u);
    t.r1 = t.r0;
  } else {
    t.r0 = make_rsrc(a.ae + t0 * ktiles * kTileAE, valid ? ktiles * (uint32_t)kTileAE : 0u);
    t.r1 = make_rsrc(a.lo + t0 * ktiles * kTileLO, valid ? ktiles * (uint32_t)kTileLO : 0u);
  }
  return t;
}

constexpr int kEscPre = 4;   // escapes per lane fetched ahead (16 per row)

template <int FMT, int M, int D, int KS, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv(GemvArgs a) {
  constexpr int kT = 64 * NW;                    // threads per workgroup (NW waves)
  extern __shared__ u32x4 xs[];                 // [M][kn / 8] in 16-byte words
  __shared__ float red[NW][M][64];               // partial sums of the KS waves of a tile
  constexpr int TPB = NW / KS;                   // tiles per workgroup pass
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const uint32_t lane16 = 16u * lane;
  // this workgroup's k range [k0, k0 + kn) and workgroup group
  const int sp = (int)(blockIdx.x % (uint32_t)a.splits);
  const int64_t grp = blockIdx.x / (uint32_t)a.splits, n_grp = gridDim.x / (uint32_t)a.splits;
  const int64_t k0 = a.k0 + (int64_t)sp * a.kn;
  const int kn = (int)(a.kend - k0 < a.kn ? a.kend - k0 : a.kn), kn8 = kn >> 3;
  float* const yout = a.y + sp * a.ysplit;

  const uint16_t* xs16 = reinterpret_cast<const uint16_t*>(xs);

  const uint32_t e112 = exp112_pair();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = w % KS, tsub = w / KS;
  const uint32_t ktiles = (uint32_t)(a.k / kTileCols);
  const int64_t tiles = (a.n + kTileRows - 1) / kTileRows;
  const int64_t passes = (tiles + TPB - 1) / TPB;
  const uint32_t kb0 = (uint32_t)(k0 / kTileCols);
  const int nblk = kn / kTileCols;
  const int mine = (nblk - part + KS - 1) / KS;  // blocks of this slice owned by this wave
  const int JP = ((nblk + KS - 1) / KS + D - 1) / D * D;   // ring steps per tile, all waves
  // block of step j (0 <= j < JP) of this wave, ~0 for a padding step
  const auto blk = [&](int j) { return j < mine ? kb0 + (uint32_t)(part + j * KS) : ~0u; };

  int64_t pass = grp;
  const auto tile_of = [&](int64_t ps) { return ps * TPB + tsub; };
  TileRsrc<FMT> cur = tile_rsrc<FMT>(a, tile_of(pass), pass < passes && tile_of(pass) < tiles, ktiles);
  int64_t npass = pass + n_grp;
  TileRsrc<FMT> nxt = tile_rsrc<FMT>(a, tile_of(npass), npass < passes && tile_of(npass) < tiles, ktiles);

  // escape metadata of a tile for this lane's row (part-0 waves only; others load nothing):
  // bounds [e0, e1) of the row, the tile's first escape te0, and entries e0 + g + 4 i
  constexpr bool kEsc = FMT != kFmtBF16;
  uint32_t ce0 = 0, ce1 = 0, ecol[kEscPre], evalv[kEscPre];   // current tile
  uint32_t ne0 = 0, ne1 = 0, nte0 = 0;                         // next tile (bounds only)
  uint32_t cbase = 0, nbase = 0;        // window bottom of the row (float bits of the 8-bit copy's scale)
  const auto esc_bounds = [&](int64_t ps, uint32_t& e0, uint32_t& e1, uint32_t& te0, uint32_t& bs) {
    const int64_t t = tile_of(ps);
    const bool use = kEsc && part == 0 && ps < passes && t < tiles;
    const int64_t r = use ? t * kTileRows + r16 : 0;
    e0 = use ? a.esc_ptr[r < a.n ? r : a.n] : 0u;
    e1 = use ? a.esc_ptr[r + 1 < a.n ? r + 1 : a.n] : 0u;
    if constexpr (FMT == kFmtI8) bs = use ? __float_as_uint(a.scale[r < a.n ? r : a.n - 1]) : 0u;
    else bs = use ? a.base[r < a.n ? r : a.n - 1] : 0u;
    te0 = use ? a.esc_ptr[t * kTileRows] : 0u;   // made uniform only when used, a tile later:
  };                                              // a uniform copy now would wait for the ring
  const auto esc_entries = [&](uint32_t e0, uint32_t e1, uint32_t te0v) {
    const uint32_t te0 = __builtin_amdgcn_readfirstlane(te0v);
    const Rsrc rc = make_rsrc(a.esc_col + te0, 0x7FFFFFF0u), rv = make_rsrc(a.esc_val + te0, 0x7FFFFFF0u);
#pragma unroll
    for (int i = 0; i < kEscPre; ++i) {
      const uint32_t e = e0 + g + 4 * i;
      ecol[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, e < e1 ? 4u * (e - te0) : kOOB, 0, 0);
      evalv[i] = __builtin_amdgcn_raw_buffer_load_b16(rv, e < e1 ? 2u * (e - te0) : kOOB, 0, 0);
    }
  };
  // x first (loads complete in issue order: x queued behind the weight stream would hold the
  // workgroup's first barrier until the first blocks arrived), then the first tile's escape
  // bounds (so the escape entries, whose addresses need them, can go out right after the
  // barrier without waiting for the weight stream), then the weight stream.  The first kXF words
  // per thread cover x of every shape with 2 m kn <= 16 KiB; the rest (long rows) is copied
  // after.
  constexpr int kXF = 4;
  const Rsrc r_x = make_rsrc(a.x, (uint32_t)(M * a.ldx * 2));
  u32x4 xv[kXF];
#pragma unroll
  for (int q = 0; q < kXF; ++q) {
    const int i = tid + q * kT, m = i / kn8, j = i - m * kn8;
    xv[q] = __builtin_amdgcn_raw_buffer_load_b128(
        r_x, i < M * kn8 ? (uint32_t)(2 * (m * a.ldx + k0 + 8 * j)) : kOOB, 0, 0);
  }
  uint32_t te0 = 0;
  if constexpr (kEsc) esc_bounds(pass, ce0, ce1, te0, cbase);
  __builtin_amdgcn_sched_barrier(0);
  BlockRegs<FMT> buf[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_block<FMT>(cur, blk(d), lane16, buf[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < kXF; ++q) {
    const int i = tid + q * kT;
    if (i < M * kn8) xs[i] = xv[q];
  }
  for (int i = tid + kXF * kT; i < M * kn8; i += kT) {
    const int m = i / kn8, j = i - m * kn8;
    xs[i] = *reinterpret_cast<const u32x4*>(a.x + m * a.ldx + k0 + 8 * j);
  }
  lds_barrier();
  if constexpr (kEsc) esc_entries(ce0, ce1, te0);

  for (; pass < passes; pass += n_grp) {
    const int64_t tile = tile_of(pass);
    const bool valid = tile < tiles;
    if constexpr (kEsc) esc_bounds(pass + n_grp, ne0, ne1, nte0, nbase);

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;

    // do-while: at least one body runs, so its first wait also covers the older escape loads
    // and the epilogue needs no wait of its own
    int j0 = 0;
    do {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int j = j0 + d;
        uint32_t p[16];
        block_pairs<FMT>(buf[d], e112, p);
        if constexpr (FMT != kFmtBF16) pin16(p);
        __builtin_amdgcn_sched_barrier(0);
        // refill: step j + D of this tile, or of the wave's next tile (dense blocks are their own
        // operands: refilled after the arithmetic below)
        const auto refill = [&]() {
          const bool here = j + D < JP;
          TileRsrc<FMT> t;
          t.r0 = here ? cur.r0 : nxt.r0;
          t.r1 = here ? cur.r1 : nxt.r1;
          load_block<FMT>(t, blk(here ? j + D : j + D - JP), lane16, buf[d]);
        };
        if constexpr (FMT != kFmtBF16) refill();
        if (j < mine) {
          const int kb = part + j * KS;          // block within the slice
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const u32x4* xr = xs + m * kn8 + (kTileCols * kb + 32 * g) / 8;
            const u32x4 x0 = xr[0], x1 = xr[1], x2 = xr[2], x3 = xr[3];
            float s = acc[m];
            s = dot2_bf16(p[0], x0.x, s);  s = dot2_bf16(p[1], x0.y, s);
            s = dot2_bf16(p[2], x0.z, s);  s = dot2_bf16(p[3], x0.w, s);
            s = dot2_bf16(p[4], x1.x, s);  s = dot2_bf16(p[5], x1.y, s);
            s = dot2_bf16(p[6], x1.z, s);  s = dot2_bf16(p[7], x1.w, s);
            s = dot2_bf16(p[8], x2.x, s);  s = dot2_bf16(p[9], x2.y, s);
            s = dot2_bf16(p[10], x2.z, s); s = dot2_bf16(p[11], x2.w, s);
            s = dot2_bf16(p[12], x3.x, s); s = dot2_bf16(p[13], x3.y, s);
            s = dot2_bf16(p[14], x3.z, s); s = dot2_bf16(p[15], x3.w, s);
            acc[m] = s;
          }
        }
        if constexpr (FMT == kFmtBF16) refill();
        __builtin_amdgcn_sched_barrier(0);
      }
      j0 += D;
    } while (j0 < JP);
    cur = nxt;
    npass += n_grp;
    nxt = tile_rsrc<FMT>(a, tile_of(npass), npass < passes && tile_of(npass) < tiles, ktiles);

    const int64_t row = tile * kTileRows + r16;
    float q[M];
#pragma unroll
    for (int m = 0; m < M; ++m) q[m] = 0.0f;
    if constexpr (kEsc) {
      // Escapes of this lane's row inside the slice (part-0 wave; the 4 column-group lanes of the
      // row share the list): remove the placeholder from P, collect Q = sum x * v.
      const auto patch = [&](uint32_t col, uint32_t vbits) {
        const int64_t c = (int64_t)col - k0;
        if (c >= 0 && c < kn) {
          const float v = bf16_to_float(vbits);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float xv = bf16_to_float(xs16[m * kn + c]);
            if constexpr (has_placeholder<FMT>()) acc[m] = fmaf(-xv, placeholder_of<FMT>(), acc[m]);
            q[m] = fmaf(xv, v, q[m]);
          }
        }
      };
#pragma unroll
      for (int i = 0; i < kEscPre; ++i)
        if (ce0 + g + 4 * i < ce1) patch(ecol[i], evalv[i]);
      for (uint32_t e = ce0 + g + 4 * kEscPre; e < ce1; e += 4) patch(a.esc_col[e], a.esc_val[e]);
#pragma unroll
      for (int m = 0; m < M; ++m) q[m] = group_sum(q[m]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = group_sum(acc[m]);

    if constexpr (KS > 1) {
#pragma unroll
      for (int m = 0; m < M; ++m) red[w][m][lane] = acc[m];
      lds_barrier();
      if (part == 0) {
#pragma unroll
        for (int pp = 1; pp < KS; ++pp)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[m] += red[w + pp][m][lane];
      }
      lds_barrier();
    }

    if (a.silu && part == 0 && valid) {
      // SiLU(gate) * up: rows r16 < 8 of the tile are gate rows, r16 + 8 the matching up rows
      // (lane ^ 8 of the same wave); h [m][ldy / 2] gets 8 outputs per tile
      float sc = 1.0f;
      if constexpr (FMT == kFmtI8) sc = __uint_as_float(cbase);
      else if constexpr (FMT != kFmtBF16) sc = window_scale(cbase);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = FMT != kFmtBF16 ? fmaf(sc, acc[m], q[m]) : acc[m];
        const float up = __shfl_xor(v, 8);
        if (g == 0 && r16 < 8) {
          const float hv = silu(v) * up;
          const int64_t at = m * (a.ldy >> 1) + tile * 8 + r16;
          if (a.y16) a.y16[at] = float_to_bf16_rne(hv);
          else yout[at] = hv;
        }
      }
    } else if (part == 0 && valid && g == 0 && row < a.n) {
      float sc = 1.0f;
      if constexpr (FMT == kFmtI8) sc = __uint_as_float(cbase);
      else if constexpr (FMT != kFmtBF16) sc = window_scale(cbase);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = FMT != kFmtBF16 ? fmaf(sc, acc[m], q[m]) : acc[m];
        if (a.y16) {
          a.y16[m * a.ldy + row] = float_to_bf16_rne(v);
          continue;
        }
        float* yp = yout + m * a.ldy + row;
        // later k-slices add to y; the read stays in its branch (a hoisted read would make every
        // tile wait for the whole stream in flight)
        if (a.accumulate) *yp = *reinterpret_cast<volatile float*>(yp) + v;
        else *yp = v;
      }
    }
    if constexpr (kEsc) {
      // the next tile's entries and window bottoms (its bounds arrived during this tile)
      ce0 = ne0;
      ce1 = ne1;
      cbase = nbase;
      esc_entries(ne0, ne1, nte0);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
typedef void (*GemvKernel)(GemvArgs);

// Blocks in flight per wave (D), k-split per tile (KS) and waves per workgroup (NW), by rows of
// x: 1-2 rows split the blocks of a tile over all waves of the workgroup (more waves in flight
// per tile), 3-4 over 2 of 4, 5-8 keep one wave per tile.
constexpr int kNWSmall = 4;
// Shapes of at most one tile per CU at 1-2 rows (a layer's k and v projections): 8 waves per
// tile, so the blocks in flight per tile double (us, [1024, 5120], 4 / 8 waves: W12 6.57 / 6.23
// at one row, 7.77 / 6.74 at two; Q8 6.11 / 5.43; the dense baseline 5.69 / 5.94 at one row and
// 6.64 / 6.17 at two, so it keeps 4 waves at one row).  More tiles: 8 waves lose ([5120, 5120]:
// W12 11.05 / 11.86 us).
constexpr int kNWFew = 8;
static bool few_tiles(Fmt f, int m, int64_t tiles, const DevInfo& di) {
  return m <= 2 && tiles <= di.cus && (f != kFmtBF16 || m == 2);
}
template <int FMT, int M>
static GemvKernel pick_m(bool few) {
  if constexpr (M <= 2) return few ? k_gemv<FMT, M, 3, kNWFew, kNWFew> : k_gemv<FMT, M, 3, kNWSmall, kNWSmall>;
  else if constexpr (M <= 4) return k_gemv<FMT, M, 4, 2, 4>;
  else return k_gemv<FMT, M, 4, 1, 4>;
}
static int ks_for(int m, bool few) { return m <= 2 ? (few ? kNWFew : kNWSmall) : m <= 4 ? 2 : 1; }
static int nw_for(int m, bool few) { return m <= 2 ? (few ? kNWFew : kNWSmall) : 4; }

template <int FMT>
static GemvKernel pick(int m, bool few) {
  switch (m) {
    case 1: return pick_m<FMT, 1>(few);
    case 2: return pick_m<FMT, 2>(few);
    case 3: return pick_m<FMT, 3>(few);
    case 4: return pick_m<FMT, 4>(few);
    case 5: return pick_m<FMT, 5>(few);
    case 6: return pick_m<FMT, 6>(few);
    case 7: return pick_m<FMT, 7>(few);
    default: return pick_m<FMT, 8>(few);
  }
}

static GemvKernel pick_kernel(Fmt f, int m, bool few) {
  if (f == kFmtW12) return pick<kFmtW12>(m, few);
  if (f == kFmtQ8) return pick<kFmtQ8>(m, few);
  if (f == kFmtQ8M) return pick<kFmtQ8M>(m, few);
  if (f == kFmtI8) return pick<kFmtI8>(m, few);
  return pick<kFmtBF16>(m, few);
}

int64_t gemv_k_slice(const DevInfo& di, int mb) {
  // longest k range whose x copy fits the LDS budget (2*m*k <= 80 KiB: the whole row)
  const int64_t red_bytes = (int64_t)kNWFew * mb * 64 * 4;
  int64_t budget = 81920;
  if (budget > di.max_lds - red_bytes) budget = di.max_lds - red_bytes;
  int64_t slice = (budget / (2 * mb)) / kTileCols * kTileCols;
  return slice < kTileCols ? kTileCols : slice;
}

hipError_t launch_gemv(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                       YOut y, hipStream_t s, const Scratch& sc) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t nkb = k / kTileCols;
  for (int64_t m0 = 0; m0 < m; m0 += 8) {
    const int mb = (int)((m - m0) < 8 ? (m - m0) : 8);
    const bool few = few_tiles(f, mb, tiles, di);
    GemvKernel kern = pick_kernel(f, mb, few);
    const int ks = ks_for(mb, few), nw = nw_for(mb, few);
    const int64_t tpb = nw / ks;
    const int64_t passes = (tiles + tpb - 1) / tpb;
    int64_t slice = gemv_k_slice(di, mb);
    if (slice > k) slice = k;
    int occ = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern),
                                                       64 * nw, (size_t)2 * mb * slice);
    if (err != hipSuccess) return err;
    if (occ < 1) occ = 1;
    const int64_t slots = (int64_t)di.cus * occ;
    // k ranges in one launch: when the shape has few tiles and long rows (more than 16 blocks per
    // wave of a tile), as many as keep every workgroup slot busy, with at least two blocks per
    // wave in each; at least as many as the LDS needs; their partial outputs must fit the
    // workspace.  (On shorter rows -- the k and v projections included -- the second kernel
    // costs more than the ranges gain.)
    int64_t ranges = nkb / ks > 16 ? slots / passes : 1;
    if (ranges > nkb / (2 * ks)) ranges = nkb / (2 * ks);
    const int64_t need = (k + slice - 1) / slice;
    if (ranges < need) ranges = need;
    int64_t rlen = (nkb + ranges - 1) / ranges * kTileCols;
    if (rlen > slice) rlen = slice;
    ranges = (k + rlen - 1) / rlen;
    float* ws = nullptr;
    if (ranges > 1 && (size_t)ranges * mb * n * sizeof(float) <= sc.bytes) {
      err = sc.get(&ws);
      if (err != hipSuccess) return err;
    }
    GemvArgs a;
    a.ldx = k;
    a.base = p.base; a.ae = p.ae; a.lo = p.lo;
    a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
    a.w = p.w;
    a.scale = p.scale;
    a.ldy = n;
    a.n = n; a.k = k;
    a.x = x + m0 * k;
    a.y16 = nullptr;
    a.silu = 0;
    if (ws) {
      // one launch over all ranges into the workspace, then the ordered sum into y
      int64_t groups = slots / ranges;
      if (groups > passes) groups = passes;
      if (groups < 1) groups = 1;
      a.y = ws;
      a.k0 = 0; a.kn = (int)rlen; a.kend = k;
      a.accumulate = 0;
      a.splits = (int)ranges;
      a.ysplit = (int64_t)mb * n;
      hipLaunchKernelGGL(kern, dim3((unsigned)(groups * ranges)), dim3(64 * nw), (size_t)2 * mb * rlen, s, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
      err = launch_split_reduce(ws, (int)ranges, mb, n, y + m0 * n, n, s);
      if (err != hipSuccess) return err;
      continue;
    }
    // one range per launch: later slices add to y in slice order (bfloat16 output over several
    // slices: they add in float in the workspace, then a one-range reduce rounds them into y).
    // One workgroup per tile pass, not a persistent grid of the resident slots: the hardware
    // starts each further workgroup on the first CU with a free slot, so CUs that finish early
    // take more tiles (gate+up [34816, 5120] at one row: 44.6 -> 43.6 us on one box, 43.0 ->
    // 42.3 on another; the LM-head-like [152064, 5120]: 173.6 -> 166.8 us).
    const int64_t groups = passes;
    const YOut yp = y + m0 * n;
    float* acc32 = nullptr;
    if ((yp.h || yp.silu) && k > slice) {
      if ((size_t)mb * n * sizeof(float) > sc.bytes) return hipErrorInvalidValue;
      err = sc.get(&acc32);
      if (err != hipSuccess) return err;
    }
    // (several slices with bfloat16 or SiLU outputs: float sums in the workspace, then a
    // one-range reduce rounds or pairs them into y)
    a.y = acc32 ? acc32 : yp.f;
    a.y16 = acc32 ? nullptr : yp.h;
    a.silu = acc32 ? 0 : (int)yp.silu;
    a.splits = 1;
    a.ysplit = 0;
    for (int64_t k0 = 0; k0 < k; k0 += slice) {
      const int kn = (int)((k - k0) < slice ? (k - k0) : slice);
      a.k0 = k0; a.kn = kn; a.kend = k0 + kn;
      a.accumulate = k0 > 0;
      hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(64 * nw), (size_t)2 * mb * kn, s, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    if (acc32) {
      err = launch_split_reduce(acc32, 1, mb, n, yp, n, s);
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace w12
