// Skinny GEMM for 1..8 activation rows: y[m][n] = sum_k x[m][k] * W[n][k].
//
// The W12 planes are turned back into bfloat16 inside the kernel's registers, never through
// memory (SpecPilot, arXiv 2611.02501, figure-captions page, Fig. 5(b)).  Here the decoded pairs
// feed v_dot2_f32_bf16 rather than a matrix-unit operand: with this few rows of x the product is
// a bandwidth-bound matrix-vector stream, not a dense contraction.  Rows are summed across lanes
// with two cross-lane shuffles.
//
// Work split: persistent workgroups of 4 waves.  A workgroup copies its k-slice of x into LDS
// once.  A wave owns one 16-row tile of the tiled plane storage (see w12_device.hpp) at a time
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
#include "w12_device.hpp"
#include "w12_launch.hpp"

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
// CU-streaming kernel for 1..16 rows of x on shapes with several tiles per CU
// ---------------------------------------------------------------------------------------------
// One workgroup of kSW waves per CU.  Workgroup c owns tiles c, c + G, c + 2G, ... (G workgroups):
// T tiles of nkb 128-column blocks.  The blocks are taken in `nph` k phases of kbp = nkb / nph
// blocks; in each phase the workgroup's T kbp (tile, block) units are split into kSW contiguous
// ranges of equal length (to one unit), the same ranges of tiles in every phase, so every wave of
// the chip streams the same number of bytes and none waits on another inside a phase.  The x
// columns of the phase stay in LDS for the phase (rows one bank apart); a phase change is two
// barriers and a reload of x, while the weight ring of every wave keeps streaming the next
// phase's first blocks.  A wave's range crosses at most kSMaxSlots tiles; at every tile boundary
// it adds the partial sums of the tile's 16 rows into LDS (one slot per wave and tile, written
// only by that wave).  At the end of each phase, wave w patches the escapes of the phase's columns
// for the tiles it finalises (w, w + kSW, ...: entries prefetched at the start), and after one
// last barrier it adds the tile's partial sums in wave order (deterministic), applies the escapes
// and the scale and stores y.  1-2 rows: dot2 (lane r16 + 16 g computes row r16 over columns
// 32 g .. +31); 3-16 rows: the B operand of v_mfma_f32_16x16x32_bf16 (x rows past m are zero).
// In the final pass lane r16 + 16 g owns the outputs of x rows g, g + 4, ...
constexpr int kSW = 16;         // waves per workgroup
constexpr int kSMaxSlots = 4;   // tiles one wave's range may touch (the launcher checks)

struct StreamArgs {
  const uint16_t* x;      // x[m][k]
  const uint8_t* base;
  const uint8_t* ae;
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc_col;
  const uint16_t* esc_val;
  const uint16_t* w;
  const float* scale;
  float* y;               // y[m][ldy] (or y16)
  uint16_t* y16;
  int64_t ldy;
  int64_t n, k;
  int nph;                // k phases (nkb % nph == 0)
};

template <int FMT>
__device__ __forceinline__ TileRsrc<FMT> stream_rsrc(const StreamArgs& a, int64_t tile, bool valid,
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

// SFIN: tiles one wave finalises at most (T <= kSW SFIN)
template <int FMT, int M, int D, int SFIN>
__global__ __launch_bounds__(64 * kSW) void k_stream(StreamArgs a) {
  constexpr bool kMF = M > 2;                       // matrix cores for 3..16 rows
  constexpr bool kEsc = FMT != kFmtBF16;
  constexpr int MQ = (M + 3) / 4;                   // x rows a lane finalises: g, g + 4, ...
  extern __shared__ u32x4 xs[];                    // x row m of the phase at word m * kxrow
  __shared__ float s_part[kSW][kSMaxSlots][kTileRows][M];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const uint32_t lane16 = 16u * lane;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t G = gridDim.x, c = blockIdx.x;
  const int64_t tiles = (a.n + kTileRows - 1) / kTileRows;
  const uint32_t nkb = (uint32_t)(a.k / kTileCols);
  const int nph = a.nph;
  const uint32_t kbp = nkb / (uint32_t)nph;        // blocks per phase
  const int T = (int)((tiles - c + G - 1) / G);   // tiles c + j G, j < T (the grid keeps c < tiles)
  const uint32_t U = (uint32_t)T * kbp;            // units per phase
  const auto range_start = [&](int wv) { return (uint32_t)(((uint64_t)wv * U) / kSW); };
  const uint32_t u0 = range_start(w), u1 = range_start(w + 1), L = u1 - u0;
  const uint32_t s0 = u0 / kbp, k0l = u0 - s0 * kbp;   // first slot and its first block (in the phase)
  const int kxrow = (int)(kbp * 16) + 1;           // 16-byte words per x row of a phase in LDS
  const uint16_t* xs16 = reinterpret_cast<const uint16_t*>(xs);
  const uint32_t e112 = exp112_pair();

  // ---- the tiles this wave finalises: bounds and scale of the lane's row, prefetched first ----
  uint32_t fe0[SFIN], fe1[SFIN], fte0[SFIN], fsc[SFIN];
#pragma unroll
  for (int q = 0; q < SFIN; ++q) {
    const int j = w + kSW * q;
    const bool use = kEsc && j < T;
    const int64_t t = c + (int64_t)j * G;
    const int64_t r = use ? t * kTileRows + r16 : 0;
    const int64_t rr = r < a.n ? r : a.n;
    fe0[q] = use ? a.esc_ptr[rr] : 0u;
    fe1[q] = use ? a.esc_ptr[r + 1 < a.n ? r + 1 : a.n] : 0u;
    fte0[q] = use ? a.esc_ptr[t * kTileRows] : 0u;
    if constexpr (FMT == kFmtI8) fsc[q] = use ? __float_as_uint(a.scale[rr < a.n ? rr : a.n - 1]) : 0u;
    else if constexpr (kEsc) fsc[q] = use ? a.base[rr < a.n ? rr : a.n - 1] : 0u;
    else fsc[q] = 0u;
  }

  // ---- x of phase 0 into LDS: loads first, then the ring, then the LDS writes ----
  const int xw = (int)(kbp * 16);                  // 16-byte words of one x row per phase
  const Rsrc r_x = make_rsrc(a.x, (uint32_t)(M * a.k * 2));
  const auto x_word = [&](int ph, int i) {          // global offset of word i of the phase's x
    const int m = i / xw, j = i - m * xw;
    return i < M * xw ? (uint32_t)(2 * (m * a.k + (int64_t)ph * kbp * kTileCols + 8 * j)) : kOOB;
  };
  constexpr int kXF = 4;
  u32x4 xv[kXF];
#pragma unroll
  for (int q = 0; q < kXF; ++q)
    xv[q] = __builtin_amdgcn_raw_buffer_load_b128(r_x, x_word(0, tid + q * 64 * kSW), 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // the refill cursor: phase rp, slot rs, block rk (in the phase), position ri in the range
  uint32_t rp = 0, rs = s0, rk = k0l, ri = 0;
  const auto next_unit = [&](uint32_t& p_, uint32_t& s_, uint32_t& k_, uint32_t& i_) {
    k_ += 1;
    i_ += 1;
    const bool wrap = k_ == kbp;
    k_ = wrap ? 0u : k_;
    s_ = wrap ? s_ + 1 : s_;
    const bool pend = i_ == L;                       // the range ends: the next phase's range
    p_ = pend ? p_ + 1 : p_;
    s_ = pend ? s0 : s_;
    k_ = pend ? k0l : k_;
    i_ = pend ? 0u : i_;
  };
  const auto load_unit = [&](BlockRegs<FMT>& r) {
    const bool have = rp < (uint32_t)nph && L > 0;
    load_block<FMT>(stream_rsrc<FMT>(a, c + (int64_t)rs * G, have, nkb), have ? rp * kbp + rk : ~0u,
                    lane16, r);
    next_unit(rp, rs, rk, ri);
  };
  BlockRegs<FMT> buf[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_unit(buf[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < kXF; ++q) {
    const int i = tid + q * 64 * kSW, m = i / xw, j = i - m * xw;
    if (i < M * xw) xs[m * kxrow + j] = xv[q];
  }
  for (int i = tid + kXF * 64 * kSW; i < M * xw; i += 64 * kSW) {
    const int m = i / xw, j = i - m * xw;
    xs[m * kxrow + j] = __builtin_amdgcn_raw_buffer_load_b128(r_x, x_word(0, i), 0, 0);
  }
  lds_barrier();

  // ---- escape entries of the tiles to finalise (their bounds arrived before the first block) ----
  uint32_t ecol[SFIN][kEscPre], evalv[SFIN][kEscPre];
#pragma unroll
  for (int q = 0; q < SFIN; ++q) {
    const uint32_t te0 = __builtin_amdgcn_readfirstlane(fte0[q]);
    const Rsrc rc = make_rsrc(a.esc_col + te0, 0x7FFFFFF0u), rv = make_rsrc(a.esc_val + te0, 0x7FFFFFF0u);
#pragma unroll
    for (int i = 0; i < kEscPre; ++i) {
      const uint32_t e = fe0[q] + g + 4 * i;
      const bool in = kEsc && e < fe1[q];
      ecol[q][i] = __builtin_amdgcn_raw_buffer_load_b32(rc, in ? 4u * (e - te0) : kOOB, 0, 0);
      evalv[q][i] = __builtin_amdgcn_raw_buffer_load_b16(rv, in ? 2u * (e - te0) : kOOB, 0, 0);
    }
  }
  // escape corrections of the finalised tiles, over the phases: dP (placeholders) and Q (values)
  float dP[SFIN][MQ], Qe[SFIN][MQ];
#pragma unroll
  for (int q = 0; q < SFIN; ++q)
#pragma unroll
    for (int i = 0; i < MQ; ++i) dP[q][i] = Qe[q][i] = 0.0f;
  // the escapes of row r16 of each finalised tile whose column lies in phase ph: every lane of the
  // row takes all of them (the prefetched entries of its three row-mates through shuffles) for its
  // own x rows g + 4 i, x from the phase's LDS copy
  const auto phase_escapes = [&](int ph) {
    if constexpr (kEsc) {
      const uint32_t c0 = (uint32_t)ph * kbp * kTileCols, c1 = c0 + kbp * kTileCols;
#pragma unroll
      for (int q = 0; q < SFIN; ++q) {
        const auto patch = [&](uint32_t col, uint32_t vbits) {
          if (col < c0 || col >= c1) return;
          const float v = bf16_to_float(vbits);
#pragma unroll
          for (int i = 0; i < MQ; ++i) {
            const int m = g + 4 * i;
            if (m >= M) continue;
            const float xv = bf16_to_float(xs16[(int64_t)m * kxrow * 8 + (col - c0)]);
            if constexpr (has_placeholder<FMT>()) dP[q][i] = fmaf(-xv, placeholder_of<FMT>(), dP[q][i]);
            Qe[q][i] = fmaf(xv, v, Qe[q][i]);
          }
        };
#pragma unroll
        for (int sg = 0; sg < 4; ++sg)
#pragma unroll
          for (int i = 0; i < kEscPre; ++i) {
            const uint32_t col = (uint32_t)__shfl((int)ecol[q][i], r16 + 16 * sg, 64);
            const uint32_t vb = (uint32_t)__shfl((int)evalv[q][i], r16 + 16 * sg, 64);
            if (fe0[q] + (uint32_t)sg + 4 * i < fe1[q]) patch(col, vb);
          }
        for (uint32_t e = fe0[q] + 4 * kEscPre; e < fe1[q]; ++e) patch(a.esc_col[e], a.esc_val[e]);
      }
    }
  };

  // ---- the wave's ranges: ring of D blocks, partial sums added into LDS at every tile boundary ----
  float acc[kMF ? 4 : M];
#pragma unroll
  for (int i = 0; i < (kMF ? 4 : M); ++i) acc[i] = 0.0f;
  uint32_t cp = 0, cs = s0, ck = k0l, ci = 0;       // consumption cursor
  const auto flush = [&]() {
    const int i = (int)(cs - s0);
    const bool first = cp == 0;
    if constexpr (kMF) {
      if (r16 < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float& dst = s_part[w][i][4 * g + r][r16];
          dst = first ? acc[r] : dst + acc[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = 0.0f;
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = group_sum(acc[m]);
        if (g == m) {
          float& dst = s_part[w][i][r16][m];
          dst = first ? v : dst + v;
        }
        acc[m] = 0.0f;
      }
    }
  };
  const uint32_t steps = L * (uint32_t)nph;
  for (uint32_t ib = 0; ib < steps; ib += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const uint32_t it = ib + d;
      uint32_t p[16];
      block_pairs<FMT>(buf[d], e112, p);
      if constexpr (FMT != kFmtBF16) pin16(p);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (FMT != kFmtBF16) load_unit(buf[d]);
      if (it < steps) {
        if constexpr (kMF) {
          floatx4 acc4 = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 av = {p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]};
            const u32x4 bv = r16 < M ? xs[r16 * kxrow + (kTileCols * ck + 32 * g + 8 * t) / 8]
                                     : (u32x4){0u, 0u, 0u, 0u};
            acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, bv), acc4, 0, 0, 0);
          }
          acc[0] = acc4[0]; acc[1] = acc4[1]; acc[2] = acc4[2]; acc[3] = acc4[3];
        } else {
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const u32x4* xr = xs + m * kxrow + (kTileCols * ck + 32 * g) / 8;
            const u32x4 x0 = xr[0], x1 = xr[1], x2 = xr[2], x3 = xr[3];
            float sa = acc[m];
            sa = dot2_bf16(p[0], x0.x, sa);  sa = dot2_bf16(p[1], x0.y, sa);
            sa = dot2_bf16(p[2], x0.z, sa);  sa = dot2_bf16(p[3], x0.w, sa);
            sa = dot2_bf16(p[4], x1.x, sa);  sa = dot2_bf16(p[5], x1.y, sa);
            sa = dot2_bf16(p[6], x1.z, sa);  sa = dot2_bf16(p[7], x1.w, sa);
            sa = dot2_bf16(p[8], x2.x, sa);  sa = dot2_bf16(p[9], x2.y, sa);
            sa = dot2_bf16(p[10], x2.z, sa); sa = dot2_bf16(p[11], x2.w, sa);
            sa = dot2_bf16(p[12], x3.x, sa); sa = dot2_bf16(p[13], x3.y, sa);
            sa = dot2_bf16(p[14], x3.z, sa); sa = dot2_bf16(p[15], x3.w, sa);
            acc[m] = sa;
          }
        }
        if (ck + 1 == kbp || ci + 1 == L) flush();
        const uint32_t cph = cp;
        next_unit(cp, cs, ck, ci);
        if (cp != cph) {
          // end of the phase: its escapes, then the next phase's x (the ring keeps streaming)
          phase_escapes((int)cph);
          if (cp < (uint32_t)nph) {
            lds_barrier();
            for (int i = tid; i < M * xw; i += 64 * kSW) {
              const int m = i / xw, j = i - m * xw;
              xs[m * kxrow + j] = __builtin_amdgcn_raw_buffer_load_b128(r_x, x_word((int)cp, i), 0, 0);
            }
            lds_barrier();
          }
        }
      }
      if constexpr (FMT == kFmtBF16) load_unit(buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // a wave with an empty range (fewer units than waves: then one phase) still patches the escapes
  // of the tiles it finalises
  if (L == 0) phase_escapes(0);
  lds_barrier();

  // ---- finalise tiles w, w + kSW, ...: partial sums in wave order, escapes, scale, store ----
  const auto wave_of = [&](uint32_t unit) {        // the wave whose range holds `unit`
    return (int)(((uint64_t)kSW * (unit + 1) + U - 1) / U) - 1;
  };
#pragma unroll
  for (int q = 0; q < SFIN; ++q) {
    const int j = w + kSW * q;
    if (j >= T) break;
    const int64_t tile = c + (int64_t)j * G;
    const int64_t row = tile * kTileRows + r16;
    const int wf = wave_of((uint32_t)j * kbp), wl = wave_of((uint32_t)j * kbp + kbp - 1);
    float P[MQ];
#pragma unroll
    for (int i = 0; i < MQ; ++i) P[i] = 0.0f;
    for (int wv = wf; wv <= wl; ++wv) {
      if (range_start(wv) == range_start(wv + 1)) continue;   // an empty range (U < kSW)
      const int si = j - (int)(range_start(wv) / kbp);
#pragma unroll
      for (int i = 0; i < MQ; ++i)
        if (g + 4 * i < M) P[i] += s_part[wv][si][r16][g + 4 * i];
    }
    float sc = 1.0f;
    if constexpr (FMT == kFmtI8) sc = __uint_as_float(fsc[q]);
    else if constexpr (kEsc) sc = window_scale(fsc[q]);
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      const int m = g + 4 * i;
      if (m >= M || row >= a.n) continue;
      const float v = kEsc ? fmaf(sc, P[i] + dP[q][i], Qe[q][i]) : P[i];
      if (a.y16) a.y16[m * a.ldy + row] = float_to_bf16_rne(v);
      else a.y[m * a.ldy + row] = v;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
typedef void (*GemvKernel)(GemvArgs);

// Blocks in flight per wave (D), k-split per tile (KS) and waves per workgroup (NW), by rows of
// x: 1-2 rows split the blocks of a tile over all kNWSmall waves of the workgroup (more waves in
// flight per tile), 3-4 over 2 of 4, 5-8 keep one wave per tile.
constexpr int kNWSmall = 4;
template <int FMT, int M>
static GemvKernel pick_m() {
  if constexpr (M <= 2) return k_gemv<FMT, M, 3, kNWSmall, kNWSmall>;
  else if constexpr (M <= 4) return k_gemv<FMT, M, 4, 2, 4>;
  else return k_gemv<FMT, M, 4, 1, 4>;
}
static int ks_for(int m) { return m <= 2 ? kNWSmall : m <= 4 ? 2 : 1; }
static int nw_for(int m) { return m <= 2 ? kNWSmall : 4; }

template <int FMT>
static GemvKernel pick(int m) {
  switch (m) {
    case 1: return pick_m<FMT, 1>();
    case 2: return pick_m<FMT, 2>();
    case 3: return pick_m<FMT, 3>();
    case 4: return pick_m<FMT, 4>();
    case 5: return pick_m<FMT, 5>();
    case 6: return pick_m<FMT, 6>();
    case 7: return pick_m<FMT, 7>();
    default: return pick_m<FMT, 8>();
  }
}

static GemvKernel pick_kernel(Fmt f, int m) {
  if (f == kFmtW12) return pick<kFmtW12>(m);
  if (f == kFmtQ8) return pick<kFmtQ8>(m);
  if (f == kFmtQ8M) return pick<kFmtQ8M>(m);
  if (f == kFmtI8) return pick<kFmtI8>(m);
  return pick<kFmtBF16>(m);
}

// ---- the CU-streaming kernel's launcher ----
typedef void (*StreamKernel)(StreamArgs);

template <int FMT, int M>
static StreamKernel stream_pick_m(int sfin) {
  return sfin == 1 ? k_stream<FMT, M, 3, 1> : k_stream<FMT, M, 3, 3>;
}

template <int FMT>
static StreamKernel stream_pick(int m, int sfin) {
  switch (m) {
    case 1: return stream_pick_m<FMT, 1>(sfin);
    case 2: return stream_pick_m<FMT, 2>(sfin);
    case 3: return stream_pick_m<FMT, 3>(sfin);
    case 4: return stream_pick_m<FMT, 4>(sfin);
    case 5: case 6: return stream_pick_m<FMT, 6>(sfin);
    case 7: case 8: return stream_pick_m<FMT, 8>(sfin);
    case 9: case 10: case 11: case 12: return stream_pick_m<FMT, 12>(sfin);
    default: return stream_pick_m<FMT, 16>(sfin);
  }
}

static StreamKernel stream_kernel(Fmt f, int m, int sfin) {
  if (f == kFmtW12) return stream_pick<kFmtW12>(m, sfin);
  if (f == kFmtQ8) return stream_pick<kFmtQ8>(m, sfin);
  if (f == kFmtQ8M) return stream_pick<kFmtQ8M>(m, sfin);
  if (f == kFmtI8) return stream_pick<kFmtI8>(m, sfin);
  return stream_pick<kFmtBF16>(m, sfin);
}

// rows of x the kernel instance for mb rows is compiled for (x rows past mb read zeros)
static int stream_rows(int mb) {
  return mb <= 4 ? mb : mb <= 6 ? 6 : mb <= 8 ? 8 : mb <= 12 ? 12 : 16;
}

// k phases for mb rows: the fewest that divide the row's blocks and let one phase of x and the
// partial sums fit the LDS; a phase change needs every wave busy in each phase (0: none fits)
static int stream_phases(const DevInfo& di, int mb, int64_t k, int64_t tiles_min) {
  const int64_t nkb = k / kTileCols;
  const int rows = stream_rows(mb);
  const int64_t part = (int64_t)kSW * kSMaxSlots * kTileRows * rows * 4;
  for (int64_t ph = 1; ph <= nkb; ++ph) {
    if (nkb % ph) continue;
    const int64_t kbp = nkb / ph;
    if (rows * (kbp * 16 + 1) * 16 + part > di.max_lds) continue;
    if (ph > 1 && tiles_min * kbp < kSW) return 0;
    return (int)ph;
  }
  return 0;
}

bool stream_fits(const DevInfo& di, int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t g = tiles < di.cus ? tiles : di.cus;
  const int mb = (int)(m < 16 ? m : 16);
  return m >= 1 && (tiles + g - 1) / g <= 3 * kSW && k * 16 * 2 < (int64_t(1) << 32) &&
         stream_phases(di, mb, k, tiles / g) > 0 && stream_phases(di, (int)((m - 1) % 16) + 1, k, tiles / g) > 0;
}

hipError_t launch_stream(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                         YOut y, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  if (!stream_fits(di, m, n, k) || y.silu) return hipErrorInvalidValue;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t g = tiles < di.cus ? tiles : di.cus;
  const int sfin = (tiles + g - 1) / g <= kSW ? 1 : 3;
  for (int64_t m0 = 0; m0 < m; m0 += 16) {
    const int mb = (int)((m - m0) < 16 ? (m - m0) : 16);
    const int rows = stream_rows(mb);
    const int nph = stream_phases(di, mb, k, tiles / g);
    StreamArgs a;
    a.x = x + m0 * k;
    a.base = p.base; a.ae = p.ae; a.lo = p.lo;
    a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
    a.w = p.w;
    a.scale = p.scale;
    const YOut yp = y + m0 * n;
    a.y = yp.f;
    a.y16 = yp.h;
    a.ldy = n;
    a.n = n; a.k = k;
    a.nph = nph;
    const int64_t kbp = k / kTileCols / nph;
    hipLaunchKernelGGL(stream_kernel(f, mb, sfin), dim3((unsigned)g), dim3(64 * kSW),
                       (size_t)(rows * (kbp * 16 + 1) * 16), s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

int64_t gemv_k_slice(const DevInfo& di, int mb) {
  // longest k range whose x copy fits the LDS budget (2*m*k <= 80 KiB: the whole row)
  const int64_t red_bytes = (int64_t)4 * mb * 64 * 4;
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
    GemvKernel kern = pick_kernel(f, mb);
    const int ks = ks_for(mb), nw = nw_for(mb);
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
    // slices: they add in float in the workspace, then a one-range reduce rounds them into y)
    int64_t groups = passes < slots ? passes : slots;
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
