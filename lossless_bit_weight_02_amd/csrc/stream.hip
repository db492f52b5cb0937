// Streaming GEMM for 1..64 rows of x, y[m][n] = sum_k x[m][k] W[n][k], with every wave of a CU
// streaming the same number of weight blocks.
//
// One workgroup of W waves per CU (W = 16 up to 16 rows of x, 12 with 168 VGPRs and a deeper ring
// for 17..32 rows, 8 with 256 VGPRs for 33..64, whose ranges may touch three tiles).  Workgroup c
// owns the 16-row tiles c, c + G, c + 2 G, ... (G workgroups), so every CU gets the same number
// of tiles to within one.  Each wave finalises up to FT of the CU's tiles (on shapes with more
// tiles than waves on the chip FT = 3 for 3..16 rows of x and 2 for 17..64; else 1); a shape with
// more tiles than FT W per CU runs as row groups of such workgroups in one launch (workgroup b:
// group b / G).  In top-1 mode each workgroup reduces its outputs to one key per x row instead of
// storing them.
// Inside the CU the work is dealt by (tile, 128-column block) units rather than by tiles, so no
// wave idles while others stream:
//
// k phases.  x stays in LDS, but 32 rows of a 5120-column x do not fit, so the blocks run in
// `nph` phases of kbp blocks each.  In phase q the CU's T kbp units (tile-major: blocks
// q kbp .. q kbp + kbp - 1 of its T tiles) are split into W contiguous ranges, the same ranges of
// tiles in every phase; the launcher picks kbp so that the ranges are equal (or nearly: the
// busiest wave sets the phase's time).  x of phase q + 1 is loaded straight from memory into the
// second of two LDS buffers (global-to-LDS loads dealt over the waves) while phase q runs, so a
// phase change costs one barrier; the weight ring (D blocks in flight per wave) runs on across
// phases.
//
// Partial sums.  A wave's range touches at most two tiles (three at 64 rows or with FT = 2, four
// with FT = 3); it keeps one running sum per touched tile in registers over all phases and adds
// them into LDS at the end.  Tile j of the CU is then finalised by wave j % W: the partial sums of the waves that
// touch it, added in wave order (deterministic), plus its escape corrections, collected during
// each phase from x in LDS (the first 384 entries of a tile, 128 with FT > 1, copied to the
// wave's LDS slot at the start; entries past the copy are read at the end).
//
// Decode and arithmetic as in the GEMV: 1-2 rows by dot2 (lane r16 + 16 g computes row r16 over
// columns 32 g .. +31 of each block); 3-64 rows on the matrix cores, the decoded block as operand
// A of v_mfma_f32_16x16x32_bf16 (one to four 16-row activation tiles as operand B, read from LDS).
// Escapes as everywhere: y = 2^(base - 112) (P - 2^-15 sum_esc x) + sum_esc x v.
#include "block.hpp"

namespace w12 {

// escapes of a finalised tile copied to LDS (more: read at the end), with one and with two or
// three tiles finalised per wave; value slots 128 more (copied as 4-byte pairs from an even entry)
constexpr int kSECap = 384, kSECap3 = 128;
constexpr int kSPieces = 80;    // x pieces (1 KiB) per phase buffer at most

struct StreamArgs {
  const uint16_t* x;      // x [mrows][k] (this pass's rows)
  int mrows;
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
  uint32_t kbp;           // blocks per phase (kbp * nph = k / 128)
  int nph;                // phases
  uint32_t rs;            // 16-byte words per x row in LDS: 64 per 512-column segment
  uint32_t xwords;        // 16-byte words of one x buffer: MR rows of rs
  uint32_t eoff;          // 16-byte word offset of the escape copies: [W FT][cap] columns, then
                          // [W FT][cap + 128] values
  int64_t gtiles;         // 16-row tiles per row group (workgroup b takes group b / G)
  int64_t G;              // workgroups per group
  uint64_t* keys;         // top-1 mode (y not written): workgroup b's best key of x row j at
                          // keys[32 b + j], j < 32 (0 for rows past mrows and idle workgroups)
};

template <int FMT>
__device__ __forceinline__ TileRsrc<FMT> stream_rsrc(const StreamArgs& a, int64_t tile, bool valid,
                                                     uint32_t nkb) {
  TileRsrc<FMT> t;
  const int64_t t0 = valid ? tile : 0;
  if constexpr (FMT == kFmtBF16) {
    t.r0 = make_rsrc(a.w + t0 * nkb * (kTileBF / 2), valid ? nkb * (uint32_t)kTileBF : 0u);
    t.r1 = t.r0;
  } else {
    t.r0 = make_rsrc(a.ae + t0 * nkb * kTileAE, valid ? nkb * (uint32_t)kTileAE : 0u);
    t.r1 = make_rsrc(a.lo + t0 * nkb * kTileLO, valid ? nkb * (uint32_t)kTileLO : 0u);
  }
  return t;
}

// Wait until at most N vector-memory operations of this wave are outstanding (they complete in
// issue order).
template <int N>
__device__ __forceinline__ void s_vm_wait_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Wait until at most min(L, D) ring steps of kLPS loads each are outstanding (L a runtime value).
template <int D, int kLPS>
__device__ __forceinline__ void s_vm_wait_steps(uint32_t L) {
  if (L >= (uint32_t)D) s_vm_wait_le<D * kLPS>();
  else if constexpr (D > 3) {
    if (L == 3) s_vm_wait_le<3 * kLPS>();
    else if (L == 2) s_vm_wait_le<2 * kLPS>();
    else if (L == 1) s_vm_wait_le<kLPS>();
    else s_vm_wait_le<0>();
  } else {
    if (L == 2) s_vm_wait_le<2 * kLPS>();
    else if (L == 1) s_vm_wait_le<kLPS>();
    else s_vm_wait_le<0>();
  }
}

template <int W>
struct StreamShape {
  static_assert(W == 8 || W == 12 || W == 16, "8, 12 or 16 waves per workgroup");
  static constexpr int D = W == 16 ? 3 : 4;     // blocks in flight per wave
  static constexpr int FW = (kSPieces + W - 1) / W;   // x pieces a wave may load per phase
};

// MR: rows of x the instance is built for (x rows mrows .. MR - 1 read zeros).  FT: tiles a wave
// finalises at most (1: the CU has at most W tiles, whose escapes the waves walk phase by phase
// from LDS; 3: up to 3 W tiles, so a shape of up to 3 W tiles per CU needs no row groups, with
// the escapes patched at the end from memory).
template <int FMT, int MR, int W, int FT>
__global__ __launch_bounds__(64 * W) void k_stream(StreamArgs a) {
  // W12 with three tiles per wave at 8 and 16 rows: a 2-deep ring keeps the escape walk's
  // registers within the 16-wave budget (3 deep spilled; LM head [152064, 5120], 16 rows: 183.1
  // us against 198.7 in row groups of one tile per wave)
  constexpr int D = (FMT == kFmtW12 && FT == 3 && MR >= 8) ? 2 : StreamShape<W>::D;
  constexpr int FW = StreamShape<W>::FW;
  static_assert(FT == 1 || (FT == 3 && W == 16 && MR <= 16) || (FT == 2 && ((W == 8 && MR == 64) || (W == 12 && MR == 32))),
                "FT 3: up to 16 rows, 16 waves; FT 2: 64 rows, 8 waves");
  // tiles one wave's range touches at most: its length is at most FT kbp units + 1
  constexpr int SL = FT == 3 ? 4 : (MR > 32 || FT == 2) ? 3 : 2;
  constexpr bool kMF = MR > 2;                       // matrix cores for 3..64 rows
  constexpr int NT = (MR + 15) / 16;                 // 16-row activation tiles
  constexpr int NACC = kMF ? 4 * NT : MR;            // running sums per lane
  constexpr int MP = MR + 1;                         // row stride of the LDS partial sums
  constexpr bool kEsc = FMT != kFmtBF16;
  constexpr int ECAP = FT == 1 ? kSECap : kSECap3, EVAL = ECAP + 128;
  constexpr int kLPS = FMT == kFmtBF16 ? 4 : FMT == kFmtW12 ? 3 : 2;   // loads per ring step
  // LDS: x buffers [2][MR][rs] of 16-byte words; column word c16 (columns 8 c16 .. +7 of the
  // phase) of x row r sits at r * rs + (c16 & ~15) + ((c16 & 15) ^ (r & 15)): the 16 rows an
  // operand read takes then hit distinct banks.  At the end the partial sums [W][SL][16][MP]
  // over them.
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const uint32_t lane16 = 16u * lane;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // row group b / G (its tiles tb .. tb + tiles - 1), workgroup c of it
  const int64_t G = a.G, c = blockIdx.x % G, tb = (blockIdx.x / G) * a.gtiles;
  const int64_t tiles_all = (a.n + kTileRows - 1) / kTileRows;
  const int64_t tiles = tiles_all - tb < a.gtiles ? tiles_all - tb : a.gtiles;
  if (c >= tiles) {                                  // a last group with fewer tiles than G
    if (a.keys && tid < 32) a.keys[(int64_t)blockIdx.x * 32 + tid] = 0;
    return;
  }
  const uint32_t nkb = (uint32_t)(a.k / kTileCols);
  const uint32_t kbp = a.kbp;
  const int nph = a.nph;
  const int T = (int)((tiles - c + G - 1) / G);     // tiles tb + c + j G, j < T
  const uint32_t U = (uint32_t)T * kbp;              // units per phase of the CU
  const auto rstart = [&](int wv) { return (uint32_t)(((uint64_t)wv * U) / W); };
  const uint32_t r0 = rstart(w), r1 = rstart(w + 1);
  const uint32_t L = r1 - r0;                        // units per phase of this wave
  const uint32_t s0 = r0 / kbp, k0l = r0 - s0 * kbp; // the wave's first tile (local) and block
  const uint16_t* xs16 = reinterpret_cast<const uint16_t*>(lds);
  const uint32_t e112 = exp112_pair();

  // ---- the tiles this wave finalises: local tiles w + f W, f < FT ----
  // Lane layout of the finalisation: lane r16 + 16 g owns weight row r16 of each and x rows
  // xm(i) = g + 4 i (i < NX; rows past MR idle), so a lane walks the escapes of one row per tile.
  constexpr int NX = (MR + 3) / 4;
  const auto xm = [&](int i) { return g + 4 * i; };
  bool fin[FT];
  int64_t row0[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    fin[f] = w + f * W < T;
    row0[f] = (fin[f] ? tb + c + (int64_t)(w + f * W) * G : 0) * kTileRows;
  }
  // escape bounds of the lane's row r16 of tile f: entries [st[f][0], st[f][1]), and its window
  // bottom (or 8-bit scale); loaded after phase 0's x (the first barrier waits for x)
  uint32_t st[FT][2], fsc[FT];
  // tile f's escape list [te0, te1): its first ECAP entries are copied to this wave's LDS slot f
  // (loaded after the ring's first blocks, waited for before phase 0's walk)
  uint32_t fte0[FT];
  const auto load_meta = [&]() {
#pragma unroll
    for (int f = 0; f < FT; ++f) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int64_t rr = row0[f] + r16 + r;
        st[f][r] = kEsc && fin[f] ? a.esc_ptr[rr < a.n ? rr : a.n] : 0u;
      }
      const int64_t rr = row0[f] + r16, rc = rr < a.n ? rr : a.n - 1;
      if constexpr (FMT == kFmtI8) fsc[f] = fin[f] ? __float_as_uint(a.scale[rc]) : 0u;
      else if constexpr (kEsc) fsc[f] = fin[f] ? a.base[rc] : 0u;
      else fsc[f] = 0u;
      fte0[f] = kEsc && fin[f] ? a.esc_ptr[row0[f]] : 0u;
    }
  };

  // ---- x of a phase into LDS buffer `buf`: piece P = (row, 512-column segment), one coalesced
  // 1 KiB read of the row (lane j reads the column word its LDS slot holds), by wave P % W;
  // columns past the phase read zeros into the row's last segment ----
  const uint32_t rs = a.rs, segs = rs >> 6;
  const Rsrc r_x = make_rsrc(a.x, (uint32_t)(a.mrows * a.k * 2));
  const auto issue_x = [&](int ph, int buf) {
#pragma unroll
    for (int i = 0; i < FW; ++i) {
      const uint32_t P = (uint32_t)(w + W * i);
      if (P < MR * segs) {
        const uint32_t row = P / segs, sg = P - row * segs;
        const uint32_t c16 = 64u * sg + (((uint32_t)lane & ~15u) | (((uint32_t)lane & 15u) ^ (row & 15u)));
        const bool ok = c16 < kbp * 16u && (int)row < a.mrows;
        const uint32_t off = ok ? 2u * (row * (uint32_t)a.k + (uint32_t)ph * kbp * kTileCols + 8u * c16) : kOOB;
        u32x4* dst = lds + buf * a.xwords + row * rs + 64u * sg;   // lane j at word j
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_x, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
      }
    }
  };

  // ---- ring cursors: phase, tile (local), block in the phase, index in the range ----
  uint32_t rp = 0, rt = s0, rk = k0l, ri = 0;
  const auto advance = [&](uint32_t& p_, uint32_t& t_, uint32_t& k_, uint32_t& i_) {
    k_ += 1;
    i_ += 1;
    const bool wrap = k_ == kbp;
    k_ = wrap ? 0u : k_;
    t_ = wrap ? t_ + 1 : t_;
    const bool pend = i_ == L;                       // the range ends: the next phase's range
    p_ = pend ? p_ + 1 : p_;
    t_ = pend ? s0 : t_;
    k_ = pend ? k0l : k_;
    i_ = pend ? 0u : i_;
  };
  const auto load_next = [&](BlockRegs<FMT>& r) {
    const bool have = rp < (uint32_t)nph && L > 0;
    load_block<FMT>(stream_rsrc<FMT>(a, tb + c + (int64_t)rt * G, have, nkb), have ? rp * kbp + rk : ~0u, lane16, r);
    advance(rp, rt, rk, ri);
  };

  issue_x(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_meta();
  __builtin_amdgcn_sched_barrier(0);
  BlockRegs<FMT> buf[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_next(buf[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  s_vm_wait_le<D * kLPS>();                          // phase 0's x is in LDS
  lds_barrier();
  if (nph > 1) issue_x(1, 1);
  __builtin_amdgcn_sched_barrier(0);

  // ---- escape entries of the tiles to finalise (their bounds went out right after phase 0's x,
  // before the ring, so the wait for x covered them) ----
  // The copy goes straight to the wave's LDS slots with global-to-LDS loads (no registers held;
  // the first phase's escape walk waits for them): columns 64 per load, values 128 per load as
  // 4-byte pairs from the even entry at or below te0 (a 4-byte word holding one value of the list
  // lies in the same page as that value), so the value copy starts one slot early for an odd te0.
  uint32_t te0[FT], lds_end[FT];
  uint32_t* s_ecol[FT];
  uint16_t* s_eval[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    te0[f] = __builtin_amdgcn_readfirstlane(fte0[f]);
    const uint32_t tvsh = te0[f] & 1u;
    const int sl = w * FT + f;                          // this wave's slot f
    s_ecol[f] = reinterpret_cast<uint32_t*>(lds + a.eoff) + sl * ECAP;
    uint16_t* s_evalb = reinterpret_cast<uint16_t*>(lds + a.eoff + W * FT * ECAP / 4) + sl * EVAL;
    s_eval[f] = s_evalb + tvsh;                         // entry te0 + i at s_eval[f][i]
    lds_end[f] = te0[f] + ECAP;                         // entries past this stay in memory
    if (kEsc && fin[f]) {
      const uint32_t te1 = (uint32_t)__builtin_amdgcn_readlane((int)st[f][1], 15);   // row0 + 16
      const uint32_t cnt = te1 - te0[f] < (uint32_t)ECAP ? te1 - te0[f] : (uint32_t)ECAP;
      const Rsrc rc = make_rsrc(a.esc_col + te0[f], cnt * 4u);
      const Rsrc rv = make_rsrc(a.esc_val + (te0[f] - tvsh), ((cnt + tvsh) * 2u + 3u) & ~3u);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < ECAP / 64; ++i)
        if (64u * i < cnt)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)(s_ecol[f] + 64 * i), 4,
                                                   4u * (lane + 64 * i), 0, 0, 0);
#pragma unroll
      for (int i = 0; i < EVAL / 128; ++i)
        if (128u * i < cnt + tvsh)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(s_evalb + 128 * i), 4,
                                                   4u * (lane + 64 * i), 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const auto run_end = [&](int f) { return st[f][1] < lds_end[f] ? st[f][1] : lds_end[f]; };
  // escape corrections: with one tile per wave dP (placeholders) and Qe (values) apart, with three
  // Qe[f] alone, the placeholder terms scaled into it (x v - x 2^(base - 112) ph per entry); per
  // tile a cursor (absolute entry index) with the column and value under it (column ~0: none left
  // in LDS)
  float dP[FT == 1 ? NX : 1], Qe[FT][NX];
  uint32_t cur[FT], ncol[FT], nval[FT];
#pragma unroll
  for (int cc = 0; cc < (FT == 1 ? NX : 1); ++cc) dP[cc] = 0.0f;
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    cur[f] = st[f][0];
    ncol[f] = ~0u;
    nval[f] = 0u;
#pragma unroll
    for (int cc = 0; cc < NX; ++cc) Qe[f][cc] = 0.0f;
  }
  const bool xlane = g < MR;                          // the lane owns an x row
  const auto entry_at = [&](int f) {                  // the entry under tile f's cursor
    const bool in = cur[f] < run_end(f);
    const uint32_t at = in ? cur[f] - te0[f] : 0u;
    ncol[f] = in ? s_ecol[f][at] : ~0u;
    nval[f] = s_eval[f][at];
  };
  // the escapes of the lane's rows with a column in phase ph (runs are sorted by column), x from
  // the phase's LDS buffer; the reads of the x values at an entry and of the row's next entry go
  // out together.
  const auto phase_escapes = [&](int ph) {
    if constexpr (kEsc) {
      if (!fin[0]) return;
      if (ph == 0) {
        // the escape copies have landed: they went out before every refill of this phase, so
        // waiting until at most min(L, D) refills are outstanding covers them (the phase change
        // waits the same for the next phase's x)
        s_vm_wait_steps<D, kLPS>(L);
#pragma unroll
        for (int f = 0; f < FT; ++f) entry_at(f);
      }
      const uint32_t c0 = (uint32_t)ph * kbp * kTileCols, c1 = c0 + kbp * kTileCols;
      const uint16_t* xb = xs16 + (size_t)(ph & 1) * a.xwords * 8;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        float scph = 0.0f;                            // 2^(base - 112) ph (three tiles per wave)
        if constexpr (FT > 1 && has_placeholder<FMT>()) {
          if constexpr (FMT == kFmtI8) scph = __uint_as_float(fsc[f]) * placeholder_of<FMT>();
          else scph = window_scale(fsc[f]) * placeholder_of<FMT>();
        }
        while (ncol[f] < c1) {
          const uint32_t cc0 = ncol[f] - c0, c16 = cc0 >> 3;
          const float v = bf16_to_float(nval[f]);
          float xv[NX];
#pragma unroll
          for (int cc = 0; cc < NX; ++cc) {
            const int m = xm(cc) < MR ? xm(cc) : 0;
            xv[cc] = bf16_to_float(
                xb[(m * rs + (c16 & ~15u) + ((c16 & 15u) ^ (uint32_t)(m & 15))) * 8 + (cc0 & 7)]);
          }
          cur[f] += 1;
          entry_at(f);
#pragma unroll
          for (int cc = 0; cc < NX; ++cc) {
            if (!xlane || xm(cc) >= MR) continue;
            if constexpr (FT == 1) {
              if constexpr (has_placeholder<FMT>()) dP[cc] = fmaf(-xv[cc], placeholder_of<FMT>(), dP[cc]);
              Qe[f][cc] = fmaf(xv[cc], v, Qe[f][cc]);
            } else {
              Qe[f][cc] = fmaf(xv[cc], v, Qe[f][cc]);
              if constexpr (has_placeholder<FMT>()) Qe[f][cc] = fmaf(-xv[cc], scph, Qe[f][cc]);
            }
          }
        }
      }
    }
  };
  // end of phase ph: its escapes; then (not the last phase) wait for the next phase's x, the
  // barrier that publishes it and frees buffer ph & 1, and the loads of phase ph + 2 into it.
  // The next phase's x went out before the L ring refills of this phase, and loads complete in
  // issue order, so waiting until at most min(L, D) refills are outstanding waits for it.
  const auto phase_end = [&](int ph) {
    __builtin_amdgcn_sched_barrier(0);
    phase_escapes(ph);
    if (ph + 1 < nph) {
      __builtin_amdgcn_sched_barrier(0);
      s_vm_wait_steps<D, kLPS>(L);
      lds_barrier();
      if (ph + 2 < nph) issue_x(ph + 2, ph & 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the wave's ranges: ring of D blocks; a running sum per touched tile ----
  float acc[NACC], tot[SL][NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) {
    acc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < SL; ++s) tot[s][i] = 0.0f;
  }
  uint32_t cp = 0, ct = s0, ck = k0l, ci = 0;       // consumption cursor
  const auto flush = [&]() {
    const uint32_t slot = ct - s0;
    // every slot takes acc or 0 (a select per element, so the slots stay in registers)
#pragma unroll
    for (int s = 0; s < SL; ++s)
#pragma unroll
      for (int i = 0; i < NACC; ++i) tot[s][i] += slot == (uint32_t)s ? acc[i] : 0.0f;
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = 0.0f;
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
      if constexpr (FMT != kFmtBF16) load_next(buf[d]);
      if (it < steps) {
        const u32x4* xb = lds + (cp & 1u) * a.xwords + ck * 16u;   // block ck of the phase
        if constexpr (kMF) {
          // k-group t outer, activation tile cc inner: the NT accumulators' chains interleave, so
          // no product waits on the one before it
          floatx4 a4[NT];
#pragma unroll
          for (int cc = 0; cc < NT; ++cc)
            a4[cc] = (floatx4){acc[4 * cc], acc[4 * cc + 1], acc[4 * cc + 2], acc[4 * cc + 3]};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 av = {p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]};
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              const int xr = 16 * cc + r16;
              const u32x4 bv = (MR >= 16 * (cc + 1) || xr < MR) ? xb[xr * rs + ((4 * g + t) ^ r16)]
                                                                : (u32x4){0u, 0u, 0u, 0u};
              a4[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, bv), a4[cc], 0, 0, 0);
            }
          }
#pragma unroll
          for (int cc = 0; cc < NT; ++cc) {
            acc[4 * cc] = a4[cc][0]; acc[4 * cc + 1] = a4[cc][1];
            acc[4 * cc + 2] = a4[cc][2]; acc[4 * cc + 3] = a4[cc][3];
          }
        } else {
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const u32x4* xr = xb + m * rs;
            const u32x4 x0 = xr[(4 * g) ^ m], x1 = xr[(4 * g + 1) ^ m];
            const u32x4 x2 = xr[(4 * g + 2) ^ m], x3 = xr[(4 * g + 3) ^ m];
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
        advance(cp, ct, ck, ci);
        if (cp != cph) phase_end((int)cph);
      }
      if constexpr (FMT == kFmtBF16) load_next(buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // a wave with an empty range still takes part in every phase change and patches the escapes
  // of the tile it finalises
  if (L == 0)
    for (int ph = 0; ph < nph; ++ph) phase_end(ph);

  // ---- the running sums into LDS (over the x buffers, after the last phase's reads) ----
  float* s_part = reinterpret_cast<float*>(lds);     // [W][SL][16][MP]
  lds_barrier();
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    float* dst = s_part + ((w * SL + s) * kTileRows) * MP;
    if constexpr (kMF) {
#pragma unroll
      for (int cc = 0; cc < NT; ++cc)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (MR >= 16 * (cc + 1) || 16 * cc + r16 < MR) dst[(4 * g + r) * MP + 16 * cc + r16] = tot[s][4 * cc + r];
    } else {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float v = group_sum(tot[s][m]);
        if (g == m) dst[r16 * MP + m] = v;
      }
    }
  }
  lds_barrier();

  // ---- finalise local tiles w + f W: partial sums in wave order, escapes, scale, store ----
  const auto owner = [&](uint32_t u) {               // the wave whose range holds unit u
    return (int)(((uint64_t)W * (u + 1) + U - 1) / U) - 1;
  };
  // top-1 mode: the lane's best key per x row over its tiles (value order of the float bits, NaN
  // above +Inf; ties to the lowest row index), in place of the stores
  uint64_t best[NX];
#pragma unroll
  for (int cc = 0; cc < NX; ++cc) best[cc] = 0;
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    if (!fin[f]) break;
    // escapes past the LDS copy of a crowded tile: entries and x from memory
    if constexpr (kEsc) {
      float scph = 0.0f;
      if constexpr (FT > 1 && has_placeholder<FMT>()) {
        if constexpr (FMT == kFmtI8) scph = __uint_as_float(fsc[f]) * placeholder_of<FMT>();
        else scph = window_scale(fsc[f]) * placeholder_of<FMT>();
      }
      for (uint32_t e = cur[f] > lds_end[f] ? cur[f] : lds_end[f]; e < st[f][1]; ++e) {
        const uint32_t col = a.esc_col[e];
        const float v = bf16_to_float(a.esc_val[e]);
#pragma unroll
        for (int cc = 0; cc < NX; ++cc) {
          const int m = xm(cc);
          if (!xlane || m >= a.mrows) continue;
          const float xv = bf16_to_float(a.x[(int64_t)m * a.k + col]);
          if constexpr (FT == 1) {
            if constexpr (has_placeholder<FMT>()) dP[cc] = fmaf(-xv, placeholder_of<FMT>(), dP[cc]);
            Qe[f][cc] = fmaf(xv, v, Qe[f][cc]);
          } else {
            Qe[f][cc] = fmaf(xv, v, Qe[f][cc]);
            if constexpr (has_placeholder<FMT>()) Qe[f][cc] = fmaf(-xv, scph, Qe[f][cc]);
          }
        }
      }
    }
    // the partial sums of the tile for the lane's row, in wave order
    const int j = w + f * W;
    const int wf = owner((uint32_t)j * kbp), wl = owner((uint32_t)j * kbp + kbp - 1);
    float P[NX];
#pragma unroll
    for (int cc = 0; cc < NX; ++cc) P[cc] = 0.0f;
    for (int wv = wf; wv <= wl; ++wv) {
      const uint32_t v0 = rstart(wv);
      if (v0 == rstart(wv + 1)) continue;            // an empty range
      const int si = j - (int)(v0 / kbp);
      const float* src = s_part + ((wv * SL + si) * kTileRows) * MP;
#pragma unroll
      for (int cc = 0; cc < NX; ++cc)
        if (xlane && xm(cc) < MR) P[cc] += src[r16 * MP + xm(cc)];
    }
    if (!xlane) continue;
    // y = 2^(base - 112) (P + dP) + Qe (the 8-bit copy: its row scale; three tiles per wave: the
    // placeholder terms are in Qe), or P for the dense baseline
    const int64_t row = row0[f] + r16;
    if (row >= a.n) continue;
    float sc = 1.0f;
    if constexpr (FMT == kFmtI8) sc = __uint_as_float(fsc[f]);
    else if constexpr (kEsc) sc = window_scale(fsc[f]);
#pragma unroll
    for (int cc = 0; cc < NX; ++cc) {
      const int m = xm(cc);
      if (m >= a.mrows) continue;
      float v = P[cc];
      if constexpr (kEsc) v = FT == 1 ? fmaf(sc, P[cc] + dP[cc], Qe[f][cc]) : fmaf(sc, P[cc], Qe[f][cc]);
      if (a.keys) {
        const uint32_t u = __float_as_uint(v);
        const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        const uint64_t key = ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
        best[cc] = key > best[cc] ? key : best[cc];
      } else if (a.y16) {
        a.y16[m * a.ldy + row] = float_to_bf16_rne(v);
      } else {
        a.y[m * a.ldy + row] = v;
      }
    }
  }
  if (a.keys) {
    // the best over the lane's 16 rows (lanes r16 of one g), then over the waves through LDS:
    // wave w's 32 keys at word w * 32 of the escape-copy area, unused by now (every wave walked
    // its last phase before the barrier ahead of the partial sums; the area holds at least
    // 256 bytes per wave)
    uint64_t* s_key = reinterpret_cast<uint64_t*>(lds + a.eoff) + w * 32;
#pragma unroll
    for (int cc = 0; cc < NX; ++cc) {
      uint64_t b = best[cc];
#pragma unroll
      for (int sh = 1; sh < 16; sh *= 2) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)b, sh, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(b >> 32), sh, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        b = o > b ? o : b;
      }
      if (r16 == 0 && xm(cc) < 32) s_key[xm(cc)] = b;
    }
    if (MR < 32 && lane >= MR && lane < 32) s_key[lane] = 0;
    lds_barrier();
    if (w == 0 && lane < 32) {
      uint64_t b = 0;
      for (int wv = 0; wv < W; ++wv) {
        const uint64_t o = reinterpret_cast<const uint64_t*>(lds + a.eoff)[wv * 32 + lane];
        b = o > b ? o : b;
      }
      a.keys[(int64_t)blockIdx.x * 32 + lane] = b;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
typedef void (*StreamKernel)(StreamArgs);

template <int FMT>
static StreamKernel stream_pick(int mr, int ft) {
  if (ft == 2) return mr == 32 ? k_stream<FMT, 32, 12, 2> : k_stream<FMT, 64, 8, 2>;
  if (ft == 3) {
    switch (mr) {
      case 4: return k_stream<FMT, 4, 16, 3>;
      case 8: return k_stream<FMT, 8, 16, 3>;
      default: return k_stream<FMT, 16, 16, 3>;
    }
  }
  switch (mr) {
    case 1: return k_stream<FMT, 1, 16, 1>;
    case 2: return k_stream<FMT, 2, 16, 1>;
    case 4: return k_stream<FMT, 4, 16, 1>;
    case 8: return k_stream<FMT, 8, 16, 1>;
    case 16: return k_stream<FMT, 16, 16, 1>;
    case 32: return k_stream<FMT, 32, 12, 1>;
    default: return k_stream<FMT, 64, 8, 1>;
  }
}

static StreamKernel stream_kernel(Fmt f, int mr, int ft) {
  if (f == kFmtW12) return stream_pick<kFmtW12>(mr, ft);
  if (f == kFmtQ8) return stream_pick<kFmtQ8>(mr, ft);
  if (f == kFmtQ8M) return stream_pick<kFmtQ8M>(mr, ft);
  if (f == kFmtI8) return stream_pick<kFmtI8>(mr, ft);
  return stream_pick<kFmtBF16>(mr, ft);
}

constexpr int64_t kPassRows = 64;   // rows of x per pass (per weight read)

// rows of x the kernel instance for mb rows is built for, its waves per workgroup (16 of up to
// 128 VGPRs, 12 of up to 168, 8 of up to 256 for the accumulators of 64 rows) and the tiles one
// wave's range may touch
static int stream_rows(int64_t mb) {
  return mb <= 2 ? (int)mb : mb <= 4 ? 4 : mb <= 8 ? 8 : mb <= 16 ? 16 : mb <= 32 ? 32 : 64;
}
static int stream_waves(int mr) { return mr > 32 ? 8 : mr > 16 ? 12 : 16; }
// tiles a wave finalises on shapes with more tiles than waves on the chip: 3 for 3..16 rows
// (instances for 4, 8 and 16 rows), 2 for 17..64 rows (each row group re-reads all of x through
// the CU, as much as the CU's weights at 64 rows; at 32 rows the LM-head-like [152064, 5120] takes
// 209.8 us instead of 229.6 in four groups); else 1
static int stream_ft(const DevInfo& di, Fmt, int mr, int64_t tiles) {
  if (tiles <= (int64_t)stream_waves(mr) * di.cus) return 1;
  return mr >= 3 && mr <= 16 ? 3 : mr > 16 ? 2 : 1;
}
static int stream_slots(int mr, int ft) { return ft == 3 ? 4 : (mr > 32 || ft == 2) ? 3 : 2; }

struct StreamPlan {
  int mr = 0, waves = 0, nph = 0, ft = 1;
  int64_t G = 0;
  uint32_t kbp = 0, rs = 0, xwords = 0, eoff = 0;
  size_t lds = 0;
};

// The phase length for a pass of mb rows over a group of n rows, with ft tiles finalised per
// wave: among the divisors of the row's blocks whose x buffers (two, one for a single phase) fit
// the LDS and that keep every wave's range within the kernel's tile slots, the one with the
// fewest blocks for the busiest wave over all phases (a phase change counted as half a block).
// A CU with 8 or more tiles of 16 or more blocks takes 4 to 10 phases where one fits: its waves
// then walk the escapes phase by phase while their next blocks load, rather than all at the end
// (gate+up [34816, 5120], 4 rows: Q8 36.0 -> 33.8 us, W12 46.7 -> 46.0; the LM head [152064,
// 5120]: Q8 139.7 -> 133.2; with fewer tiles per CU the extra barriers cost more: [8192, 5120]
// W12 15.9 -> 17.4).  False if none fits.
static bool stream_plan(const DevInfo& di, int64_t mb, int64_t n, int64_t k, int ft, StreamPlan* out) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows, nkb = k / kTileCols;
  const int mr = stream_rows(mb), W = stream_waves(mr);
  const int64_t G = tiles < di.cus ? tiles : di.cus;
  const int64_t tmax = (tiles + G - 1) / G;          // tiles of the busiest CU
  const int64_t minph = tmax >= 8 && nkb >= 16 ? 4 : 1;
  double best = 0;
  bool found = false;
  for (int pass = 0; pass < 2 && !found; ++pass)
  for (int64_t kbp = nkb; kbp >= 1; --kbp) {
    if (nkb % kbp) continue;
    const int64_t nph = nkb / kbp;
    if (pass == 0 && minph > 1 && (nph < minph || nph > 10)) continue;
    const int64_t segs = (kbp + 3) / 4, rs = 64 * segs, xwords = mr * rs;
    if (mr * segs > kSPieces) continue;
    const int64_t U = tmax * kbp;
    if (U >= (int64_t(1) << 31)) continue;
    const int64_t lmax = (U + W - 1) / W;
    if (tmax > (int64_t)ft * W) continue;            // the waves finalise every tile
    const int SL = stream_slots(mr, ft);
    if ((lmax - 1) / kbp + 2 > SL) continue;         // a range over at most SL tiles
    const int64_t part = (int64_t)W * SL * kTileRows * (mr + 1) * 4;
    const int64_t xb = (nph > 1 ? 2 : 1) * xwords * 16;
    const int64_t body = ((xb > part ? xb : part) + 15) / 16 * 16;
    // then the escape copies (walked per phase with one tile per wave)
    const int64_t cap = ft == 1 ? kSECap : kSECap3;
    const int64_t lds = body + (int64_t)W * ft * (cap * 4 + (cap + 128) * 2);
    if (lds > di.max_lds) continue;
    const double cost = (double)(lmax * nph) + 0.5 * (double)(nph - 1);
    if (found && cost >= best) continue;
    found = true;
    best = cost;
    out->mr = mr; out->waves = W; out->nph = (int)nph; out->G = G; out->ft = ft;
    out->kbp = (uint32_t)kbp; out->rs = (uint32_t)rs; out->xwords = (uint32_t)xwords; out->lds = (size_t)lds;
    out->eoff = (uint32_t)(body / 16);
  }
  return found;
}

// Row groups of a shape with more 16-row tiles than the waves on the chip finalise: as few as
// keep every CU at ft tiles per wave or fewer, of equal size (whole tiles).  One launch runs
// them all, group after group in workgroup order, so a CU that finishes its workgroup of one
// group takes one of the next without waiting for a kernel boundary.
static int64_t stream_group_rows(const DevInfo& di, int64_t mb, int64_t n, int ft) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t cap = (int64_t)stream_waves(stream_rows(mb)) * ft * di.cus;
  const int64_t groups = (tiles + cap - 1) / cap;
  return (tiles + groups - 1) / groups * kTileRows;
}

bool stream_fits(const DevInfo& di, Fmt f, int64_t m, int64_t n, int64_t k) {
  if (m < 1 || n < 1 || k * kPassRows * 2 >= (int64_t(1) << 32)) return false;
  StreamPlan p;
  const int64_t full = m < kPassRows ? m : kPassRows, tail = (m - 1) % kPassRows + 1;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  for (const int64_t mb : {full, tail}) {
    const int ft = stream_ft(di, f, stream_rows(mb), tiles);
    const int64_t gr = stream_group_rows(di, mb, n, ft);
    // the plan of a full group (a smaller last group runs the same plan with fewer tiles)
    if (!stream_plan(di, mb, gr < n ? gr : n, k, ft, &p)) return false;
  }
  return true;
}

hipError_t launch_stream(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                         YOut y, hipStream_t s, uint64_t* keys, int* key_groups) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  if (!stream_fits(di, f, m, n, k) || y.silu) return hipErrorInvalidValue;
  for (int64_t m0 = 0; m0 < m; m0 += kPassRows) {
    const int64_t mb = (m - m0) < kPassRows ? (m - m0) : kPassRows;
    const int ft = stream_ft(di, f, stream_rows(mb), (n + kTileRows - 1) / kTileRows);
    const int64_t gr = stream_group_rows(di, mb, n, ft);   // a multiple of 16
    StreamPlan pl;
    if (!stream_plan(di, mb, gr < n ? gr : n, k, ft, &pl)) return hipErrorInvalidValue;
    const int64_t groups = (n + gr - 1) / gr;
    StreamArgs a;
    a.x = x + m0 * k;
    a.mrows = (int)mb;
    a.base = p.base; a.ae = p.ae; a.lo = p.lo;
    a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
    a.w = p.w;
    a.scale = p.scale;
    const YOut yp = y + m0 * n;
    a.y = yp.f;
    a.y16 = yp.h;
    a.ldy = n;
    a.n = n; a.k = k;
    a.kbp = pl.kbp; a.nph = pl.nph; a.rs = pl.rs; a.xwords = pl.xwords; a.eoff = pl.eoff;
    a.gtiles = gr / kTileRows;                         // (the last group may be smaller)
    a.G = pl.G;
    a.keys = keys;
    if (keys) {
      // top-1 mode: one pass of at most 32 rows, keys [grid][32]
      if (m > 32) return hipErrorInvalidValue;
      *key_groups = (int)(groups * pl.G);
    }
    hipLaunchKernelGGL(stream_kernel(f, pl.mr, pl.ft), dim3((unsigned)(groups * pl.G)), dim3(64 * pl.waves), pl.lds, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

bool stream_top1_fits(const DevInfo& di, Fmt f, int64_t m, int64_t n, int64_t k) {
  if (m < 1 || m > 32 || !stream_fits(di, f, m, n, k)) return false;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t gr = stream_group_rows(di, m, n, stream_ft(di, f, stream_rows(m), tiles));
  const int64_t grid = (n + gr - 1) / gr * (tiles < di.cus ? tiles : di.cus);
  return (uint64_t)grid * 32u * 8u <= kWorkspaceBytes;
}

hipError_t launch_stream_top1(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                              int32_t* idx, float* val, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  if (!stream_top1_fits(di, f, m, n, k)) return hipErrorInvalidValue;
  Scratch sc;
  sc.s = s;
  float* ws = nullptr;
  err = sc.get(&ws);
  if (err != hipSuccess) return err;
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws);                 // [grid][32]
  int groups = 0;
  err = launch_stream(f, x, m, p, n, k, YOut{}, s, keys, &groups);
  if (err != hipSuccess) return err;
  return launch_top1_final(keys, groups, (int)m, idx, val, s);
}

}  // namespace w12
