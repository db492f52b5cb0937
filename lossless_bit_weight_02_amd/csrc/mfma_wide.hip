// Skinny GEMM for 33..64 activation rows (three or four 16-row activation tiles) on the matrix
// cores: y[m][n] = sum_k x[m][k] W[n][k].  Up to two tiles run k_mfma in mfma.hip, which stages
// x with global-to-LDS loads; with three or four tiles the register-staged pipeline below is
// faster (the larger x chunks leave the global-to-LDS variant fewer weight blocks in flight).
//
// From about 16 rows the product is a dense contraction again (SpecPilot, arXiv 2611.02501,
// summary page, "Main Findings": the W12 GEMM is measured at 1 and at 32 rows), so the decoded
// weights feed v_mfma_f32_16x16x32_bf16 as its A operand -- the register operand of the pages'
// design (figure-captions page, Fig. 5(b), there for wgmma).
//
// Work split.  One workgroup of kWaves waves per CU (the x chunks fill most of the CU's LDS).
// A wave owns one 16-row tile at a time and streams all of its 128-column blocks; tiles are dealt
// round-robin over the workgroups first, so every CU gets the same number of tiles to within one
// (the weight stream is the bottleneck, and a CU with one more workgroup than the rest would set
// the kernel's time).  The tiled plane storage (w12_device.hpp) holds each 16-row x 128-column
// block in operand order: lane l = r + 16g loads row r, columns 32g..32g+31 with wave-wide 1 KiB
// reads and decodes them straight into four A operands.
//
// Software pipeline.  Every load is a buffer load whose offset is pushed past the buffer's range
// when there is nothing to load (the hardware then returns zeros and fetches nothing), so no load
// sits behind a branch and every ring slot is a compile-time register set.  Vector-memory loads
// complete in issue order, so a wait for one load is a wait for all older ones; the kernel
// therefore issues its loads in one fixed pattern per step -- one x fragment, then the refill of
// the A block D steps ahead -- and consumes each load exactly D - 1 (x) or D (A) steps later, and
// the prologue issues the same pattern for D virtual steps.  No wait then ever covers a block
// that is not due yet.
//
// x: chunks of S k-blocks (128 S columns) of the m rows live in LDS in fragment order (each B
// operand is one contiguous 1 KiB read), double buffered.  While chunk c is consumed, the 4 NT
// pieces per step of chunk c+1 stream in through a D-deep register ring; the piece jobs rotate
// over the waves.  A piece is 1 KiB of row-major x (2 rows x 256 columns: a coalesced read);
// its lanes scatter into the fragment layout, whose 16-byte slots are XOR-swizzled inside each
// 128-byte row (slot = lane ^ (t | (g & 1) << 2) for k-group t and column group g) so that
// both these writes and the operand reads are free of bank conflicts.  One barrier per chunk.
//
// Escapes (exact weights outside a row's window): the lanes of column group g own output rows
// 4g..4g+3 of the tile.  The tile's escape list (up to kEscCap entries) is copied to LDS at the
// start of the tile; at the end of every chunk each lane walks its rows' column-sorted runs up to
// the chunk's last column, reading x from the chunk still in LDS, and accumulates
//   y = 2^(base-112) * (acc - 2^-15 * sum_esc x) + sum_esc x * v,
// which takes the placeholder value 2^-15 of an escaped slot (AE = 0, B = 0) back out of acc.
// Escapes past the LDS copy of a crowded tile are read from memory after the loop.
#include "mfma_common.hpp"

namespace w12 {

// Compile-time shape of one instantiation: a 3-deep ring of weight blocks at three activation
// tiles and a 2-deep one at four (the accumulators take the rest of the 168 VGPRs).
template <int FMT, int NT>
struct ShapeWide {
  static_assert(NT == 3 || NT == 4, "one and two tiles run k_mfma");
  static constexpr int D = NT == 3 ? 3 : 2;
  static constexpr int S = D == 3 ? 6 : 4;            // k-blocks per x chunk
  static constexpr int FS = 4 * NT;                   // 1 KiB x pieces per k-block
  static constexpr int F = FS * S;                    // 1 KiB x pieces per chunk
  static constexpr int XL = (FS + kWaves - 1) / kWaves;  // pieces a wave loads per step
  static_assert(S % D == 0 && S % 2 == 0, "a chunk must hold whole rings and 256-column blocks");
};

// Twelve waves (three per SIMD) on the CU: at most 168 VGPRs.
template <int FMT, int NT, bool SILU = false>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3, 3)))
void k_mfma_wide(MfmaArgs a) {
  using SH = ShapeWide<FMT, NT>;
  constexpr int D = SH::D, S = SH::S, FS = SH::FS, F = SH::F, XL = SH::XL;
  constexpr bool kEsc = FMT != kFmtBF16;
  __shared__ __attribute__((aligned(16))) u32x4 s_x[2][F * 64];
  __shared__ __attribute__((aligned(16))) u32x4 s_scratch[64];   // stores of waves with no piece
  __shared__ uint32_t s_ecol[kEsc ? kWaves : 1][kEsc ? kEscCap : 1];   // per wave: tile escapes
  __shared__ uint16_t s_eval[kEsc ? kWaves : 1][kEsc ? kEscCap : 1];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const uint32_t lane16 = 16u * lane;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t KB = (uint32_t)(a.k / kTileCols);
  const uint32_t KBp = (KB + S - 1) / S * S;
  const int64_t tiles = (a.n + kTileRows - 1) / kTileRows;
  const uint32_t e112 = exp112_pair();
  const uint32_t kx = (uint32_t)a.k;
  const Rsrc rx = make_rsrc(a.x, (uint32_t)a.m * kx * 2u);

  // Piece I of chunk c (I < F): lanes 0..31 and 32..63 read rows 2q and 2q+1, columns
  // 256 hb + 8 (lane % 32) .. +7 of the chunk, where q = I % (8 NT), hb = I / (8 NT).  Pieces
  // are numbered per tile, P = c F + I.
  const uint32_t prow = lane >> 5, pcol = 8u * (lane & 31);
  const uint32_t lpart = 2u * (prow * kx + pcol);
  // The address is computed unconditionally and hidden from the optimizer, so that the
  // out-of-range select stays a select instead of a branch around the address arithmetic.
  const auto piece_load = [&](uint32_t P, bool have) {
    const uint32_t c = P / F, I = P % F, q = I % (8 * NT), hb = I / (8 * NT);
    const uint32_t col0 = 128u * S * c + 256u * hb;
    uint32_t off = 2u * (2u * q * kx + col0) + lpart;
    asm volatile("" : "+v"(off));
    const bool ok = have && col0 + pcol < kx && (int)(2 * q + prow) < a.m;
    return __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? off : kOOB, 0, 0);
  };
  // LDS slot of this lane's 16 bytes of piece I: fragment f = (k-block * 4 + t) * NT + cc holds
  // x[16 cc + r][.. + 32 g + 8 t .. +7] for operand lane r + 16 g, at slot (r + 16 g) ^ swz(t, g),
  // swz = t | (g & 1) << 2.  With a = 2q % 16 even, (a + row bit + 16 g) ^ swz splits into a
  // uniform part, a lane part and (a % 8) ^ (row bit ^ swz).
  const uint32_t pt = (pcol >> 3) & 3u, pg = (pcol >> 5) & 3u;
  const uint32_t lslot = ((pcol >> 7) * 4u + pt) * NT * 64u + 16u * pg;
  const uint32_t lkey = prow ^ (pt | ((pg & 1u) << 2));
  const auto piece_slot = [&](uint32_t I) {
    const uint32_t q = I % (8 * NT), hb = I / (8 * NT), aa = (2 * q) & 15u;
    return (2 * hb * 4 * NT + (q >> 3)) * 64u + (aa & 8u) + lslot + ((aa & 7u) ^ lkey);
  };
  // Streamed pieces (P >= F) are dealt to the waves round-robin: wave w loads the pieces
  // P = w (mod kWaves), each in the step whose range [F + (u + D - 1) FS, F + (u + D) FS) holds it,
  // and stores it D - 1 steps later (into chunk P / F, which is then the next chunk).
  const uint32_t first_piece = F + (uint32_t)((w - F % kWaves + kWaves) % kWaves);
  // Branch-free: a wave without a piece this step loads nothing (offset past the range) and
  // stores to s_scratch, which is never read; its ring entry has bit 31 set.
  const auto x_stream_load = [&](int u, uint32_t& nxt, uint32_t (&pr)[XL], u32x4 (&dst)[XL]) {
    const uint32_t hi = (uint32_t)(F + (u + D) * FS);
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const bool have = nxt < hi;
      pr[i] = have ? nxt : (nxt | 0x80000000u);
      dst[i] = piece_load(nxt, have);
      nxt = have ? nxt + kWaves : nxt;
    }
  };
  const auto x_stream_store = [&](const uint32_t (&pr)[XL], const u32x4 (&src)[XL]) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const uint32_t P = pr[i] & 0x7FFFFFFFu;
      uint32_t at = ((P / F) & 1u) * (F * 64) + piece_slot(P % F);
      asm volatile("" : "+v"(at));
      u32x4* dst = (pr[i] >> 31) ? &s_scratch[lane] : &s_x[0][0] + at;
      *dst = src[i];
    }
  };
  const uint32_t bswz = lane ^ (((uint32_t)g & 1u) << 2);   // operand slot of k-group t: bswz ^ t

  for (int round = 0; round < a.rounds; ++round) {
    const int64_t tile = ((int64_t)round * kWaves + w) * gridDim.x + blockIdx.x;
    const bool valid = tile < tiles;
    const int64_t row0 = (valid ? tile : 0) * kTileRows;

    lds_barrier();                                 // the previous tile no longer reads LDS

    // ---- escape list of the tile (oldest loads: waited for before the loop) ----
    uint32_t st[5] = {0, 0, 0, 0, 0}, t_e0 = 0;
    RowScales<FMT> rsc;
    uint32_t ecol[kEscCap / 64], evalv[kEscCap / 64];
    if constexpr (kEsc) {
      const int64_t rg = row0 + 4 * g;
      const auto ptr_at = [&](int64_t r) { return a.esc_ptr[r < a.n ? r : a.n]; };
#pragma unroll
      for (int r = 0; r < 5; ++r) st[r] = ptr_at(rg + r);
      rsc.load(a, rg);
      t_e0 = __builtin_amdgcn_readfirstlane(a.esc_ptr[row0]);
      const uint32_t t_e1 = __builtin_amdgcn_readfirstlane(valid ? ptr_at(row0 + kTileRows) : t_e0);
      const uint32_t cnt = t_e1 - t_e0 < (uint32_t)kEscCap ? t_e1 - t_e0 : (uint32_t)kEscCap;
      const Rsrc r_col = make_rsrc(a.esc_col + t_e0, cnt * 4u);
      const Rsrc r_val = make_rsrc(a.esc_val + t_e0, cnt * 2u);
#pragma unroll
      for (int i = 0; i < kEscCap / 64; ++i) {
        ecol[i] = __builtin_amdgcn_raw_buffer_load_b32(r_col, 4u * (lane + 64 * i), 0, 0);
        evalv[i] = __builtin_amdgcn_raw_buffer_load_b16(r_val, 2u * (lane + 64 * i), 0, 0);
      }
      if (!valid) {
#pragma unroll
        for (int r = 0; r < 5; ++r) st[r] = t_e0;
      }
    }

    // ---- chunk 0 of x ----
    constexpr int XF = (F + kWaves - 1) / kWaves;
    u32x4 x0[XF];
#pragma unroll
    for (int i = 0; i < XF; ++i) x0[i] = piece_load((uint32_t)(w + kWaves * i), w + kWaves * i < F);

    // ---- D virtual steps -D .. -1: the same load pattern as a loop step ----
    Rsrc ra, rl;
    if constexpr (FMT == kFmtBF16) {
      ra = make_rsrc(a.w + row0 * a.k, valid ? KB * (uint32_t)kTileBF : 0u);
      rl = ra;
    } else {
      ra = make_rsrc(a.ae + row0 * a.k, valid ? KB * (uint32_t)kTileAE : 0u);
      rl = make_rsrc(a.lo + row0 * a.k / 2, valid ? KB * (uint32_t)kTileLO : 0u);
    }
    ABlock<FMT> buf[D];
    u32x4 xr[D][XL];
    uint32_t pr[D][XL];
    uint32_t nxt = first_piece;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      x_stream_load(d - D, nxt, pr[d], xr[d]);     // step d - D uses ring slot d
      load_ablock<FMT>(ra, rl, (uint32_t)d, lane16, buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int i = 0; i < XF; ++i)
      if (w + kWaves * i < F) s_x[0][piece_slot((uint32_t)(w + kWaves * i))] = x0[i];
    if constexpr (kEsc) {
#pragma unroll
      for (int i = 0; i < kEscCap / 64; ++i) {
        s_ecol[w][lane + 64 * i] = ecol[i];
        s_eval[w][lane + 64 * i] = (uint16_t)evalv[i];
      }
    }
    lds_barrier();

    // per row r: cursor (absolute escape index) and the column under it (~0: none in LDS)
    const uint32_t lds_end = t_e0 + kEscCap;
    const auto run_end = [&](int r) { return st[r + 1] < lds_end ? st[r + 1] : lds_end; };
    uint32_t cur[4], ncol[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cur[r] = st[r];
      ncol[r] = 0xFFFFFFFFu;
      if constexpr (kEsc) ncol[r] = cur[r] < run_end(r) ? s_ecol[w][cur[r] - t_e0] : 0xFFFFFFFFu;
    }

    floatx4 acc[NT];
    float qv[NT][4];   // escape values times x; the placeholder terms go into acc directly
#pragma unroll
    for (int cc = 0; cc < NT; ++cc) {
      acc[cc] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[cc][r] = 0.f;
    }

    for (uint32_t c = 0; c * S < KBp; ++c) {       // chunk c: k-blocks S c .. S c + S - 1
      const uint32_t b = c & 1u;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int slot = s % D;
        const uint32_t kb = S * c + s;
        uint32_t p[16];
        ablock_pairs<FMT>(buf[slot], e112, p);
        if constexpr (FMT != kFmtBF16) pin16(p);
        __builtin_amdgcn_sched_barrier(0);
        // x ring: the fragments loaded at step kb - D + 1 go to LDS, then this step's fragments
        x_stream_store(pr[(s + 1) % D], xr[(s + 1) % D]);
        x_stream_load((int)kb, nxt, pr[slot], xr[slot]);
        // A ring: refill this slot with block kb + D (dense blocks are their own A operands and
        // are refilled after the MFMAs below)
        if constexpr (FMT != kFmtBF16) load_ablock<FMT>(ra, rl, kb + D, lane16, buf[slot]);

        const u32x4* xb = &s_x[b][s * FS * 64];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4 av = {p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]};
#pragma unroll
          for (int cc = 0; cc < NT; ++cc) {
            const u32x4 bv = xb[(t * NT + cc) * 64 + (bswz ^ (uint32_t)t)];
            acc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bv), acc[cc],
                                                             0, 0, 0);
          }
        }
        if constexpr (FMT == kFmtBF16) load_ablock<FMT>(ra, rl, kb + D, lane16, buf[slot]);
        __builtin_amdgcn_sched_barrier(0);
      }

      if constexpr (kEsc) {
        // escapes of rows 4g..4g+3 with a column in this chunk, x from LDS buffer b
        const uint32_t lim = 128u * S * (c + 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          while (ncol[r] < lim) {
            const uint32_t e = cur[r] - t_e0;
            const uint32_t col = ncol[r] - 128u * S * c;
            const float v = bf16_to_float(s_eval[w][e]);
            const uint32_t tt = (col >> 3) & 3u, gg = (col >> 5) & 3u;
            const uint32_t f0 = ((col >> 7) * 4u + tt) * NT;
            const uint32_t ln = (r16 + 16u * gg) ^ (tt | ((gg & 1u) << 2));
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              const float xv = bf16_to_float(
                  reinterpret_cast<const uint16_t*>(&s_x[b][(f0 + cc) * 64 + ln])[col & 7u]);
              if constexpr (has_placeholder<FMT>()) acc[cc][r] = fmaf(-xv, placeholder_of<FMT>(), acc[cc][r]);
              qv[cc][r] = fmaf(xv, v, qv[cc][r]);
            }
            cur[r] += 1;
            ncol[r] = cur[r] < run_end(r) ? s_ecol[w][e + 1] : 0xFFFFFFFFu;
          }
        }
      }
      lds_barrier();
    }

    if (!valid) continue;
    if constexpr (kEsc) {
      // escapes beyond the LDS copy of a crowded tile
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        for (uint32_t e = cur[r]; e < st[r + 1]; ++e) {
          const uint32_t col = a.esc_col[e];
          const float v = bf16_to_float(a.esc_val[e]);
#pragma unroll
          for (int cc = 0; cc < NT; ++cc) {
            const int mrow = 16 * cc + r16;
            const float xv = mrow < a.m ? bf16_to_float(a.x[(int64_t)mrow * a.k + col]) : 0.0f;
            if constexpr (has_placeholder<FMT>()) acc[cc][r] = fmaf(-xv, placeholder_of<FMT>(), acc[cc][r]);
            qv[cc][r] = fmaf(xv, v, qv[cc][r]);
          }
        }
      }
    }
    if constexpr (SILU) {
      // SiLU(gate) * up: lanes g = 0, 1 hold gate rows 4 g .. 4 g + 3, lane ^ 32 the up rows
      const int64_t ldh = a.ldy >> 1;
#pragma unroll
      for (int cc = 0; cc < NT; ++cc) {
        const int mcol = 16 * cc + r16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = kEsc ? fmaf(rsc.get(r), acc[cc][r], qv[cc][r]) : acc[cc][r];
          const float up = __shfl_xor(v, 32);
          const float hv = silu(v) * up;
          const int64_t at = mcol * ldh + row0 / 2 + 4 * g + r;
          if (g < 2 && mcol < a.m) {
            if (a.y16) a.y16[at] = float_to_bf16_rne(hv);
            else a.y[at] = hv;
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t nrow = row0 + 4 * g + r;
      if (nrow >= a.n) continue;
      const float sc = rsc.get(r);
#pragma unroll
      for (int cc = 0; cc < NT; ++cc) {
        const int mcol = 16 * cc + r16;
        if (mcol >= a.m) continue;
        const float v = kEsc ? fmaf(sc, acc[cc][r], qv[cc][r]) : acc[cc][r];
        if (a.y16) a.y16[mcol * a.ldy + nrow] = float_to_bf16_rne(v);
        else a.y[mcol * a.ldy + nrow] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// instantiations for three and four activation tiles
// ---------------------------------------------------------------------------------------------
MfmaKernel mfma_wide_kernel(Fmt f, int nt, bool silu) {
  if (silu) return nt == 3 ? k_mfma_wide<kFmtW12, 3, true> : k_mfma_wide<kFmtW12, 4, true>;
  if (f == kFmtW12) return nt == 3 ? k_mfma_wide<kFmtW12, 3> : k_mfma_wide<kFmtW12, 4>;
  if (f == kFmtQ8) return nt == 3 ? k_mfma_wide<kFmtQ8, 3> : k_mfma_wide<kFmtQ8, 4>;
  if (f == kFmtQ8M) return nt == 3 ? k_mfma_wide<kFmtQ8M, 3> : k_mfma_wide<kFmtQ8M, 4>;
  if (f == kFmtI8) return nt == 3 ? k_mfma_wide<kFmtI8, 3> : k_mfma_wide<kFmtI8, 4>;
  return nt == 3 ? k_mfma_wide<kFmtBF16, 3> : k_mfma_wide<kFmtBF16, 4>;
}

}  // namespace w12
