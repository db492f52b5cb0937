// Skinny GEMM on the matrix cores, y[m][n] = sum_k x[m][k] W[n][k], for one or two 16-row
// activation tiles (up to 32 rows) and for eight (passes of 65..128 rows).  Three and four tiles
// run the register-staged variant in mfma_wide.hip.
//
// From about 16 rows the product is a dense contraction again (SpecPilot, arXiv 2611.02501,
// summary page, "Main Findings": the W12 GEMM is measured at 1 and at 32 rows), so the decoded
// weights feed v_mfma_f32_16x16x32_bf16 as its A operand -- the register operand of the pages'
// design (figure-captions page, Fig. 5(b), there for wgmma).
//
// Work split.  One workgroup of W waves per CU: W = 12 (three waves of up to 168 VGPRs per SIMD,
// 4 blocks in flight each), or for the dense baseline on shapes whose tiles fit one round of
// 8 waves per CU, W = 8 (two waves of up to 256 VGPRs per SIMD, 8 blocks in flight each).
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
// operand is one contiguous 1 KiB read, lane l at byte 16 l), double buffered.  The fragments of
// chunk c+1 are loaded straight from memory into LDS (global-to-LDS loads: lane l of a fragment
// reads its 16 bytes of row-major x and the hardware writes them at byte 16 l) at the first step
// of chunk c, dealt round-robin over the waves; no register holds x on its way.  Rows past m and
// columns past k read zeros (buffer loads out of range).  One barrier per chunk.
//
// Split k.  A shape with too few tiles to give every wave of the chip one (the k and v
// projections of a 27B-class layer have 64, the down projection 320 tiles of 136 blocks) splits
// each row into `splits` k ranges of whole x chunks: workgroup b takes range b % splits of the
// tiles dealt to workgroup group b / splits, and writes its partial sums to its own slice of a
// workspace; a second kernel adds the slices in range order (deterministic).
//
// Escapes (exact weights outside a row's window): the lanes of column group g own output rows
// 4g..4g+3 of the tile.  The tile's escape list (up to kEscCapM entries) is copied to LDS at the
// start of the tile; at the end of every chunk each lane walks its rows' column-sorted runs up to
// the chunk's last column, reading x from the chunk still in LDS, and accumulates
//   y = 2^(base-112) * (acc - 2^-15 * sum_esc x) + sum_esc x * v,
// which takes the placeholder value 2^-15 of an escaped slot (AE = 0, B = 0) back out of acc.
// The x sums of the escaped slots are kept apart from the matrix-core accumulators: a vector
// write into an accumulator between MFMAs that feed it stalls the chain.
// Escapes past the LDS copy of a crowded tile are read from memory after the loop.
#include "mfma_common.hpp"

namespace w12 {

// Compile-time shape of one instantiation: D weight blocks in flight per wave (as many as the
// 168 VGPRs allow), chunks of S k-blocks of x (a multiple of D).  Four k-blocks per chunk
// measured faster than eight at one tile.
constexpr int kChunkBlocks = 4;   // k-blocks per x chunk with 12 waves (8 with 8 waves)
// Escapes of one tile copied to LDS: a 16-row tile of a 17408-column row holds ~315 escapes at
// the synthetic projections' escape rate (zeros dominate), ~20 at the pages' rate.
constexpr int kEscCapM = 384;
constexpr int kEscStage = 128;    // of which staged through registers with the first loads

template <int FMT, int NT, int W>
struct Shape {
  static_assert(NT == 1 || NT == 2 || NT == 8, "three and four tiles run k_mfma_wide");
  static_assert(W == 12 || W == 8, "12 or 8 waves per workgroup");
  static_assert(NT != 8 || W == 12, "eight tiles run with 12 waves");
  // blocks in flight per wave, and k-blocks per x chunk (eight activation tiles: 128 rows of x,
  // whose two 64 KiB chunk buffers fill most of the LDS, with a 2-deep ring)
  static constexpr int D = NT == 8 ? 2 : W == 12 ? 4 : 8;
  static constexpr int S = NT == 8 ? 2 : W == 12 ? kChunkBlocks : 8;
  static constexpr int FS = 4 * NT;                   // 1 KiB x fragments per k-block
  static constexpr int F = FS * S;                    // 1 KiB x fragments per chunk
  static constexpr int FW = (F + W - 1) / W;          // fragments a wave loads per chunk
  static constexpr int FPS = (FW + S - 1) / S;         // fragment loads per step
  static constexpr int LS = (FW + FPS - 1) / FPS - 1;   // last step with a fragment load
  static_assert(S % D == 0 && S % 2 == 0, "a chunk must hold whole rings and 256-column pieces");
};

// Global-to-LDS loads are not covered by the compiler's wait counts for the LDS reads that
// follow a barrier: before a barrier that publishes a chunk, a wave waits until at most N
// vector-memory operations (those it issued after its fragment loads) are outstanding; they
// complete in issue order.
template <int N>
__device__ __forceinline__ void vm_wait_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// W waves (W / 4 per SIMD) on the CU: at most 168 VGPRs with 12, 256 with 8.
// TOP1: the top-1 mode of MfmaArgs (no y; per-workgroup best keys).  SILU: the weights are
// row-interleaved gate+up (rows 0..7 of a tile gate, 8..15 up) and y / y16 hold
// h = silu(gate) * up, [m][ldy / 2], 8 outputs per tile (one k range only).
template <int FMT, int NT, int W, bool TOP1, bool SILU = false>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4)))
void k_mfma(MfmaArgs a) {
  using SH = Shape<FMT, NT, W>;
  constexpr int D = SH::D, S = SH::S, F = SH::F, FW = SH::FW, FPS = SH::FPS, LS = SH::LS;
  // kScale: decoded weights are w' = w / 2^(base - 112) and the outputs take the row's scale.
  // kEsc: escapes are patched chunk by chunk from x in LDS (up to two activation tiles); with
  // eight, their per-row sums would not fit the registers during the loop, so kEscEpi patches
  // them in the epilogue (registers free again) from the transposed x in memory.
  constexpr bool kScale = FMT != kFmtBF16;
  constexpr bool kEsc = kScale && NT <= 2;
  constexpr bool kEscEpi = kScale && !kEsc;
  constexpr bool kStage = kEsc || kEscEpi;       // the tile's escape list staged in LDS
  constexpr int kLoadsPerStep = FMT == kFmtBF16 ? 4 : FMT == kFmtW12 ? 3 : 2;
  __shared__ __attribute__((aligned(16))) u32x4 s_x[2][F * 64];
  __shared__ __attribute__((aligned(16))) u32x4 s_dummy[(FW * W > F) ? 64 : 1];   // target of unused fragment loads
  // per wave: the tile's escapes (with kEsc the values are copied in 4-byte pairs from an even
  // entry, so their copy starts one slot early when the tile's first entry is odd)
  constexpr int kValCap = kEsc ? kEscCapM + 128 : kEscCapM;
  __shared__ __attribute__((aligned(16))) uint32_t s_ecol[kStage ? W : 1][kStage ? kEscCapM : 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_eval[kStage ? W : 1][kStage ? kValCap : 1];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const uint32_t lane16 = 16u * lane;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t KB = (uint32_t)(a.k / kTileCols);
  const uint32_t n_chunks = (KB + S - 1) / S;
  const int64_t tiles = (a.n + kTileRows - 1) / kTileRows;
  // this workgroup's k range: chunks [c0, c1), blocks [kb0, kb0 + nkb), columns [col0, col1)
  const int sp = (int)(blockIdx.x % (uint32_t)a.splits);
  const int64_t grp = blockIdx.x / (uint32_t)a.splits, n_grp = gridDim.x / (uint32_t)a.splits;
  const uint32_t c0 = (uint32_t)sp * (uint32_t)a.cps;
  const uint32_t c1 = c0 + (uint32_t)a.cps < n_chunks ? c0 + (uint32_t)a.cps : n_chunks;
  const uint32_t kb0 = c0 * S;
  const uint32_t nkb = (c1 * S < KB ? c1 * S : KB) - kb0;
  const uint32_t col0 = 128u * kb0, col1 = 128u * (kb0 + nkb);
  float* const yout = a.y + sp * a.ysplit;
  const uint32_t e112 = exp112_pair();
  const uint32_t kx = (uint32_t)a.k;
  const Rsrc rx = make_rsrc(a.x, (uint32_t)a.m * kx * 2u);

  // LDS layout of a chunk: for each 256-column half hb of the chunk and each of the 16 NT rows
  // m, a 512-byte row segment at (hb * 16 NT + m) * 512, whose 16-byte column slots c16 are
  // rotated by the row: slot (c16 + m) % 32.  A global-to-LDS load moves one coalesced 1 KiB piece
  // of row-major x (rows 2q and 2q + 1, 256 columns; piece P = hb * 8 NT + q lands at P * 1 KiB):
  // lane j writes LDS slot j, so it reads the column slot ((j % 32) - row) % 32 of its row.  The
  // operand reads (16 consecutive rows, one slot each) and the escape reads then hit distinct
  // banks in every group of 8 lanes.
  // Wave w loads pieces w, w + 12, ... of a chunk (piece w + 12 i at step i / FPS of the chunk
  // before).  Every wave issues FW loads at every chunk (a fixed pattern, so the compiler's wait
  // counts stay exact): a load past the last piece reads nothing and writes zeros to s_dummy,
  // and rows past m and columns past k read zeros.
  const uint32_t prow = (uint32_t)lane >> 5, pslot = (uint32_t)lane & 31u;
  const auto x_fetch_one = [&](uint32_t c, uint32_t buf, int i) {
    const uint32_t P = (uint32_t)(w + W * i);
    const bool real = FW * W <= F || P < (uint32_t)F;
    const uint32_t q = P % (8u * NT), hb = P / (8u * NT);
    const uint32_t row = 2u * q + prow;
    const uint32_t c16 = (pslot - row) & 31u;
    const uint32_t col = 128u * S * c + 256u * hb + 8u * c16;
    const bool ok = real && (int)row < a.m && col < kx;
    u32x4* dst = real ? &s_x[buf][P * 64u] : &s_dummy[0];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)dst, 16,
                                             ok ? 2u * (row * kx + col) : kOOB, 0, 0, 0);
  };
  // LDS index (16-byte units) of row m, 16-byte column slot c16 of half hb of a chunk buffer
  const auto x_slot = [](uint32_t hb, uint32_t m, uint32_t c16) {
    return (hb * 16u * NT + m) * 32u + ((c16 + m) & 31u);
  };
  // Operand reads: lane l = r + 16 g of step t reads row 16 cc + r, slot 16 (s % 2) + 4 g + t of
  // half s / 2.  With (v + 16) % 32 = v ^ 16 and 4 g + r + t < 32 that is
  //   s / 2 * 512 NT + 512 cc + 32 r + ((4 g + r + t) ^ 16 ((s + cc) % 2)),
  // a lane part from xo[(s + cc) % 2][t] plus a constant the read instruction carries.
  uint32_t xo[2][4];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xo[par][t] = 32u * (uint32_t)r16 + ((4u * (uint32_t)g + (uint32_t)r16 + (uint32_t)t) ^ (16u * par));
      asm volatile("" : "+v"(xo[par][t]));
    }

  __shared__ unsigned long long s_best[TOP1 ? 32 : 1];   // top-1 mode: best key per x row
  if constexpr (TOP1)
    if (tid < 32) s_best[tid] = 0ull;              // published by the first barrier below

  for (int round = 0; round < a.rounds; ++round) {
    const int64_t tile = ((int64_t)round * W + w) * n_grp + grp;
    const bool valid = tile < tiles;
    const int64_t row0 = (valid ? tile : 0) * kTileRows;

    lds_barrier();                                 // the previous tile no longer reads LDS

    uint32_t st[5] = {0, 0, 0, 0, 0}, t_e0 = 0, t_cnt = 0, t_vsh = 0;
    RowScales<FMT> rsc;

    // ---- the range's first chunk of x, straight into LDS buffer 0 (the oldest loads: the
    // first barrier waits for them, not for the escape metadata) ----
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FW; ++i) x_fetch_one(c0, 0u, i);
    __builtin_amdgcn_sched_barrier(0);

    // ---- row bounds and window bottoms of the tile's escapes ----
    if constexpr (kScale) {
      const int64_t rg = row0 + 4 * g;
      const auto ptr_at = [&](int64_t r) { return a.esc_ptr[r < a.n ? r : a.n]; };
      if constexpr (kStage) {
#pragma unroll
        for (int r = 0; r < 5; ++r) st[r] = ptr_at(rg + r);
      }
      rsc.load(a, rg);
    }

    // ---- D virtual steps -D .. -1: the same load pattern as a loop step ----
    // (buffers over the range's blocks only: the ring's refills past the range read zeros)
    Rsrc ra, rl;
    if constexpr (FMT == kFmtBF16) {
      ra = make_rsrc(a.w + row0 * a.k + (int64_t)kb0 * (kTileBF / 2), valid ? nkb * (uint32_t)kTileBF : 0u);
      rl = ra;
    } else {
      ra = make_rsrc(a.ae + row0 * a.k + (int64_t)kb0 * kTileAE, valid ? nkb * (uint32_t)kTileAE : 0u);
      rl = make_rsrc(a.lo + row0 * a.k / 2 + (int64_t)kb0 * kTileLO, valid ? nkb * (uint32_t)kTileLO : 0u);
    }
    ABlock<FMT> buf[D];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load_ablock<FMT>(ra, rl, (uint32_t)d, lane16, buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- the tile's escape list into LDS (its loads go out after the ring's, so the ring is
    // not held behind the wait for the row bounds) ----
    if constexpr (kStage) {
      // escape range of the tile: row0's start (lane 0, g = 0) and row0 + 16's (lane 48, g = 3)
      t_e0 = __builtin_amdgcn_readfirstlane(st[0]);
      const uint32_t t_e1 = valid ? (uint32_t)__builtin_amdgcn_readlane((int)st[4], 48) : t_e0;
      const uint32_t cnt = t_e1 - t_e0 < (uint32_t)kEscCapM ? t_e1 - t_e0 : (uint32_t)kEscCapM;
      t_cnt = cnt;
      if constexpr (kEsc) {
        // global-to-LDS loads: no registers held and no wait here; the end of the range's first
        // chunk waits for them (they went out before any of its loads).  Columns: 64 entries
        // per load.  Values: 128 per load as 4-byte pairs from entry t_e0 rounded down to even
        // (a 4-byte word holding one value of the list lies in the same page as that value).
        t_vsh = t_e0 & 1u;
        const Rsrc r_col = make_rsrc(a.esc_col + t_e0, cnt * 4u);
        const Rsrc r_val = make_rsrc(a.esc_val + (t_e0 - t_vsh), ((cnt + t_vsh) * 2u + 3u) & ~3u);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kEscCapM / 64; ++i)
          if (64u * i < cnt)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r_col, (__attribute__((address_space(3))) void*)&s_ecol[w][64 * i],
                                                     4, 4u * (lane + 64 * i), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kValCap / 128; ++i)
          if (128u * i < cnt + t_vsh)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r_val, (__attribute__((address_space(3))) void*)&s_eval[w][128 * i],
                                                     4, 4u * (lane + 64 * i), 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const Rsrc r_col = make_rsrc(a.esc_col + t_e0, cnt * 4u);
        const Rsrc r_val = make_rsrc(a.esc_val + t_e0, cnt * 2u);
        uint32_t ecol[kEscStage / 64], evalv[kEscStage / 64];
#pragma unroll
        for (int i = 0; i < kEscStage / 64; ++i) {
          ecol[i] = __builtin_amdgcn_raw_buffer_load_b32(r_col, 4u * (lane + 64 * i), 0, 0);
          evalv[i] = __builtin_amdgcn_raw_buffer_load_b16(r_val, 2u * (lane + 64 * i), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kEscStage / 64; ++i) {
          s_ecol[w][lane + 64 * i] = ecol[i];
          s_eval[w][lane + 64 * i] = (uint16_t)evalv[i];
        }
        // a crowded tile: the rest of the LDS copy
        for (uint32_t i = kEscStage + (uint32_t)lane; i < t_cnt; i += 64) {
          s_ecol[w][i] = a.esc_col[t_e0 + i];
          s_eval[w][i] = a.esc_val[t_e0 + i];
        }
      }
      if (!valid) {
#pragma unroll
        for (int r = 0; r < 5; ++r) st[r] = t_e0;
      }
    }
    // chunk 0 is in LDS (its loads went out before the escape metadata and the ring, and the
    // escape copy after them)
    vm_wait_le<D * kLoadsPerStep>();
    lds_barrier();

    // per row r: cursor (absolute escape index) and the column under it (~0: none in LDS)
    const uint32_t lds_end = t_e0 + kEscCapM;
    const auto run_end = [&](int r) { return st[r + 1] < lds_end ? st[r + 1] : lds_end; };
    // (escapes left of the range are skipped; a crowded row whose LDS copy ends before the range
    // starts finds the rest in memory after the loop)
    uint32_t cur[4], ncol[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cur[r] = st[r];
      ncol[r] = 0xFFFFFFFFu;
    }
    floatx4 acc[NT];
    float qv[NT][4], sx[NT][4];
#pragma unroll
    for (int cc = 0; cc < NT; ++cc) {
      acc[cc] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[cc][r] = sx[cc][r] = 0.f;
    }

    for (uint32_t c = c0; c < c1; ++c) {           // chunk c: k-blocks S c .. S c + S - 1
      const uint32_t b = (c - c0) & 1u;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int slot = s % D;
        const uint32_t kb = S * (c - c0) + s;      // block within the range
        uint32_t p[16];
        ablock_pairs<FMT>(buf[slot], e112, p);
        if constexpr (FMT != kFmtBF16) pin16(p);
        __builtin_amdgcn_sched_barrier(0);
        // x: the wave's fragments FPS s .. FPS s + FPS - 1 of the next chunk at step s of a chunk
        // (spread over the steps, so the weight stream never queues behind a burst of them)
#pragma unroll
        for (int i = FPS * s; i < FPS * (s + 1) && i < FW; ++i) x_fetch_one(c + 1, b ^ 1u, i);
        // A ring: refill this slot with block kb + D (dense blocks are their own A operands and
        // are refilled after the MFMAs below)
        if constexpr (FMT != kFmtBF16) load_ablock<FMT>(ra, rl, kb + D, lane16, buf[slot]);

        const u32x4* xb = &s_x[b][0];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4 av = {p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]};
#pragma unroll
          for (int cc = 0; cc < NT; ++cc) {
            const u32x4 bv = xb[(s >> 1) * 512 * NT + 512 * cc + xo[(s + cc) & 1][t]];
            acc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bv), acc[cc],
                                                             0, 0, 0);
          }
        }
        if constexpr (FMT == kFmtBF16) load_ablock<FMT>(ra, rl, kb + D, lane16, buf[slot]);
        __builtin_amdgcn_sched_barrier(0);
      }

      if constexpr (kEsc) {
        if (c == c0) {
          // the escape copy has landed: the chunk's steps issued FW fragment loads and S ring
          // refills after it
          vm_wait_le<FW + S * kLoadsPerStep>();
          // first escape at or right of col0 of each row (runs are sorted by column): the four
          // binary searches in lockstep, branch-free, so each halving issues its four LDS reads
          // together, until every lane's searches have closed; none for the first range
          uint32_t hi[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hi[r] = run_end(r);
          if (col0 > 0) {
            for (int it = 0; it < 10; ++it) {
              bool open_any = false;
#pragma unroll
              for (int r = 0; r < 4; ++r) open_any |= cur[r] < hi[r];
              if (!__builtin_amdgcn_ballot_w64(open_any)) break;
              uint32_t v[4], mid[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                mid[r] = (cur[r] + hi[r]) >> 1;
                const uint32_t at = mid[r] - t_e0;
                v[r] = s_ecol[w][at < (uint32_t)kEscCapM ? at : 0u];
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const bool open = cur[r] < hi[r];
                const bool right = v[r] < col0;
                cur[r] = open && right ? mid[r] + 1 : cur[r];
                hi[r] = open && !right ? mid[r] : hi[r];
              }
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) ncol[r] = cur[r] < run_end(r) ? s_ecol[w][cur[r] - t_e0] : 0xFFFFFFFFu;
        }
        // escapes of rows 4g..4g+3 with a column in this chunk, x from LDS buffer b
        const uint32_t lim = 128u * S * (c + 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          while (ncol[r] < lim) {
            const uint32_t e = cur[r] - t_e0;
            const uint32_t col = ncol[r] - 128u * S * c;
            const float v = bf16_to_float(s_eval[w][e + t_vsh]);
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              const uint32_t at = x_slot(col >> 8, 16u * cc + (uint32_t)r16, (col >> 3) & 31u);
              const float xv = bf16_to_float(reinterpret_cast<const uint16_t*>(&s_x[b][at])[col & 7u]);
              sx[cc][r] += xv;
              qv[cc][r] = fmaf(xv, v, qv[cc][r]);
            }
            cur[r] += 1;
            ncol[r] = cur[r] < run_end(r) ? s_ecol[w][e + 1] : 0xFFFFFFFFu;
          }
        }
      }
      // the next chunk is in LDS: the wave's last fragment load went out at step LS, before that
      // step's refill
      vm_wait_le<(S - LS) * kLoadsPerStep>();
      lds_barrier();
    }

    if (!valid) continue;
    if constexpr (kEsc) {
      // escapes beyond the LDS copy of a crowded tile, four at a time (their loads issued
      // together, then the x values they select).  A walk that stopped inside the copy stopped at
      // a column past the range (runs are sorted) or at the row's end: nothing is left for it.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        for (uint32_t e = cur[r] >= lds_end ? cur[r] : st[r + 1]; e < st[r + 1]; e += 4) {
          uint32_t col[4], vb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool in = e + i < st[r + 1];
            col[i] = in ? a.esc_col[e + i] : 0xFFFFFFFFu;
            vb[i] = in ? a.esc_val[e + i] : 0u;
          }
          float xv[4][NT];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              const int mrow = 16 * cc + r16;
              const bool use = col[i] >= col0 && col[i] < col1 && mrow < a.m;
              xv[i][cc] = use ? bf16_to_float(a.x[(int64_t)mrow * a.k + col[i]]) : 0.0f;
            }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (col[i] < col0 || col[i] >= col1) continue;
            const float v = bf16_to_float(vb[i]);
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              sx[cc][r] += xv[i][cc];
              qv[cc][r] = fmaf(xv[i][cc], v, qv[cc][r]);
            }
          }
          if (col[3] >= col1) break;
        }
      }
    }
    uint64_t best[NT];
#pragma unroll
    for (int cc = 0; cc < NT; ++cc) best[cc] = 0;
    if constexpr (kEscEpi) {
      // the escapes of the lane's four rows, four at a time: entries from the LDS copy (memory
      // past it in a crowded tile), x values from the transposed x (the lane's eight x rows in
      // one 16-byte load); the placeholder terms come out of acc, the escape values go to q, and
      // the row's outputs are then final in acc
      static_assert(NT == 8, "the transposed x holds eight activation tiles");
      const uint32_t lds_lim = t_e0 + t_cnt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float q[NT];
#pragma unroll
        for (int cc = 0; cc < NT; ++cc) q[cc] = 0.f;
        for (uint32_t e = st[r]; e < st[r + 1]; e += 4) {
          uint32_t col[4];
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t ei = e + i;
            const bool in = ei < st[r + 1];
            const bool lds = ei < lds_lim;
            const uint32_t at = lds ? ei - t_e0 : 0u;
            col[i] = !in ? 0u : lds ? s_ecol[w][at] : a.esc_col[ei];
            v[i] = !in ? 0.f : bf16_to_float(lds ? s_eval[w][at] : a.esc_val[ei]);
          }
          u32x4 xw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xw[i] = e + i < st[r + 1]
                        ? *reinterpret_cast<const u32x4*>(a.xt + (int64_t)col[i] * 128 + 8 * r16)
                        : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (e + i >= st[r + 1]) break;
#pragma unroll
            for (int cc = 0; cc < NT; ++cc) {
              const uint32_t wd = xw[i][cc >> 1];
              const float xv = __builtin_bit_cast(float, (cc & 1) ? wd & 0xFFFF0000u : wd << 16);
              if constexpr (has_placeholder<FMT>()) acc[cc][r] = fmaf(-xv, placeholder_of<FMT>(), acc[cc][r]);
              q[cc] = fmaf(xv, v[i], q[cc]);
            }
          }
        }
        const float sc = rsc.get(r);
#pragma unroll
        for (int cc = 0; cc < NT; ++cc) acc[cc][r] = fmaf(sc, acc[cc][r], q[cc]);
      }
    }
    if constexpr (SILU) {
      // SiLU(gate) * up: lanes g = 0, 1 hold gate rows 4 g .. 4 g + 3 of x row 16 cc + r16, lanes
      // g + 2 (lane ^ 32) the matching up rows; h gets 4 consecutive outputs per lane
      const int64_t ldh = a.ldy >> 1;
#pragma unroll
      for (int cc = 0; cc < NT; ++cc) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = kEsc ? fmaf(rsc.get(r), has_placeholder<FMT>() ? fmaf(-sx[cc][r], placeholder_of<FMT>(), acc[cc][r])
                                                                       : acc[cc][r], qv[cc][r])
                               : acc[cc][r];
          const float up = __shfl_xor(v, 32);
          hv[r] = silu(v) * up;
        }
        const int mcol = 16 * cc + r16;
        if (g < 2 && mcol < a.m) {
          const int64_t at = mcol * ldh + row0 / 2 + 4 * g;
          if (a.y16) {
            const u32x2 pk = {(uint32_t)float_to_bf16_rne(hv[0]) | (uint32_t)float_to_bf16_rne(hv[1]) << 16,
                              (uint32_t)float_to_bf16_rne(hv[2]) | (uint32_t)float_to_bf16_rne(hv[3]) << 16};
            if (a.yvec) {
              *reinterpret_cast<u32x2*>(&a.y16[at]) = pk;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) a.y16[at + i] = float_to_bf16_rne(hv[i]);
            }
          } else if (a.yvec) {
            *reinterpret_cast<floatx4*>(&yout[at]) = (floatx4){hv[0], hv[1], hv[2], hv[3]};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) yout[at + i] = hv[i];
          }
        }
      }
    } else if constexpr (!TOP1) {
      // lane (g, r16) holds rows 4 g .. 4 g + 3 of x row 16 cc + r16: written to the wave's part of
      // the idle x buffer as [x row][20 floats] (4 of padding), read back so that lane l holds
      // rows 4 (l % 4) .. +3 of x row 16 j + l / 4, and stored as one 16-byte vector (or four
      // floats when y is not 16-byte aligned).  Every wave is past the last chunk's barrier, and
      // the next tile's loads into this buffer wait for the barrier at its start.
      // (two activation tiles at a time: the region of eight would not fit)
      constexpr int CG = NT < 2 ? NT : 2;
      float* res = reinterpret_cast<float*>(&s_x[0][0]) + w * (16 * CG * 20);
      const int q = lane & 3;
#pragma unroll
      for (int c0g = 0; c0g < NT; c0g += CG) {
      if (c0g > 0) __builtin_amdgcn_wave_barrier();   // the group before has read its region
#pragma unroll
      for (int cc = c0g; cc < c0g + CG; ++cc) {
        float v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v4[r] = kEsc ? fmaf(rsc.get(r), has_placeholder<FMT>() ? fmaf(-sx[cc][r], placeholder_of<FMT>(), acc[cc][r])
                                                                  : acc[cc][r], qv[cc][r])
                       : acc[cc][r];
        }
        *reinterpret_cast<floatx4*>(&res[(16 * (cc - c0g) + r16) * 20 + 4 * g]) = (floatx4){v4[0], v4[1], v4[2], v4[3]};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = c0g; j < c0g + CG; ++j) {
        const int mcol = 16 * j + (lane >> 2);
        const floatx4 o = *reinterpret_cast<const floatx4*>(&res[(16 * (j - c0g) + (lane >> 2)) * 20 + 4 * q]);
        const int64_t nrow = row0 + 4 * q;
        if (mcol < a.m && a.y16) {
          uint16_t* yq = &a.y16[mcol * a.ldy + nrow];
          if (a.yvec && nrow + 3 < a.n) {
            const u32x2 pk = {(uint32_t)float_to_bf16_rne(o[0]) | (uint32_t)float_to_bf16_rne(o[1]) << 16,
                              (uint32_t)float_to_bf16_rne(o[2]) | (uint32_t)float_to_bf16_rne(o[3]) << 16};
            *reinterpret_cast<u32x2*>(yq) = pk;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (nrow + i < a.n) yq[i] = float_to_bf16_rne(o[i]);
          }
        } else if (mcol < a.m) {
          float* yp = &yout[mcol * a.ldy + nrow];
          if (a.yvec) {
            if (nrow < a.n) *reinterpret_cast<floatx4*>(yp) = o;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (nrow + i < a.n) yp[i] = o[i];
          }
        }
      }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t nrow = row0 + 4 * g + r;
        if (nrow >= a.n) continue;
        const float sc = rsc.get(r);
#pragma unroll
        for (int cc = 0; cc < NT; ++cc) {
          const int mcol = 16 * cc + r16;
          if (mcol >= a.m) continue;
          const float v = kEsc ? fmaf(sc, has_placeholder<FMT>() ? fmaf(-sx[cc][r], placeholder_of<FMT>(), acc[cc][r])
                                                                 : acc[cc][r], qv[cc][r])
                               : acc[cc][r];   // (with kEscEpi acc is already final)
          const uint64_t key = top1_key(v, nrow);
          best[cc] = key > best[cc] ? key : best[cc];
        }
      }
    }
    if constexpr (TOP1) {
      // the tile's best row per x row: over the four row groups g (lanes r16 + 16 g), then over
      // the workgroup's waves through LDS
#pragma unroll
      for (int cc = 0; cc < NT; ++cc) {
#pragma unroll
        for (int sh = 16; sh <= 32; sh *= 2) {
          const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best[cc], sh, 64);
          const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best[cc] >> 32), sh, 64);
          const uint64_t o = ((uint64_t)hi << 32) | lo;
          best[cc] = o > best[cc] ? o : best[cc];
        }
        if (g == 0 && 16 * cc + r16 < a.m) atomicMax(&s_best[16 * cc + r16], (unsigned long long)best[cc]);
      }
    }
  }
  if constexpr (TOP1) {
    lds_barrier();
    if (tid < 32) a.top1[(int64_t)blockIdx.x * 32 + tid] = s_best[tid];
  }
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
template <int FMT, int W>
static MfmaKernel pick(int nt) {
  if constexpr (W == 12 && FMT != kFmtI8)   // the 8-bit copy runs passes of at most 64 rows
    if (nt == 8) return k_mfma<FMT, 8, W, false>;
  if (nt >= 3) return mfma_wide_kernel(static_cast<Fmt>(FMT), nt);
  return nt == 1 ? k_mfma<FMT, 1, W, false> : k_mfma<FMT, 2, W, false>;
}

// top-1 mode: the exact pass or the Q pass (truncated or midpoint), one or two activation tiles,
// 12 waves
static MfmaKernel pick_top1(Fmt f, int nt) {
  if (f == kFmtW12) return nt == 1 ? k_mfma<kFmtW12, 1, kWaves, true> : k_mfma<kFmtW12, 2, kWaves, true>;
  if (f == kFmtQ8M) return nt == 1 ? k_mfma<kFmtQ8M, 1, kWaves, true> : k_mfma<kFmtQ8M, 2, kWaves, true>;
  if (f == kFmtI8) return nt == 1 ? k_mfma<kFmtI8, 1, kWaves, true> : k_mfma<kFmtI8, 2, kWaves, true>;
  return nt == 1 ? k_mfma<kFmtQ8, 1, kWaves, true> : k_mfma<kFmtQ8, 2, kWaves, true>;
}

// the exact pass with the SiLU(gate) * up epilogue (instantiated apart, so the other kernels keep
// their registers)
static MfmaKernel pick_silu(int nt) {
  if (nt == 8) return k_mfma<kFmtW12, 8, kWaves, false, true>;
  if (nt >= 3) return mfma_wide_kernel(kFmtW12, nt, true);
  return nt == 1 ? k_mfma<kFmtW12, 1, kWaves, false, true> : k_mfma<kFmtW12, 2, kWaves, false, true>;
}

static MfmaKernel pick_kernel(Fmt f, int nt, int waves, bool silu) {
  if (silu) return pick_silu(nt);
  if (waves == 8) return pick<kFmtBF16, 8>(nt);   // only the dense baseline runs 8 waves
  if (f == kFmtW12) return pick<kFmtW12, 12>(nt);
  if (f == kFmtQ8) return pick<kFmtQ8, 12>(nt);
  if (f == kFmtQ8M) return pick<kFmtQ8M, 12>(nt);
  if (f == kFmtI8) return pick<kFmtI8, 12>(nt);
  return pick<kFmtBF16, 12>(nt);
}

// One launch (plus the split-k sum) for mb <= 64 rows of x over the n rows of `p`, output rows
// y[j * ldy + 0 .. n).
// Partial sums of a split go to the workspace from byte ws_off on.
static hipError_t mfma_pass(Fmt f, const DevInfo& di, const uint16_t* x, int mb, const Planes& p,
                            int64_t n, int64_t k, YOut y, int64_t ldy, hipStream_t s,
                            const Scratch& sc, size_t ws_off = 0) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t kb = k / kTileCols;
  const int nt = mb > 64 ? 8 : (mb + 15) / 16;   // 65..128 rows: the eight-tile instantiation
  // Up to two activation tiles: the dense baseline runs 8 waves per CU with 8 blocks in flight
  // when every tile fits one round of them (measured faster there), the W12 and Q8 kernels
  // always 12 waves with 4 (their decode needs three waves per SIMD to hide: 8 waves measured
  // 49 us against 39 us on W [17408, 5120] at 32 rows).  k ranges: as many as give every wave
  // a tile when the shape has few tiles (at least 2), with at least 4 blocks (W12, Q8: one
  // chunk) or 8 (dense) in each; their partial outputs must fit the workspace.  (Longer W12
  // ranges measured slower on every layer shape: at 32 rows, W [6144, 5120] 21.8 us with ranges
  // of 8 blocks, 24.6 with 16, 30.5 with 24.)
  int waves = kWaves;
  int64_t chunk_blocks = nt == 8 ? 2 : kChunkBlocks;
  int64_t ranges = 1;
  if (nt <= 2) {
    if (f == kFmtBF16 && tiles <= (int64_t)di.cus * 8) {
      waves = 8;
      chunk_blocks = 8;
    }
    const int64_t chunks = (kb + chunk_blocks - 1) / chunk_blocks;
    ranges = (int64_t)di.cus * waves / tiles;
    const int64_t cap = chunks * chunk_blocks / (f == kFmtBF16 ? 8 : 4);
    if (ranges > cap) ranges = cap;
    if ((size_t)ranges * mb * n * sizeof(float) > sc.bytes - ws_off)
      ranges = (int64_t)((sc.bytes - ws_off) / ((size_t)mb * n * sizeof(float)));
    if (ranges < 2) ranges = 1;
  }
  const int64_t chunks = (kb + chunk_blocks - 1) / chunk_blocks;
  const int64_t cps = (chunks + ranges - 1) / ranges;
  ranges = (chunks + cps - 1) / cps;
  float* ws = nullptr;
  if (ranges > 1) {
    hipError_t err = sc.get(&ws);
    if (err != hipSuccess) return err;
    ws += ws_off / sizeof(float);
  }
  int64_t groups = di.cus / ranges;
  if (groups > tiles) groups = tiles;
  if (groups < 1) groups = 1;
  MfmaArgs a;
  a.x = x;
  a.m = mb;
  a.base = p.base; a.ae = p.ae; a.lo = p.lo;
  a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
  a.w = p.w;
  a.scale = p.scale;
  a.y = ws ? ws : y.f;
  a.y16 = ws ? nullptr : y.h;
  const bool silu = !ws && y.silu;             // a split pairs the outputs in its sum instead
  a.ldy = ws ? n : ldy;                        // partial slices are [mb][n], contiguous
  a.n = n; a.k = k;
  a.rounds = (int)((tiles + groups * waves - 1) / (groups * waves));
  a.splits = (int)ranges;
  a.cps = (int)cps;
  a.ysplit = (int64_t)mb * n;
  a.top1 = nullptr;
  // vector stores: 16 bytes of float (y 16-byte aligned) or 8 of bfloat16 (y16 8-byte aligned)
  {
    const int64_t ld_out = silu ? a.ldy / 2 : a.ldy;     // row stride of what is stored
    a.yvec = a.y16 ? (reinterpret_cast<uintptr_t>(a.y16) & 7u) == 0 && ld_out % 4 == 0
                   : a.y && (reinterpret_cast<uintptr_t>(a.y) & 15u) == 0 && ld_out % 4 == 0;
  }
  a.xt = nullptr;
  if (nt == 8 && f != kFmtBF16) {
    // x transposed into the workspace for the epilogue's escape patch (no split here)
    float* wsx = nullptr;
    hipError_t e = sc.get(&wsx);
    if (e != hipSuccess) return e;
    uint16_t* xt = reinterpret_cast<uint16_t*>(wsx);
    e = launch_x_transpose(x, mb, k, xt, s);
    if (e != hipSuccess) return e;
    a.xt = xt;
  }
  hipLaunchKernelGGL(pick_kernel(f, nt, waves, silu), dim3((unsigned)(groups * ranges)), dim3(64 * waves), 0,
                     s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ws) return launch_split_reduce(ws, (int)ranges, mb, n, y, ldy, s);
  return hipSuccess;
}

// First row of the tail launch (0: none) -- see launch_mfma.
static int64_t tail_split_row(const DevInfo& di, int mb, int64_t tiles) {
  const int64_t per_round = (int64_t)di.cus * kWaves;
  const int64_t full = tiles / per_round, tail = tiles - full * per_round;
  return mb <= 32 && full >= 1 && tail > 0 && 2 * tail <= per_round ? full * per_round * kTileRows : 0;
}

hipError_t launch_mfma(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                       YOut y, hipStream_t s, const Scratch& sc) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  // passes of up to 128 rows of x (each reads the weights once); the W12 and Q8 passes of more
  // than 64 rows need x transposed in the workspace, else they stay at 64.  The kernels address
  // x with 32-bit byte offsets (2 * rows * k), so a pass of 128 rows also needs 256 k < 2^32.
  const bool wide_ok = f == kFmtBF16 ? 256 * k < (int64_t(1) << 32)
                      : f == kFmtI8   ? false
                                      : k * 128 * 2 <= (int64_t)sc.bytes;
  const int64_t max_step = wide_ok ? 128 : 64;
  for (int64_t m0 = 0, step = 0; m0 < m; m0 += step) {
    step = (m - m0) < max_step ? (m - m0) : max_step;
    // Fewer than 1.5 tiles per CU: passes of 32 rows, which split k over the chip's waves, instead
    // of the wider kernels, which give each wave a whole tile (W12 at 64 / 128 rows, us: [5120,
    // 17408] 70.7 / 141.1 against 207.5 / 254.8, [1024, 5120] 24.0 / 47.2 against 46.8 / 81.1,
    // [5120, 6144] 41.0 / 79.5 against 64.9 / 98.8).
    if (step > 32 && 2 * tiles < 3 * (int64_t)di.cus) step = 32;
    const int mb = (int)step;
    // A shape with more tiles than the chip's waves runs in rounds of one tile per wave; when the
    // last round would keep at most half of the waves busy (the LM head: 9504 tiles = 3 rounds
    // of 3072 and 288), the full rounds run as one launch and the remaining tiles as a second,
    // split-k launch over the same record's last rows, so they take a fraction of a round.
    const int64_t r0 = tail_split_row(di, mb, tiles);
    if (r0 > 0) {
      err = mfma_pass(f, di, x + m0 * k, mb, p, r0, k, y + m0 * n, n, s, sc);
      if (err != hipSuccess) return err;
      err = mfma_pass(f, di, x + m0 * k, mb, rows_from(p, r0, k), n - r0, k, y + m0 * n + r0, n, s, sc);
    } else {
      err = mfma_pass(f, di, x + m0 * k, mb, p, n, k, y + m0 * n, n, s, sc);
    }
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_mfma_top1(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n,
                            int64_t k, int32_t* idx, float* val, hipStream_t s) {
  DevInfo di;
  hipError_t err = dev_info(&di);
  if (err != hipSuccess) return err;
  // workspace: per-workgroup keys [groups + 1][32] at 0 (at most 257 x 32 x 8 bytes); the tail's
  // outputs [32][n - r0] (at most 32 x 1536 tiles x 16 rows x 4 bytes) from 128 KiB; the tail's
  // split partial sums from 4 MiB
  Scratch sc;
  sc.s = s;
  float* ws = nullptr;
  err = sc.get(&ws);
  if (err != hipSuccess) return err;
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws);
  float* ytail = ws + (size_t(128) << 10) / sizeof(float);
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t kb = k / kTileCols;
  for (int64_t m0 = 0; m0 < m; m0 += 32) {
    const int mb = (int)((m - m0) < 32 ? (m - m0) : 32);
    const int nt = (mb + 15) / 16;
    // the same launches as the full outputs: the full rounds in top-1 mode, the tail rows (if
    // any) through the split path into the workspace and then scanned for their best key
    const int64_t r0 = tail_split_row(di, mb, tiles);
    const int64_t nh = r0 > 0 ? r0 : n;
    const int64_t th = (nh + kTileRows - 1) / kTileRows;
    const int64_t groups = th < di.cus ? th : di.cus;
    MfmaArgs a;
    a.x = x + m0 * k;
    a.m = mb;
    a.base = p.base; a.ae = p.ae; a.lo = p.lo;
    a.esc_ptr = p.esc_ptr; a.esc_col = p.esc_col; a.esc_val = p.esc_val;
    a.w = p.w;
    a.scale = p.scale;
    a.y = nullptr;
    a.y16 = nullptr;
    a.ldy = nh;
    a.n = nh; a.k = k;
    a.rounds = (int)((th + groups * kWaves - 1) / (groups * kWaves));
    a.splits = 1;
    a.cps = (int)((kb + kChunkBlocks - 1) / kChunkBlocks);
    a.ysplit = 0;
    a.top1 = keys;
    a.yvec = 0;
    a.xt = nullptr;
    hipLaunchKernelGGL(pick_top1(f, nt), dim3((unsigned)groups), dim3(64 * kWaves), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    int g_all = (int)groups;
    if (r0 > 0) {
      err = mfma_pass(f, di, x + m0 * k, mb, rows_from(p, r0, k), n - r0, k, yout_f(ytail), n - r0, s,
                      sc, size_t(4) << 20);
      if (err != hipSuccess) return err;
      err = launch_top1_rows(ytail, mb, n - r0, r0, keys + (int64_t)groups * 32, s);
      if (err != hipSuccess) return err;
      g_all += 1;
    }
    err = launch_top1_final(keys, g_all, mb, idx + m0, val + m0, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace w12
