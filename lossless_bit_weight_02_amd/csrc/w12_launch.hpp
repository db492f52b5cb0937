// Host-side launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

// kFmtQ8M: the Q pass with the dropped B nibble read as 8 (the midpoint of its 16 values);
// kFmtI8: the Q pass on the separate 8-bit copy (int8 codes in the AE plane's storage order, one
// float scale per row, escapes exact from the record's list)
enum Fmt : int { kFmtW12 = 0, kFmtQ8 = 1, kFmtBF16 = 2, kFmtQ8M = 3, kFmtI8 = 4 };

struct DevInfo {
  int device = -1;
  int cus = 0;          // compute units
  int max_lds = 0;      // bytes of LDS one workgroup may use
};
// Properties of the current device (cached per device id).
hipError_t dev_info(DevInfo* out);

// Device workspace for the partial sums of split-k GEMMs: kWorkspaceBytes per (device, stream),
// allocated on the first call that needs it on that stream and kept until the process ends.
constexpr size_t kWorkspaceBytes = size_t(64) << 20;
hipError_t workspace(hipStream_t s, float** out);

// The scratch memory one GEMM call may use: the per-stream workspace above (allocated on first
// use), or a fixed device buffer of `bytes` bytes (`fixed`, nothing is allocated).  Split-k
// ranges and 128-row passes adapt to `bytes`; only the GEMV's bfloat16 outputs over several
// k slices need a fixed amount (rows x n floats).
struct Scratch {
  hipStream_t s = nullptr;
  void* fixed = nullptr;
  size_t bytes = kWorkspaceBytes;
  hipError_t get(float** out) const {
    if (fixed) {
      *out = static_cast<float*>(fixed);
      return hipSuccess;
    }
    return workspace(s, out);
  }
};

// The fixed scratch of the allocation-free entry point: kScratchBytes of file-scope device memory
// per device, looked up once per device (noalloc.hip).
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t fixed_scratch(void** out);

// Where a GEMM writes y: float (f), or bfloat16 bits rounded to nearest even from the float
// result (h); exactly one of them is set.  With `silu`, the n outputs of a row pair up as the
// gate and up halves of row-interleaved gate+up weights (rows 16 t .. 16 t + 7 gate, 16 t + 8 ..
// 16 t + 15 up) and the array holds h[j][i] = silu(y[j][gate row of i]) * y[j][up row of i],
// [m][n / 2]; offsets are still given in elements of y (multiples of 16 within a row), so they
// halve.  Offsets count elements of either.
struct YOut {
  float* f = nullptr;
  uint16_t* h = nullptr;
  bool silu = false;
  YOut operator+(int64_t off) const {
    YOut r;
    const int64_t o = silu ? off / 2 : off;
    r.f = f ? f + o : nullptr;
    r.h = h ? h + o : nullptr;
    r.silu = silu;
    return r;
  }
};
inline YOut yout_f(float* f) {
  YOut r;
  r.f = f;
  return r;
}

// y[r * ldy + c] = sum over j = 0 .. splits-1 (in that order) of part[j * rows * cols + r * cols + c],
// r < rows, c < cols (splits = 1: a copy, or with y.h the rounding to bfloat16); with y.silu the
// sums pair up into h[r * ldy / 2 + i], i < cols / 2 (see YOut)
hipError_t launch_split_reduce(const float* part, int splits, int64_t rows, int64_t cols, YOut y,
                               int64_t ldy, hipStream_t s);

// best key of each row of y [m][cols] (row index row0 + column), into keys[0 .. m)
hipError_t launch_top1_rows(const float* y, int m, int64_t cols, int64_t row0, uint64_t* keys, hipStream_t s);
// top-1 per x row from per-workgroup keys [groups][32] (the top-1 modes of the matrix-core and
// streaming kernels)
hipError_t launch_top1_final(const uint64_t* part, int groups, int m, int32_t* idx, float* val,
                             hipStream_t s);

// Rows of the padded (tiled) plane storage.
inline int64_t padded_rows(int64_t n) { return (n + 15) / 16 * 16; }

struct Planes {
  const uint8_t* base = nullptr;
  const uint8_t* ae = nullptr;
  const uint8_t* lo = nullptr;
  const uint32_t* esc_ptr = nullptr;
  const uint32_t* esc_col = nullptr;
  const uint16_t* esc_val = nullptr;
  const uint16_t* w = nullptr;  // kFmtBF16 only: the dense bfloat16 weight, tiled storage order
  const float* scale = nullptr; // kFmtI8 only: per-row scale (the codes are in `ae`)
};

// The record's rows r0 .. n as a record of their own (r0 a multiple of 16; escape offsets stay
// absolute indices into the escape arrays).
inline Planes rows_from(const Planes& p, int64_t r0, int64_t k) {
  Planes t = p;
  if (t.base) t.base += r0;
  if (t.ae) t.ae += r0 * k;
  if (t.lo) t.lo += r0 * k / 2;
  if (t.esc_ptr) t.esc_ptr += r0;
  if (t.w) t.w += r0 * k;
  if (t.scale) t.scale += r0;
  return t;
}

// x [m <= 128][k] bfloat16 -> xt [k][16][8], xt[c][r][t] = x[16 t + r][c] (rows past m zero),
// for the eight-tile GEMM's escapes
hipError_t launch_x_transpose(const uint16_t* x, int m, int64_t k, uint16_t* xt, hipStream_t s);

// encoder: window choice per row (writes base[n] and the escape count of row i to esc_ptr[i+1])
hipError_t launch_analyze(const uint16_t* w, int64_t n, int64_t k, uint8_t* base, uint32_t* esc_ptr,
                          hipStream_t s);
// encoder: in-place inclusive scan of esc_ptr[1..n], esc_ptr[0] = 0; totals >= 2^32-1 saturate
hipError_t launch_scan(uint32_t* esc_ptr, int64_t n, hipStream_t s);
// encoder: planes and escapes
hipError_t launch_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* base,
                       const uint32_t* esc_ptr, uint8_t* ae, uint8_t* lo, uint32_t* esc_col,
                       uint16_t* esc_val, hipStream_t s);
// decoder: planes -> bfloat16 bits, then every escape written over its slot
hipError_t launch_decode(const Planes& p, int64_t n, int64_t k, uint16_t* out, hipStream_t s);
// dst[i] = src[i] + add, i < cnt (escape offsets of a part placed after earlier parts)
hipError_t launch_rebase(const uint32_t* src, int64_t cnt, uint32_t add, uint32_t* dst, hipStream_t s);
// record of the row-interleaved gate+up weights (rows 16 t .. +7 = gate rows 8 t .. +7, rows
// 16 t + 8 .. +15 = up rows 8 t .. +7) from the two records; esc_total[2] = the parts' escape totals
hipError_t launch_interleave(const Planes& gate, const Planes& up, int64_t rows, int64_t k, uint8_t* base,
                             uint8_t* ae, uint8_t* lo, uint32_t* esc_ptr, uint32_t* esc_col, uint16_t* esc_val,
                             hipStream_t s);
// 8-bit Q-pass copy of a record: per-row scales, codes in the AE storage order, escaped slots 0
hipError_t launch_i8_build(const Planes& p, int64_t n, int64_t k, int8_t* q, float* scale, hipStream_t s);
// dense bf16 [n][k] -> tiled storage order (baseline layout)
hipError_t launch_bf16_tile(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, hipStream_t s);
// bandwidth probe
hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s);

// Columns of x one GEMV launch over mb (<= 8) rows holds in LDS: longer rows run as k slices.
int64_t gemv_k_slice(const DevInfo& di, int mb);
// GEMV family (wave-reduction kernel), any m (passes of <= 8 rows of x)
hipError_t launch_gemv(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                       YOut y, hipStream_t s, const Scratch& sc);
// Streaming family (one workgroup per CU owning whole tiles, every wave an equal share of their
// blocks, x in LDS by k phases): passes of <= 64 rows of x, and shapes with more tiles than one
// per wave of the chip (three for 3..16 rows) in equal groups of rows, one launch
// for all; stream_fits says whether a shape can run it; no SiLU pairing
bool stream_fits(const DevInfo& di, Fmt f, int64_t m, int64_t n, int64_t k);
// keys (top-1 mode, m <= 32): y is not written; workgroup b's best key of x row j goes to
// keys[32 b + j] and *key_groups = the grid size
hipError_t launch_stream(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                         YOut y, hipStream_t s, uint64_t* keys = nullptr, int* key_groups = nullptr);
// Top-1 per row of x through the streaming kernel: its workgroups reduce their outputs to one key
// per x row, then the per-row reduction over the workgroups; m <= 32 and the keys within the
// workspace (stream_top1_fits)
bool stream_top1_fits(const DevInfo& di, Fmt f, int64_t m, int64_t n, int64_t k);
hipError_t launch_stream_top1(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                              int32_t* idx, float* val, hipStream_t s);
// MFMA family (bf16 v_mfma_f32_16x16x32), any m (blocks of <= 64 rows of x)
hipError_t launch_mfma(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n, int64_t k,
                       YOut y, hipStream_t s, const Scratch& sc);
// top-1 over the n outputs of each x row (no y written), passes of <= 32 rows of x
hipError_t launch_mfma_top1(Fmt f, const uint16_t* x, int64_t m, const Planes& p, int64_t n,
                            int64_t k, int32_t* idx, float* val, hipStream_t s);

}  // namespace w12
