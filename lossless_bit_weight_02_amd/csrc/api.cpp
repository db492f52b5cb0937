// C ABI of libw12.so (declared in include/w12.h): argument checks, path choice, launches.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "w12.h"
#include "w12_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return W12_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(W12_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static_assert(W12_NOALLOC_SCRATCH_BYTES == w12::kScratchBytes, "w12.h states the fixed scratch size");

constexpr int64_t kMaxDim = int64_t(1) << 31;  // n and m below 2^31
constexpr int64_t kMaxK = int64_t(1) << 24;    // k at most 2^24: 32-bit buffer offsets in kernels

int check_nk(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return fail(W12_ERR_ARG, "n and k must be positive (n=%lld, k=%lld)",
                                    (long long)n, (long long)k);
  if (n >= kMaxDim || k > kMaxK) return fail(W12_ERR_RANGE, "n or k too large (n < 2^31, k <= 2^24)");
  if (k % 128 != 0) return fail(W12_ERR_SHAPE, "k must be a multiple of 128 (k=%lld)", (long long)k);
  return W12_OK;
}

int check_record(const w12_weight* wt, bool need_lo) {
  if (!wt) return fail(W12_ERR_ARG, "weight record is NULL");
  int rc = check_nk(wt->n, wt->k);
  if (rc) return rc;
  if (!wt->base || !wt->ae || !wt->esc_ptr || (need_lo && !wt->lo))
    return fail(W12_ERR_ARG, "a plane pointer of the record is NULL");
  if (wt->esc_cap > 0 && (!wt->esc_col || !wt->esc_val))
    return fail(W12_ERR_ARG, "escape arrays are NULL but esc_cap > 0");
  if (!aligned16(wt->ae) || (need_lo && !aligned16(wt->lo)))
    return fail(W12_ERR_ALIGN, "ae and lo must be 16-byte aligned");
  if (!aligned4(wt->esc_ptr) || (wt->esc_col && !aligned4(wt->esc_col)) ||
      (wt->esc_val && (reinterpret_cast<uintptr_t>(wt->esc_val) & 1u)))
    return fail(W12_ERR_ALIGN, "escape arrays must be naturally aligned");
  return W12_OK;
}

w12::Planes planes_of(const w12_weight* wt) {
  w12::Planes p;
  p.base = wt->base;
  p.ae = wt->ae;
  p.lo = wt->lo;
  p.esc_ptr = wt->esc_ptr;
  p.esc_col = wt->esc_col;
  p.esc_val = wt->esc_val;
  return p;
}

// The streaming kernel where it measured fastest (us, streaming vs the best other family, on
// 27B-class shapes, W12): 3..16 rows on shapes of at least 1.5 tiles per CU with rows of at
// most 8192 columns ([34816, 5120]: 4 rows 46.4 vs 47.7, 8 rows 47.2 vs 47.9, 16 rows 46.8 vs
// 48.6; [17408, 5120], 16 rows: 29.3 vs 32.8; [8192, 5120], 4 rows: 15.8 vs 18.3; [6144, 5120],
// 16 rows: 17.8 vs 20.2), and 17..32 rows on at least 2 tiles per CU ([17408, 5120]: 34.2 vs
// 37.4, [8192, 5120]: 25.0 vs 26.2; [6144, 5120]: 24.1 vs 23.0, not taken).  Long rows
// ([5120, 17408]) and shapes of 1.25 tiles per CU or fewer run the other families, and so does
// the dense baseline above 6 tiles per CU (its own measurement: [34816, 5120], 4 rows 56.9 vs
// 55.8, 32 rows 59.5 vs 57.8).  Up to 16 rows a wave finalises up to three tiles, at 17..32 two
// (with more, row groups in one launch): the LM-head-like [152064, 5120] takes 133.3 vs 138.8
// (Q pass) and 181.2 vs 193.5 (exact) at 4 rows, 131.1 vs 148.8 and 183.1 vs 206.7 at 16 rows,
// 164.4 vs 164.7 and 209.8 vs 219.4 at 32 rows (two groups); [65536, 5120] at 32 rows 75.6 vs
// 88.3 and 90.9 vs 111.3 (one group).  So at 17..32 rows the 8-bit passes take it up to 24 tiles
// per CU (one group), the exact pass on every size from 2 tiles per CU.
// At 33..64 rows (one pass of the 64-row instance, 8 waves per CU) the streaming kernel beats
// the matrix cores' three/four-tile kernel, which does not split k, on shapes of 1.5 to 3 tiles
// per CU (W12, 64 rows: [6144, 5120] 37.1 vs 48.7, [12288, 5120] 44.8 vs 51.0; at 40 rows the
// last ties, 44.5 vs 44.1); below 1.5 tiles per CU the matrix cores run passes of 32 rows that
// split k and win (64 rows: [5120, 17408] 70.7 vs 97.3, [1024, 5120] 24.0 vs 28.1, [5120, 6144]
// 41.0 vs 40.9); above 3 the three/four-tile kernel ([34816, 5120]: W12 69.7 vs 80.8 with up to
// two tiles per wave, [17408, 5120] 54.8 vs 55.1).  The dense baseline takes the streaming
// kernel at every size ([17408, 5120]: 40.5 vs 48.4, [34816, 5120] 65.5 vs 65.6, [152064, 5120]
// 277.6 vs 312.4, [5120, 17408] 60.3 vs 70.9).  Above 64 rows (passes of 64) the streaming
// kernel wins on 1.5 to 2.5 tiles per CU (128 rows: [6144, 5120] 73.1 vs 85.3, [8192, 5120] 74.7
// vs 85.2; [12288, 5120] ties, 87.1 vs 86.4), the dense baseline's up to 3 ([5120, 17408] 121.2
// vs 140.9, [5120, 6144] 55.6 vs 73.9, [8192, 5120] 54.7 vs 69.3, [12288, 5120] 68.6 vs 70.8).
bool stream_auto_pick(w12::Fmt f, int64_t m, int64_t tiles, int64_t k, int64_t cus) {
  const bool dense = f == w12::kFmtBF16;
  if (m <= 32)
    return k <= 8192 && (!dense || tiles <= 6 * cus) &&
           ((m >= 3 && m <= 16 && 2 * tiles >= 3 * cus) ||
            (m >= 17 && m <= 32 && tiles >= 2 * cus && (f == w12::kFmtW12 || tiles <= 24 * cus)));
  if (m <= 64) return dense || (2 * tiles >= 3 * cus && tiles <= 3 * cus);
  return dense ? tiles <= 3 * cus : 2 * tiles >= 3 * cus && 2 * tiles <= 5 * cus;
}

// Top-1 on the family the GEMM's automatic path takes for the shape: the streaming kernel's
// top-1 mode (each workgroup reduces its outputs to one key per x row) where that rule picks it
// for all m <= 32 rows at once, else the matrix-core kernel's top-1 mode in passes of 32 rows.
hipError_t launch_top1_auto(w12::Fmt f, const uint16_t* x, int64_t m, const w12::Planes& p, int64_t n,
                            int64_t k, int32_t* idx, float* val, hipStream_t s) {
  w12::DevInfo di;
  hipError_t e = w12::dev_info(&di);
  if (e != hipSuccess) return e;
  const int64_t tiles = (n + 15) / 16;
  if (w12::stream_top1_fits(di, f, m, n, k) && stream_auto_pick(f, m, tiles, k, di.cus))
    return w12::launch_stream_top1(f, x, m, p, n, k, idx, val, s);
  return w12::launch_mfma_top1(f, x, m, p, n, k, idx, val, s);
}

// fixed_scratch: run on the library's fixed scratch (allocation-free entry point) instead of the
// per-stream workspace
int run_gemm(w12::Fmt f, const uint16_t* x, int64_t m, const w12::Planes& p, int64_t n, int64_t k,
             float* y, uint32_t flags, void* stream, bool fixed_scratch = false, bool silu = false) {
  if (!x || !y) return fail(W12_ERR_ARG, "x or y is NULL");
  if (m <= 0) return fail(W12_ERR_ARG, "m must be positive (m=%lld)", (long long)m);
  if (m >= kMaxDim) return fail(W12_ERR_RANGE, "m too large");
  if (f == w12::kFmtQ8 && (flags & W12_Q8_MIDPOINT)) {
    f = w12::kFmtQ8M;
    flags &= ~W12_Q8_MIDPOINT;
  }
  const bool out16 = (flags & W12_OUT_BF16) != 0;
  flags &= ~W12_OUT_BF16;
  if (flags > W12_PATH_STREAM) return fail(W12_ERR_ARG, "unknown flags 0x%x", flags);
  if (!aligned16(x)) return fail(W12_ERR_ALIGN, "x must be 16-byte aligned");
  if (out16 ? (reinterpret_cast<uintptr_t>(y) & 1u) != 0 : !aligned4(y))
    return fail(W12_ERR_ALIGN, out16 ? "y must be 2-byte aligned" : "y must be 4-byte aligned");
  w12::YOut yo;
  if (out16) yo.h = reinterpret_cast<uint16_t*>(y);
  else yo.f = y;
  yo.silu = silu;
  // Automatic choice, from measurements on the 27B-class shapes (W12 / Q8, us, GEMV vs matrix
  // core): the GEMV wins at 1-2 rows everywhere; at 3-5 rows it wins on shapes with few tiles and
  // rows of at most 8192 (stacked qkv [8192, 5120], 5 rows: 18.2 vs 20.4) and loses on long rows
  // (down [5120, 17408], 4 rows: 43.0 vs 32.1); on gate+up [34816, 5120] the two are within 1 us
  // at 3-4 rows and the matrix cores win from 5 (58.6 vs 46.3).
  const int64_t tiles = (n + 15) / 16;
  w12::DevInfo dinfo;
  {
    hipError_t e = w12::dev_info(&dinfo);
    if (e != hipSuccess) return hip_fail(e, "device query");
  }
  const bool stream_ok = !silu && w12::stream_fits(dinfo, f, m, n, k);
  if (flags == W12_PATH_STREAM && !stream_ok)
    return fail(silu ? W12_ERR_ARG : W12_ERR_SHAPE, "the streaming kernel does not take this call "
                "(rows of fewer than 2^26 columns whose x phases fit the LDS; no SiLU epilogue)");
  const bool stream_auto = stream_ok && stream_auto_pick(f, m, tiles, k, dinfo.cus);
  const bool gemv_auto = m <= 2 || (m <= 5 && tiles <= 1024 && k <= 8192);
  const bool use_stream = flags == W12_PATH_STREAM || (flags == W12_PATH_AUTO && stream_auto);
  const bool gemv = !use_stream && (flags == W12_PATH_GEMV || (flags == W12_PATH_AUTO && gemv_auto));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  w12::Scratch sc;
  sc.s = s;
  if (fixed_scratch) {
    // the one fixed use of scratch: a GEMV pass with bfloat16 outputs whose x rows need several k
    // slices adds them in float (rows x n) before rounding; refused up front if too large (the
    // first pass has the most rows and the shortest slices)
    const int rows = (int)(m < 8 ? m : 8);
    w12::DevInfo di;
    hipError_t e = w12::dev_info(&di);
    if (e != hipSuccess) return hip_fail(e, "device query");
    const uint64_t need = (uint64_t)rows * (uint64_t)n * 4u;
    if (out16 && gemv && k > w12::gemv_k_slice(di, rows) && need > w12::kScratchBytes)
      return fail(W12_ERR_RANGE, "bfloat16 outputs of %d rows x n=%lld over several k slices need "
                  "%llu bytes of scratch, more than the fixed %llu", rows, (long long)n,
                  (unsigned long long)need, (unsigned long long)w12::kScratchBytes);
    void* ptr = nullptr;
    e = w12::fixed_scratch(&ptr);
    if (e != hipSuccess) return hip_fail(e, "fixed scratch lookup");
    sc.fixed = ptr;
    sc.bytes = w12::kScratchBytes;
  }
  hipError_t e = use_stream ? w12::launch_stream(f, x, m, p, n, k, yo, s)
                 : gemv     ? w12::launch_gemv(f, x, m, p, n, k, yo, s, sc)
                            : w12::launch_mfma(f, x, m, p, n, k, yo, s, sc);
  if (e != hipSuccess) return hip_fail(e, use_stream ? "stream launch" : gemv ? "gemv launch" : "mfma launch");
  return ok();
}

}  // namespace

namespace w12 {

hipError_t dev_info(DevInfo* out) {
  static std::mutex mu;
  static DevInfo cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].device != dev) {
    DevInfo d;
    d.device = dev;
    e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&d.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    cache[dev] = d;
  }
  *out = cache[dev];
  return hipSuccess;
}

namespace {
struct WsEntry {
  int device;
  hipStream_t stream;
  void* ptr;
};
std::mutex ws_mu;
std::vector<WsEntry> ws_table;   // the workspaces, one per (device, stream)
}  // namespace

hipError_t workspace(hipStream_t s, float** out) {
  std::mutex& mu = ws_mu;
  std::vector<WsEntry>& table = ws_table;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const WsEntry& en : table)
    if (en.device == dev && en.stream == s) {
      *out = static_cast<float*>(en.ptr);
      return hipSuccess;
    }
  // The first call on a stream may come while that stream is being captured into a graph (a
  // graph is often captured on a stream of its own): the allocation is not a stream operation,
  // so this thread's capture mode is relaxed around it.
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  e = hipThreadExchangeStreamCaptureMode(&mode);
  if (e != hipSuccess) return e;
  void* p = nullptr;
  e = hipMalloc(&p, kWorkspaceBytes);
  hipError_t e2 = hipThreadExchangeStreamCaptureMode(&mode);
  if (e != hipSuccess) return e;
  if (e2 != hipSuccess) return e2;
  table.push_back(WsEntry{dev, s, p});
  *out = static_cast<float*>(p);
  return hipSuccess;
}

}  // namespace w12

namespace {
// The 8-bit copy and the record whose escape list it shares: same shape, codes 16-byte aligned.
int check_i8(const w12_i8* cp, const w12_weight* wt) {
  if (!cp || !wt) return fail(W12_ERR_ARG, "the 8-bit copy or the record is NULL");
  int rc = check_nk(wt->n, wt->k);
  if (rc) return rc;
  if (cp->n != wt->n || cp->k != wt->k)
    return fail(W12_ERR_ARG, "the 8-bit copy is [%lld, %lld], the record [%lld, %lld]", (long long)cp->n,
                (long long)cp->k, (long long)wt->n, (long long)wt->k);
  if (!cp->q || !cp->scale || !wt->esc_ptr) return fail(W12_ERR_ARG, "q, scale or esc_ptr is NULL");
  if (wt->esc_cap > 0 && (!wt->esc_col || !wt->esc_val))
    return fail(W12_ERR_ARG, "escape arrays are NULL but esc_cap > 0");
  if (!aligned16(cp->q) || !aligned4(cp->scale)) return fail(W12_ERR_ALIGN, "q must be 16-byte and scale 4-byte aligned");
  if (!aligned4(wt->esc_ptr) || (wt->esc_col && !aligned4(wt->esc_col)) ||
      (wt->esc_val && (reinterpret_cast<uintptr_t>(wt->esc_val) & 1u)))
    return fail(W12_ERR_ALIGN, "escape arrays must be naturally aligned");
  return W12_OK;
}

w12::Planes planes_i8(const w12_i8* cp, const w12_weight* wt) {
  w12::Planes p = planes_of(wt);
  p.base = nullptr;
  p.ae = reinterpret_cast<const uint8_t*>(cp->q);
  p.lo = nullptr;
  p.scale = cp->scale;
  return p;
}
}  // namespace

extern "C" {

int w12_release_workspace(void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(w12::ws_mu);
    for (size_t i = 0; i < w12::ws_table.size(); ++i)
      if (w12::ws_table[i].device == dev && w12::ws_table[i].stream == s) {
        p = w12::ws_table[i].ptr;
        w12::ws_table.erase(w12::ws_table.begin() + (ptrdiff_t)i);
        break;
      }
  }
  if (!p) return W12_OK;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  e = hipFree(p);
  if (e != hipSuccess) return hip_fail(e, "hipFree");
  return W12_OK;
}

int w12_abi_version(void) { return W12_ABI_VERSION; }

const char* w12_last_error(void) { return g_err; }

int w12_encode(const uint16_t* w, w12_weight* out, uint64_t* n_esc, void* stream) {
  if (!w || !out || !n_esc) return fail(W12_ERR_ARG, "w, out or n_esc is NULL");
  int rc = check_record(out, true);
  if (rc) return rc;
  if (!aligned16(w)) return fail(W12_ERR_ALIGN, "w must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n = out->n, k = out->k;
  hipError_t e = w12::launch_analyze(w, n, k, out->base, out->esc_ptr, s);
  if (e != hipSuccess) return hip_fail(e, "analyze launch");
  e = w12::launch_scan(out->esc_ptr, n, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  uint32_t total = 0;
  e = hipMemcpyAsync(&total, out->esc_ptr + n, sizeof total, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "escape total copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "encode synchronisation");
  if (total == 0xFFFFFFFFu) {
    *n_esc = total;
    return fail(W12_ERR_RANGE, "escape total does not fit the 32-bit CSR");
  }
  *n_esc = total;
  if (out->esc_cap < total)
    return fail(W12_ERR_CAPACITY, "esc_cap %llu < escape total %u", (unsigned long long)out->esc_cap, total);
  e = w12::launch_pack(w, n, k, out->base, out->esc_ptr, out->ae, out->lo, out->esc_col, out->esc_val, s);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

int w12_decode(const w12_weight* wt, uint16_t* w_out, void* stream) {
  int rc = check_record(wt, true);
  if (rc) return rc;
  if (!w_out) return fail(W12_ERR_ARG, "w_out is NULL");
  if (!aligned16(w_out)) return fail(W12_ERR_ALIGN, "w_out must be 16-byte aligned");
  hipError_t e = w12::launch_decode(planes_of(wt), wt->n, wt->k, w_out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int w12_gemm(const uint16_t* x, int64_t m, const w12_weight* wt, float* y, uint32_t flags, void* stream) {
  int rc = check_record(wt, true);
  if (rc) return rc;
  return run_gemm(w12::kFmtW12, x, m, planes_of(wt), wt->n, wt->k, y, flags, stream);
}

int w12_gemm_noalloc(const uint16_t* x, int64_t m, const w12_weight* wt, float* y, uint32_t flags,
                     void* stream) {
  int rc = check_record(wt, true);
  if (rc) return rc;
  return run_gemm(w12::kFmtW12, x, m, planes_of(wt), wt->n, wt->k, y, flags, stream, true);
}

int w12_gemm_silu_mul(const uint16_t* x, int64_t m, const w12_weight* wt, float* h, uint32_t flags,
                      void* stream) {
  int rc = check_record(wt, true);
  if (rc) return rc;
  if (wt->n % 16 != 0)
    return fail(W12_ERR_SHAPE, "row-interleaved gate+up weights need n %% 16 == 0 (n=%lld)", (long long)wt->n);
  return run_gemm(w12::kFmtW12, x, m, planes_of(wt), wt->n, wt->k, h, flags, stream, false, true);
}

int w12_interleave_rows(const w12_weight* gate, const w12_weight* up, w12_weight* out, uint64_t* n_esc,
                        void* stream) {
  if (!gate || !up || !out || !n_esc) return fail(W12_ERR_ARG, "gate, up, out or n_esc is NULL");
  int rc = check_record(gate, true);
  if (!rc) rc = check_record(up, true);
  if (!rc) rc = check_record(out, true);
  if (rc) return rc;
  if (gate->n != up->n || gate->k != up->k || gate->n % 8 != 0)
    return fail(W12_ERR_SHAPE, "gate and up must have the same shape with n %% 8 == 0 (gate [%lld, %lld], up "
                "[%lld, %lld])", (long long)gate->n, (long long)gate->k, (long long)up->n, (long long)up->k);
  if (out->n != 2 * gate->n || out->k != gate->k)
    return fail(W12_ERR_ARG, "out must be [%lld, %lld]", (long long)(2 * gate->n), (long long)gate->k);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t tot[2];
  hipError_t e = hipMemcpyAsync(&tot[0], gate->esc_ptr + gate->n, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&tot[1], up->esc_ptr + up->n, 4, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "escape total copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "interleave synchronisation");
  const uint64_t total = (uint64_t)tot[0] + tot[1];
  *n_esc = total;
  if (total >= 0xFFFFFFFFull) return fail(W12_ERR_RANGE, "escape total does not fit the 32-bit CSR");
  if (out->esc_cap < total)
    return fail(W12_ERR_CAPACITY, "esc_cap %llu < escape total %llu", (unsigned long long)out->esc_cap,
                (unsigned long long)total);
  e = w12::launch_interleave(planes_of(gate), planes_of(up), out->n, out->k, out->base, out->ae, out->lo,
                             out->esc_ptr, out->esc_col, out->esc_val, s);
  if (e != hipSuccess) return hip_fail(e, "interleave launch");
  return ok();
}

int w12_q8_gemm(const uint16_t* x, int64_t m, const w12_weight* wt, float* y, uint32_t flags, void* stream) {
  int rc = check_record(wt, false);
  if (rc) return rc;
  return run_gemm(w12::kFmtQ8, x, m, planes_of(wt), wt->n, wt->k, y, flags, stream);
}

namespace {
int run_top1(w12::Fmt f, const uint16_t* x, int64_t m, const w12_weight* wt, int32_t* idx, float* val,
             uint32_t flags, void* stream) {
  if (!x || !idx || !val) return fail(W12_ERR_ARG, "x, idx or val is NULL");
  if (f == w12::kFmtQ8 && flags == W12_Q8_MIDPOINT) {
    f = w12::kFmtQ8M;
    flags = 0;
  }
  if (flags != 0) return fail(W12_ERR_ARG, "unknown flags 0x%x", flags);
  if (m <= 0) return fail(W12_ERR_ARG, "m must be positive (m=%lld)", (long long)m);
  if (m >= kMaxDim) return fail(W12_ERR_RANGE, "m too large");
  if (!aligned16(x)) return fail(W12_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned4(idx) || !aligned4(val)) return fail(W12_ERR_ALIGN, "idx and val must be 4-byte aligned");
  hipError_t e = launch_top1_auto(f, x, m, planes_of(wt), wt->n, wt->k, idx, val,
                                  reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "top-1 launch");
  return ok();
}
}  // namespace

int w12_gemm_top1(const uint16_t* x, int64_t m, const w12_weight* wt, int32_t* idx, float* val,
                  uint32_t flags, void* stream) {
  int rc = check_record(wt, true);
  if (rc) return rc;
  return run_top1(w12::kFmtW12, x, m, wt, idx, val, flags, stream);
}

int w12_q8_top1(const uint16_t* x, int64_t m, const w12_weight* wt, int32_t* idx, float* val,
                uint32_t flags, void* stream) {
  int rc = check_record(wt, false);
  if (rc) return rc;
  return run_top1(w12::kFmtQ8, x, m, wt, idx, val, flags, stream);
}

int w12_concat_rows(const w12_weight* parts, int count, w12_weight* out, uint64_t* n_esc, void* stream) {
  if (!parts || !out || !n_esc) return fail(W12_ERR_ARG, "parts, out or n_esc is NULL");
  if (count < 1 || count > 64) return fail(W12_ERR_ARG, "count must be 1..64 (count=%d)", count);
  int rc = check_record(out, true);
  if (rc) return rc;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) {
    rc = check_record(&parts[i], true);
    if (rc) return rc;
    if (parts[i].k != out->k) return fail(W12_ERR_SHAPE, "part %d has k=%lld, out has k=%lld", i,
                                          (long long)parts[i].k, (long long)out->k);
    if (i + 1 < count && parts[i].n % 16 != 0)
      return fail(W12_ERR_SHAPE, "part %d has n=%lld, not a multiple of 16 (only the last part may be)", i,
                  (long long)parts[i].n);
    rows += parts[i].n;
  }
  if (rows != out->n) return fail(W12_ERR_ARG, "out->n=%lld but the parts hold %lld rows",
                                  (long long)out->n, (long long)rows);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t tot[64];
  for (int i = 0; i < count; ++i) {
    hipError_t e = hipMemcpyAsync(&tot[i], parts[i].esc_ptr + parts[i].n, sizeof(uint32_t),
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "escape total copy");
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "concat synchronisation");
  uint64_t total = 0;
  for (int i = 0; i < count; ++i) total += tot[i];
  *n_esc = total;
  if (total >= 0xFFFFFFFFull) return fail(W12_ERR_RANGE, "escape total does not fit the 32-bit CSR");
  if (out->esc_cap < total)
    return fail(W12_ERR_CAPACITY, "esc_cap %llu < escape total %llu", (unsigned long long)out->esc_cap,
                (unsigned long long)total);
  const int64_t k = out->k;
  int64_t r0 = 0;
  uint64_t e0 = 0;
  for (int i = 0; i < count; ++i) {
    const w12_weight& p = parts[i];
    const int64_t np = w12::padded_rows(p.n);
    const struct { void* dst; const void* src; size_t bytes; } cp[] = {
        {out->base + r0, p.base, (size_t)p.n},
        {out->ae + r0 * k, p.ae, (size_t)(np * k)},
        {out->lo + r0 * k / 2, p.lo, (size_t)(np * k / 2)},
        {out->esc_col + e0, p.esc_col, (size_t)tot[i] * 4},
        {out->esc_val + e0, p.esc_val, (size_t)tot[i] * 2},
    };
    for (const auto& c : cp) {
      if (c.bytes == 0) continue;
      e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "concat copy");
    }
    e = w12::launch_rebase(p.esc_ptr, p.n + 1, (uint32_t)e0, out->esc_ptr + r0, s);
    if (e != hipSuccess) return hip_fail(e, "escape offset launch");
    r0 += p.n;
    e0 += tot[i];
  }
  return ok();
}


int w12_i8_build(const w12_weight* wt, w12_i8* out, void* stream) {
  int rc = check_record(wt, true);
  if (rc) return rc;
  if (!out) return fail(W12_ERR_ARG, "out is NULL");
  if (out->n != wt->n || out->k != wt->k)
    return fail(W12_ERR_ARG, "out is [%lld, %lld], the record [%lld, %lld]", (long long)out->n,
                (long long)out->k, (long long)wt->n, (long long)wt->k);
  if (!out->q || !out->scale) return fail(W12_ERR_ARG, "out->q or out->scale is NULL");
  if (!aligned16(out->q) || !aligned4(out->scale)) return fail(W12_ERR_ALIGN, "q must be 16-byte and scale 4-byte aligned");
  hipError_t e = w12::launch_i8_build(planes_of(wt), wt->n, wt->k, out->q, out->scale,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "8-bit copy launch");
  return ok();
}

int w12_i8_gemm(const uint16_t* x, int64_t m, const w12_i8* cp, const w12_weight* wt, float* y,
                uint32_t flags, void* stream) {
  int rc = check_i8(cp, wt);
  if (rc) return rc;
  if (flags & W12_Q8_MIDPOINT) return fail(W12_ERR_ARG, "W12_Q8_MIDPOINT does not apply to the 8-bit copy");
  return run_gemm(w12::kFmtI8, x, m, planes_i8(cp, wt), wt->n, wt->k, y, flags, stream);
}

int w12_i8_top1(const uint16_t* x, int64_t m, const w12_i8* cp, const w12_weight* wt, int32_t* idx,
                float* val, uint32_t flags, void* stream) {
  int rc = check_i8(cp, wt);
  if (rc) return rc;
  if (!x || !idx || !val) return fail(W12_ERR_ARG, "x, idx or val is NULL");
  if (flags != 0) return fail(W12_ERR_ARG, "unknown flags 0x%x", flags);
  if (m <= 0) return fail(W12_ERR_ARG, "m must be positive (m=%lld)", (long long)m);
  if (m >= kMaxDim) return fail(W12_ERR_RANGE, "m too large");
  if (!aligned16(x)) return fail(W12_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned4(idx) || !aligned4(val)) return fail(W12_ERR_ALIGN, "idx and val must be 4-byte aligned");
  hipError_t e = launch_top1_auto(w12::kFmtI8, x, m, planes_i8(cp, wt), wt->n, wt->k, idx, val,
                                  reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "top-1 launch");
  return ok();
}

int w12_bf16_gemm(const uint16_t* x, int64_t m, const uint16_t* w, int64_t n, int64_t k, float* y,
                  uint32_t flags, void* stream) {
  if (!w) return fail(W12_ERR_ARG, "w is NULL");
  int rc = check_nk(n, k);
  if (rc) return rc;
  if (!aligned16(w)) return fail(W12_ERR_ALIGN, "w must be 16-byte aligned");
  w12::Planes p;
  p.w = w;
  return run_gemm(w12::kFmtBF16, x, m, p, n, k, y, flags, stream);
}

int w12_bf16_to_tiles(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, void* stream) {
  if (!w || !out) return fail(W12_ERR_ARG, "w or out is NULL");
  int rc = check_nk(n, k);
  if (rc) return rc;
  if (!aligned16(w) || !aligned16(out)) return fail(W12_ERR_ALIGN, "w and out must be 16-byte aligned");
  hipError_t e = w12::launch_bf16_tile(w, n, k, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bf16 tiling launch");
  return ok();
}

int w12_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(W12_ERR_ARG, "buf or sink is NULL");
  if (bytes == 0 || bytes % 16) return fail(W12_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned16(buf) || !aligned4(sink)) return fail(W12_ERR_ALIGN, "buf must be 16-byte aligned");
  hipError_t e = w12::launch_read_probe(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read probe launch");
  return ok();
}

}  // extern "C"
