/*
 * w12.h -- C ABI of libw12.so: the W12 lossless 12-bit weight format and the skinny GEMMs
 * that read it on AMD Instinct MI355X (gfx950).
 *
 * The format (SpecPilot, arXiv 2611.02501, figure-captions page, Fig. 5(a)): every bfloat16
 * weight of W [n, k] (PyTorch Linear layout, n = output channels) is split into three 4-bit
 * planes -- A (sign and mantissa bits 6..4), E (exponent offset inside a 16-binade window
 * chosen per output channel) and B (mantissa bits 3..0).  Weights outside their row's window
 * go to an exact escape list.  A and E together are the 8-bit view that a low-precision
 * "Q pass" reads without touching B (same page, Fig. 5(a) and Fig. 7).
 *
 * Logical content of a record (the pages fix only the plane contents; this layout is ours):
 *   base[n]      u8   lowest biased exponent of row n's window, 1..239 (window = base..base+15)
 *   AE[n][k]     u8   s<<7 | E<<3 | m[6:4],  E = e - base       (the 8-bit view)
 *   B[n][k/2]    u8   B plane.  For weights k = 8g+i (i = 0..7) the nibble m[3:0] is in byte
 *                     4g + (i % 4) of the row: low nibble for i < 4, high nibble for i >= 4
 *   esc_ptr[n+1] u32  row CSR offsets into the escape arrays, esc_ptr[0] = 0
 *   esc_col[]    u32  column k of each escape, strictly ascending within a row
 *   esc_val[]    u16  exact bfloat16 bits of each escape
 * Storage order of the AE and B planes on the device (`ae`, `lo` below): tiles of 16 rows x 128
 * columns in row-tile-major order, rows padded with zero bytes to npad = 16 * ceil(n / 16).
 * Inside a tile (2048 bytes of AE, 1024 bytes of B), the AE byte of (row r, column c) sits at
 * 1024*((c % 32) / 16) + 16*(r + 16*(c / 32)) + c % 16, and the 16 B-plane bytes of row r for
 * columns 32g..32g+31 (row bytes 16g..16g+15 of the tile's 64) sit at 16*(r + 16*g).  Every
 * wave-wide 128-bit load of a kernel then reads 1 KiB of contiguous memory, already in the lane
 * order of the 16x16x32 matrix-core operand.
 * Window rule: the window holds as many of the row's weights as possible; ties go to the
 * smallest base; a row with no normal weight gets base 1.  Zeros, subnormals, Inf and NaN
 * (exponent field 0 or 255) are never inside a window, so they are always escapes.  An
 * escaped slot holds AE = 0 and a zero nibble.  Decoding reproduces every input bit (NaN
 * payloads and -0 included).
 *
 * Conventions for every call:
 *   - Pointers named as device memory must be device memory of the current HIP device,
 *     16-byte aligned; the caller owns every buffer and keeps it alive until the stream work
 *     is finished.  The only device memory the library allocates is the GEMM workspace below;
 *     it keeps no other per-call state.
 *   - GEMM workspace: a GEMM call whose shape has too few 16-row tiles to occupy the device
 *     (for example W [1024, 5120], or [5120, 17408] at up to 32 rows of x) splits each row into
 *     k ranges whose partial sums go to a 64 MiB device buffer, then adds them in range order;
 *     a W12 or Q8 call with more than 64 rows of x puts a transposed copy of each pass's (up to
 *     128) rows there (k x 256 bytes; with k > 262144 the passes stay at 64 rows and need none).
 *     The buffer belongs to the (device, stream) pair, is allocated with hipMalloc on the first
 *     such call on that stream (also while the stream is being captured into a graph: the
 *     allocation is made under the relaxed capture mode) and is kept until the process ends
 *     or w12_release_workspace(stream).
 *     Calls on one stream are ordered by the stream; a captured graph uses the buffer of the
 *     stream it was captured on, so replaying it concurrently with other GEMM calls on that
 *     stream races.  Whether a shape splits depends only on the shape and the device, so
 *     repeated calls give bit-identical results.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work and return
 *     without synchronising, except w12_encode (see there).
 *   - Arguments are checked on the host before anything is launched; on a non-zero status
 *     nothing has been enqueued unless stated, and w12_last_error() returns a message
 *     (thread-local, valid until the next call on the same thread).  Faults inside kernels
 *     surface at the caller's next synchronisation, as usual in HIP.
 *   - k must be a multiple of 128 (W12_ERR_SHAPE otherwise) and at most 2^24, n below 2^31
 *     (W12_ERR_RANGE otherwise).
 */
#ifndef W12_H
#define W12_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W12_ABI_VERSION 1

/* status codes */
#define W12_OK            0
#define W12_ERR_ARG      (-1)  /* null pointer, n, k or m <= 0, unknown flag */
#define W12_ERR_SHAPE    (-2)  /* k % 128 != 0 */
#define W12_ERR_ALIGN    (-3)  /* a device pointer is not 16-byte aligned */
#define W12_ERR_CAPACITY (-4)  /* esc_cap smaller than the escape total (w12_encode) */
#define W12_ERR_RANGE    (-5)  /* escape total >= 2^32 - 1, k > 2^24, n or m >= 2^31 */
#define W12_ERR_HIP      (-6)  /* HIP runtime or launch error; message from hipGetErrorString */

/* flags for the GEMM calls: which kernel family runs */
#define W12_PATH_AUTO 0u  /* the family measured fastest for the shape: the streaming kernel for
                           * 3 <= m <= 16 on shapes of at least 1.5 16-row tiles per compute unit
                           * and k <= 8192, for 17 <= m <= 32 on at least 2 tiles per unit
                           * (the 8-bit passes: 2 to 24; the dense baseline: 2 to 6), for
                           * 33 <= m <= 64 on 1.5 to 3 tiles per unit (the dense baseline:
                           * every shape), and above 64 rows on 1.5 to 2.5 (the dense baseline:
                           * at most 3); otherwise the GEMV
                           * with wave reductions for m <= 2, and for m <= 5 on shapes of at most
                           * 1024 tiles and k <= 8192; bf16 MFMA otherwise */
#define W12_PATH_GEMV 1u  /* force the GEMV (m > 8 runs as several passes of <= 8 rows) */
#define W12_PATH_MFMA 2u  /* force the MFMA kernel (any m; columns padded to 16; passes of 32
                           * rows above 32 on shapes of fewer than 1.5 tiles per unit) */
#define W12_PATH_STREAM 3u /* force the streaming kernel (one workgroup per CU owning whole 16-row
                            * tiles, every wave of it an equal share of their 128-column blocks;
                            * passes of <= 64 rows of x; a wave finalises up to three tiles at
                            * 3..16 rows and two at 17..64 rows, and shapes with more tiles than
                            * that in equal row groups, all in one launch; W12_ERR_SHAPE when k is
                            * 2^26 or more or no phase length fits the LDS) */
/* w12_q8_gemm only, or-ed with a path: read the dropped B nibble as 8 (the midpoint of the 16
 * values the 8-bit view stands for) instead of 0; escapes stay exact */
#define W12_Q8_MIDPOINT 0x10u
/* flag for w12_gemm, w12_q8_gemm and w12_bf16_gemm: y is written as bfloat16 bits instead of
 * float -- each output is the float result of the same call without the flag, rounded to nearest
 * (ties to even; NaN stays NaN).  y then points to uint16_t [m][n] (2-byte aligned), passed as the
 * float* argument.  The rounding happens where the output is stored (the GEMM's epilogue, or the
 * ordered sum of a split-k launch), so no float copy of y is written; a GEMV whose x rows do not
 * fit LDS in one piece (several k slices) adds them in float in the GEMM workspace first.  The
 * error bound becomes 1e-3 * sum_k |x[m][k] * W[n][k]| plus half a bfloat16 unit in the last
 * place of the output. */
#define W12_OUT_BF16 0x20u

/* A W12 tensor: a non-owning view.  Every pointer is device memory owned by the caller. */
typedef struct w12_weight {
    int64_t   n;        /* output channels (rows of W)  */
    int64_t   k;        /* input features (columns of W) */
    uint8_t  *base;     /* [n]                           */
    uint8_t  *ae;       /* [npad * k]      tiled storage */
    uint8_t  *lo;       /* [npad * k / 2]  tiled storage */
    uint32_t *esc_ptr;  /* [n + 1]                       */
    uint32_t *esc_col;  /* [esc_cap]                     */
    uint16_t *esc_val;  /* [esc_cap]                     */
    uint64_t  esc_cap;  /* entries available in esc_col / esc_val */
} w12_weight;

/*
 * w12_encode -- bfloat16 W [n, k] (device, row-major) -> W12 record `out`.
 * Implements the plane split, window choice and escape list of Fig. 5(a) (figure-captions
 * page) under the rules above.  The result is byte-identical to a canonical CPU encoder.
 * Steps: per-row exponent histogram and window choice (writes base and per-row escape
 * counts), an in-place scan into esc_ptr, one synchronisation of `stream` to read the
 * escape total into *n_esc (host pointer), then the pack kernel writes ae, lo and the
 * escapes.  If out->esc_cap < *n_esc the call returns W12_ERR_CAPACITY after the sync:
 * base, esc_ptr and *n_esc are valid, ae/lo/escapes are not written; allocate and call
 * again.  out->n, out->k must be set by the caller.  n_esc may not be NULL.
 */
int w12_encode(const uint16_t *w, w12_weight *out, uint64_t *n_esc, void *stream);

/*
 * w12_decode -- W12 record -> bfloat16 bits W [n, k] (device, row-major).  Bit-exact inverse of
 * w12_encode (the format is lossless: figure-captions page, Fig. 5(a) "exact escape list";
 * summary page, "Key Contributions" 3).  Reads 1.5 bytes per weight plus metadata, writes 2.
 */
int w12_decode(const w12_weight *wt, uint16_t *w_out, void *stream);

/*
 * w12_gemm -- the exact pass: y[m][n] = sum_k x[m][k] * W[n][k], fp32 accumulate, fp32 y.
 * x is bfloat16 [m, k] (device, row-major), y is float [m, n] (device, row-major, fully
 * overwritten).  W is read only through its record: the planes are decoded to bfloat16 in
 * registers (figure-captions page, Fig. 5(b)) and each escape is patched exactly.
 * Error bound: |y - y_exact| <= 1e-3 * sum_k |x[m][k] * W[n][k]| per element.
 */
int w12_gemm(const uint16_t *x, int64_t m, const w12_weight *wt, float *y, uint32_t flags,
             void *stream);

/*
 * w12_gemm_noalloc -- w12_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments, flags,
 * kernels and results as w12_gemm (bit-identical for every shape whose split-k partial sums and
 * 128-row passes fit the fixed scratch below, which covers every 27B-class projection).  The
 * scratch a call needs (split-k partial sums, the transposed x of passes of more than 64 rows)
 * comes from a fixed 16 MiB array of device memory in the library (W12_NOALLOC_SCRATCH_BYTES),
 * one per GPU, held from the library's first use on that GPU until the process ends; the call
 * itself allocates nothing (no hipMalloc, no allocating library routine).  Split-k ranges and
 * 128-row passes adapt to that size; a call that cannot fit -- bfloat16 outputs on the GEMV path
 * whose x rows need several k slices, with more than 16 MiB of float partial outputs
 * (min(m, 8) x n x 4 bytes) -- returns W12_ERR_RANGE before anything is enqueued.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (on different streams, or
 * graphs replayed concurrently) race on it and must be ordered by the caller.  Nothing in the
 * array needs to start at zero; it keeps the last call's contents.
 */
#define W12_NOALLOC_SCRATCH_BYTES (16u << 20)
int w12_gemm_noalloc(const uint16_t *x, int64_t m, const w12_weight *wt, float *y, uint32_t flags,
                     void *stream);

/*
 * w12_q8_gemm -- the Q pass of two-level verification (figure-captions page, Fig. 7):
 * the same product with every in-window weight taken from the 8-bit view alone (A + E, the
 * B nibble read as 0, i.e. the bfloat16 bits & 0xFFF0) and escapes exact.  Reads base, ae
 * and the escape arrays only; wt->lo may be NULL.  Same shapes and error bound as
 * w12_gemm, against that truncated weight.  With W12_Q8_MIDPOINT in flags the in-window weight
 * is bits & 0xFFF0 | 0x8 instead (same bytes read, half the worst-case weight error).
 */
int w12_q8_gemm(const uint16_t *x, int64_t m, const w12_weight *wt, float *y, uint32_t flags,
                void *stream);

/*
 * w12_q8_top1 / w12_gemm_top1 -- the top-1 output of each row of x, for the Q pass (8-bit view,
 * as w12_q8_gemm) or the exact pass (as w12_gemm), without writing the [m, n] outputs: the
 * two-level verification compares only the argmax chain of the cheap pass with the exact one
 * (figure-captions page, Fig. 7; summary page, Main Findings: 98.7% top-1 agreement).
 * idx[j] (int32, device) = the n at which y[j][n] is largest, ties to the smallest n; val[j]
 * (float, device) = that y[j][n] (a NaN output counts as the largest).  Where the automatic path
 * of w12_q8_gemm / w12_gemm takes the streaming kernel for all m <= 32 rows, y is exactly that
 * path's output; otherwise y is computed exactly as the matrix-core path computes it for a shape
 * too large to split, in passes of up to 32 rows of x (each pass reads the weights once).  Either
 * kernel reduces its outputs to per-workgroup keys in the workspace instead of writing them, and
 * one small kernel per pass picks the winners.  Uses the GEMM workspace (see the conventions
 * above).
 * Same record checks as w12_q8_gemm / w12_gemm; idx and val 4-byte aligned.  flags: 0, or for
 * w12_q8_top1 W12_Q8_MIDPOINT (the midpoint view, as in w12_q8_gemm); anything else is
 * W12_ERR_ARG.
 */
int w12_q8_top1(const uint16_t *x, int64_t m, const w12_weight *wt, int32_t *idx, float *val,
                uint32_t flags, void *stream);
int w12_gemm_top1(const uint16_t *x, int64_t m, const w12_weight *wt, int32_t *idx, float *val,
                  uint32_t flags, void *stream);

/*
 * w12_interleave_rows -- the record of the gate and up projections of an MLP stacked with their
 * rows interleaved in groups of 8: output rows 16 t .. 16 t + 7 are gate rows 8 t .. 8 t + 7 and
 * rows 16 t + 8 .. 16 t + 15 are up rows 8 t .. 8 t + 7, so the two inputs of one
 * SiLU(gate) * up output sit in one 16-row tile (summary page, Main Findings: W12 also speeds up
 * plain decoding, where gate and up feed SiLU(gate) * up).  Built on the device from the two
 * records without decoding (windows and escape lists are per row); byte-identical to w12_encode
 * of the interleaved matrix.  gate and up: same [I, k], I % 8 == 0.  out: a record of
 * [2 I, k] sized for it.  Synchronises `stream` once to read the parts' escape totals into
 * *n_esc (host); if out->esc_cap is smaller, returns W12_ERR_CAPACITY before writing anything.
 */
int w12_interleave_rows(const w12_weight *gate, const w12_weight *up, w12_weight *out, uint64_t *n_esc,
                        void *stream);

/*
 * w12_gemm_silu_mul -- the exact pass on row-interleaved gate+up weights (w12_interleave_rows)
 * with the MLP activation applied where the outputs are stored: h[j][i] = silu(g) * u, where
 * g = y[j][16 (i / 8) + i % 8] and u = y[j][16 (i / 8) + i % 8 + 8] are the gate and up outputs of
 * w12_gemm on the same record and silu(z) = z / (1 + exp(-z)) in float.  x bfloat16 [m, k]; h is
 * float [m, n / 2] (or bfloat16 bits with W12_OUT_BF16: each h rounded to nearest even), fully
 * overwritten; wt->n % 16 == 0 (W12_ERR_SHAPE otherwise).  flags: W12_PATH_*, W12_OUT_BF16.
 * The y values are never written to memory except as split-k partial sums in the GEMM workspace.
 * Error bound per output, with B = 1e-3 * sum_k |x[j][k] W[row][k]| of each input row:
 * 1.1 B_g (|u| + B_u) + |silu(g)| B_u + 2^-20 |h| (1.1 bounds the slope of silu), plus half a
 * bfloat16 unit in the last place with W12_OUT_BF16.
 */
int w12_gemm_silu_mul(const uint16_t *x, int64_t m, const w12_weight *wt, float *h, uint32_t flags,
                      void *stream);

/*
 * The separate 8-bit copy for the Q pass (summary page, Main Findings: the RTX PRO 6000 port reads
 * an INT6/INT8 copy of the weights in the Q pass instead of the zero-copy 8-bit view).  It sits
 * beside a W12 record and shares that record's exact escape list.  The pages give no quantiser;
 * this one is linear per output row: M_n = the largest magnitude among the row's in-window
 * weights (2^(base - 127), the window's smallest magnitude, for a row with none), scale
 * s_n = M_n / 127 in float32, and every in-window weight becomes q = round-half-even(w / s_n)
 * (float32 division), clamped to +-127; escaped slots hold q = 0.  The Q pass then sees s_n * q
 * for in-window weights and the exact value for escapes.  1 byte per weight plus 4 per row, the
 * same bytes per pass as the 8-bit view, and 1 extra byte per weight of memory.
 */
typedef struct w12_i8 {
    int64_t  n;        /* rows of W (must equal the record's)    */
    int64_t  k;        /* columns of W (must equal the record's) */
    int8_t  *q;        /* [npad * k] codes, in the storage order of the record's AE plane (device, 16-byte aligned) */
    float   *scale;    /* [n] per-row scale (device, 4-byte aligned) */
} w12_i8;

/*
 * w12_i8_build -- the 8-bit copy of record `wt` into the caller's out->q and out->scale (out->n,
 * out->k set by the caller to the record's).  Reads the whole record (planes and escape list);
 * padding rows of the storage get code 0.  Enqueued on `stream`, no synchronisation.
 */
int w12_i8_build(const w12_weight *wt, w12_i8 *out, void *stream);

/*
 * w12_i8_gemm -- the Q pass on the 8-bit copy: y[m][n] = s_n * sum_k x[m][k] q[n][k] + the exact
 * escapes' products, fp32 accumulate.  Reads cp->q, cp->scale and wt's escape arrays (wt->base,
 * wt->ae and wt->lo are not read and may be NULL).  Same x, y, flags (W12_PATH_*, W12_OUT_BF16),
 * kernel families and error bound as w12_q8_gemm, against the weights s_n * q; more than 64 rows
 * of x run as passes of at most 64.  W12_Q8_MIDPOINT is W12_ERR_ARG.
 */
int w12_i8_gemm(const uint16_t *x, int64_t m, const w12_i8 *cp, const w12_weight *wt, float *y,
                uint32_t flags, void *stream);

/*
 * w12_i8_top1 -- top-1 of the Q pass on the 8-bit copy per row of x, as w12_q8_top1 (idx int32,
 * val float; ties to the smallest n); flags must be 0.
 */
int w12_i8_top1(const uint16_t *x, int64_t m, const w12_i8 *cp, const w12_weight *wt, int32_t *idx,
                float *val, uint32_t flags, void *stream);

/*
 * w12_concat_rows -- the record of W = [W_0; W_1; ...; W_{count-1}] (the parts' rows stacked in
 * order) built on the device from the parts' records, without decoding or re-encoding.  Windows
 * and escape lists are per output row (figure-captions page, Fig. 5(a)), so the stacked record is
 * the parts' window bottoms, planes and escapes side by side, with the escape offsets rebased; it
 * is byte-identical to w12_encode of the stacked matrix.  Used to run projections that read the
 * same activations (q, k and v; gate and up) as one GEMM.
 * parts: host array of `count` (1..64) records; every part has the same k, and every part but
 * the last has n % 16 == 0 (whole 16-row tiles of the storage order).  out: a record whose n is
 * the sum of the parts' n and whose arrays are sized for it (ae npad*k, lo npad*k/2, base n,
 * esc_ptr n+1, esc_col/esc_val esc_cap entries).  Synchronises `stream` once to read the parts'
 * escape totals into *n_esc (host); if out->esc_cap is smaller, returns W12_ERR_CAPACITY before
 * writing anything.  The parts must not overlap `out`.
 */
int w12_concat_rows(const w12_weight *parts, int count, w12_weight *out, uint64_t *n_esc,
                    void *stream);

/*
 * w12_bf16_gemm -- same-build dense baseline: y = x * W^T with W bfloat16 in the same tiled
 * storage order as the W12 planes (npad * k values, from w12_bf16_to_tiles), same kernel
 * structure and flags as w12_gemm, 2 bytes per weight.
 */
int w12_bf16_gemm(const uint16_t *x, int64_t m, const uint16_t *w_tiles, int64_t n, int64_t k,
                  float *y, uint32_t flags, void *stream);

/*
 * w12_bf16_to_tiles -- dense bfloat16 W [n, k] (device, row-major) -> the tiled storage order of
 * the baseline (out: npad * k values; padding rows zero).  Inside a tile (16 rows x 128 columns,
 * 4096 bytes) the 8 values of row r at columns 32g + 8q .. +7 sit at byte 1024*q + 16*(r + 16g).
 */
int w12_bf16_to_tiles(const uint16_t *w, int64_t n, int64_t k, uint16_t *out, void *stream);

/*
 * w12_read_probe -- bandwidth probe: streams `bytes` bytes of `buf` (device, 16-byte
 * aligned, bytes % 16 == 0) with 128-bit loads and writes one word per workgroup of a
 * checksum to `sink` (device, at least 4096 u32).  Measures the achievable HBM read rate.
 */
int w12_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, void *stream);

/*
 * w12_release_workspace -- frees the GEMM workspace of (current device, `stream`), if the
 * library allocated one (see the conventions above), for callers that create and destroy
 * streams (per request or per thread): without it a destroyed stream's 64 MiB stay allocated
 * until the process ends.  Waits for the stream's work first (hipStreamSynchronize), then frees
 * the buffer; a later GEMM call on the stream allocates a new one.  Graphs captured on the
 * stream still point at the freed buffer: do not replay them after this call.  Returns W12_OK
 * whether or not there was a buffer; not for use while `stream` is being captured.
 */
int w12_release_workspace(void *stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char *w12_last_error(void);

/* W12_ABI_VERSION of the loaded library. */
int w12_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W12_H */
