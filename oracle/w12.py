"""W12 oracle: plain numpy encode / decode / validate / float64 GEMMs.

Test infrastructure only (see the package docstring): the product path never
imports this module.

Sources (SpecPilot, arXiv 2611.02501):
* figure-captions page, Fig. 5(a): every BF16 weight becomes three 4-bit
  planes -- A = sign and the top three mantissa bits, E = a 4-bit exponent
  offset inside a 16-binade window chosen per output channel, B = the low
  mantissa bits; weights outside the window go to an exact escape list.
* figure-captions page, Fig. 5(a) and Fig. 7: A and E together are the 8-bit
  view, nested in each record, that the low-precision Q pass reads.
* summary page, "Main Findings": 12.01-12.02 bits per weight on average and an
  escape fraction of 7.3e-5 on Qwen3.8-27B; the format is lossless.

The pages give no bit layout, window rule, tie rule, zero handling or escape
layout.  The readings used here (numbered as in the design notes):
* R1  AE byte = s<<7 | E<<3 | m[6:4] (one byte per weight, row-major [n, k]).
      B plane: per aligned group of 8 weights k = 8g+i, the nibble m[3:0]
      lives in byte 4g + (i % 4) of the row, low nibble for i < 4, high nibble
      for i >= 4.
* R2  E = e - base, with base the window's lowest biased exponent, 1..239, so
      the window [base, base+15] stays inside the normal range 1..254.
* R3  base minimises the number of escapes; ties go to the smallest base; a
      row with no normal value gets base 1.
* R4  e = 0 (zeros, subnormals) and e = 255 (Inf, NaN) are never inside a
      window: they are always escapes.
* R5  an escaped slot holds AE = 0 and B = 0.
* R6  escapes are a row CSR: esc_ptr u32 [n+1], esc_col u32 and esc_val u16
      (raw bits), ascending k within each row.
* R8  the Q pass weight is the 8-bit view with B taken as 0 (for an
      in-window weight that is bits & 0xFFF0); escapes stay exact.
* R8m the midpoint variant of the Q pass (a next step the scope table lists):
      the dropped nibble is read as 8, the middle of its 16 possible values,
      so an in-window weight becomes bits & 0xFFF0 | 0x8; escapes stay exact.
* R11 argmax ties go to the lowest index.
* R15 storage order of the planes on the device: 16-row x 128-column tiles
      (rows padded with zero bytes to a multiple of 16, k a multiple of 128),
      tiles in row-tile-major order; inside a tile the AE byte of (row r,
      column c) sits at 1024*h + 16*(r + 16*g) + j with g = c // 32,
      h = (c % 32) // 16, j = c % 16, and the B-plane bytes of row r for
      columns [32g, 32g+32) sit at 16*(r + 16*g) .. +16.  This is only a
      permutation of the logical arrays above (see ``to_storage``).

* R16 the separate 8-bit Q-pass copy (a next step the scope table lists):
      per-row int8 with a float32 scale from the row's largest in-window
      magnitude; escapes exact through the record's list (``i8_copy``).
* R17 SiLU(gate) * up on the gate+up product, with gate and up rows
      interleaved in groups of 8 in one record (``interleave_rows``).

Parity status: every function below is pinned by the CPU tests against
values fixed independently of this file (exhaustive round trip over all 65536
bfloat16 patterns, brute-force window search, hand-worked examples of the
readings, exact rational GEMMs, arithmetic formulations of the truncated and
midpoint views, the bits-per-weight closed form).  The readings themselves
(bit order R1, tie rule R3, placeholder R5, escape layout R6, storage order
R15, the midpoint value R8m) cannot be pinned to the pages, which print no
layout or worked example: parity unpinned on those points.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WINDOW = 16                       # binades per window (Fig. 5a)
BASE_MIN = 1                      # R2: lowest normal biased exponent
BASE_MAX = 254 - WINDOW + 1       # 239: window top stays at 254
U32_MAX = 0xFFFFFFFF


class ValidationError(ValueError):
    pass


@dataclass
class W12Record:
    """A W12 tensor as numpy arrays (layout R1, R6)."""
    n: int
    k: int
    base: np.ndarray      # uint8  [n]
    ae: np.ndarray        # uint8  [n, k]          the 8-bit view (A + E)
    lo: np.ndarray        # uint8  [n, lo_row_bytes(k)]   the B plane
    esc_ptr: np.ndarray   # uint32 [n + 1]
    esc_col: np.ndarray   # uint32 [n_esc]
    esc_val: np.ndarray   # uint16 [n_esc]

    @property
    def n_esc(self) -> int:
        return int(self.esc_col.shape[0])

    def rows(self, r0: int, r1: int) -> "W12Record":
        """The sub-record of rows [r0, r1), with esc_ptr rebased to 0."""
        e0, e1 = int(self.esc_ptr[r0]), int(self.esc_ptr[r1])
        return W12Record(r1 - r0, self.k, self.base[r0:r1].copy(), self.ae[r0:r1].copy(),
                         self.lo[r0:r1].copy(),
                         (self.esc_ptr[r0:r1 + 1].astype(np.int64) - e0).astype(np.uint32),
                         self.esc_col[e0:e1].copy(), self.esc_val[e0:e1].copy())


# ----------------------------------------------------------------------------
# bfloat16 fields
# ----------------------------------------------------------------------------
def bf16_fields(bits):
    """Sign, biased exponent and 7-bit mantissa of raw bfloat16 bits (int64 arrays)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return u >> 15, (u >> 7) & 0xFF, u & 0x7F


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 value of raw bfloat16 bits (NaN payloads become some NaN)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Window choice (Fig. 5a; readings R2, R3, R4)
# ----------------------------------------------------------------------------
def exponent_histogram(w_bits) -> np.ndarray:
    """hist[n, e] = number of weights of row n with biased exponent e, for e in 1..254.

    Bins 0 and 255 (zeros/subnormals, Inf/NaN) stay 0: those values are never
    inside a window (R4).
    """
    w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
    n = w.shape[0]
    _, e, _ = bf16_fields(w)
    counted = (e >= 1) & (e <= 254)
    row = np.broadcast_to(np.arange(n, dtype=np.int64)[:, None], e.shape)
    idx = (row * 256 + e)[counted]
    return np.bincount(idx, minlength=n * 256).reshape(n, 256)


def window_coverage(hist: np.ndarray) -> np.ndarray:
    """cov[n, b] = sum of hist[n, b .. b+15] for b in 1..239 (entries b=0 and b>239 unused)."""
    hist = np.asarray(hist, dtype=np.int64)
    cov = np.zeros((hist.shape[0], 256), dtype=np.int64)
    b = np.arange(BASE_MIN, BASE_MAX + 1)
    for j in range(WINDOW):
        cov[:, b] += hist[:, b + j]
    return cov


def choose_window(w_bits):
    """(base [n] uint8, escapes per row [n] int64): fewest escapes, ties to the smallest base (R3)."""
    w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
    cov = window_coverage(exponent_histogram(w))[:, BASE_MIN:BASE_MAX + 1]
    pick = np.argmax(cov, axis=1)                 # first maximum = smallest base
    best = cov[np.arange(w.shape[0]), pick]
    return (pick + BASE_MIN).astype(np.uint8), w.shape[1] - best


# ----------------------------------------------------------------------------
# B-plane nibble placement (R1)
# ----------------------------------------------------------------------------
def lo_row_bytes(k: int) -> int:
    """Bytes of B plane per row: 4 per started group of 8 weights (= k/2 when 8 | k)."""
    return 4 * ((k + 7) // 8)


def lo_position(k_index):
    """(byte offset within the row, bit shift) of weight k's B nibble (R1)."""
    k_index = np.asarray(k_index, dtype=np.int64)
    g, i = k_index // 8, k_index % 8
    return 4 * g + (i % 4), 4 * (i // 4)


def _pack_lo(nib: np.ndarray) -> np.ndarray:
    n, k = nib.shape
    lo = np.zeros((n, lo_row_bytes(k)), dtype=np.int64)
    byte, shift = lo_position(np.arange(k))
    for kk in range(8):                       # place each of the 8 group positions in turn
        sel = np.arange(kk, k, 8)
        if sel.size:
            lo[:, byte[sel]] |= nib[:, sel] << shift[sel]
    return lo.astype(np.uint8)


def _unpack_lo(lo: np.ndarray, k: int) -> np.ndarray:
    byte, shift = lo_position(np.arange(k))
    return (lo.astype(np.int64)[:, byte] >> shift) & 0xF


# ----------------------------------------------------------------------------
# Encode / decode (Fig. 5a; R1-R6)
# ----------------------------------------------------------------------------
def encode(w_bits) -> W12Record:
    """Split every weight into the A/E/B planes, escaping those outside the row window."""
    w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
    n, k = w.shape
    s, e, m = bf16_fields(w)
    base, n_esc_row = choose_window(w)
    b = base.astype(np.int64)[:, None]
    inside = (e >= b) & (e <= b + WINDOW - 1)
    E = e - b
    ae = np.where(inside, (s << 7) | (E << 3) | (m >> 4), 0).astype(np.uint8)
    nib = np.where(inside, m & 0xF, 0)
    rows, cols = np.nonzero(~inside)              # row-major: rows ascending, k ascending
    counts = np.bincount(rows, minlength=n)
    assert np.array_equal(counts, n_esc_row)
    total = int(counts.sum())
    if total > U32_MAX:
        raise OverflowError("escape total does not fit the u32 CSR")
    esc_ptr = np.zeros(n + 1, dtype=np.uint64)
    esc_ptr[1:] = np.cumsum(counts)
    return W12Record(n, k, base, ae, _pack_lo(nib), esc_ptr.astype(np.uint32),
                     cols.astype(np.uint32), w[rows, cols].astype(np.uint16))


def _escape_rows(rec: W12Record) -> np.ndarray:
    return np.repeat(np.arange(rec.n), np.diff(rec.esc_ptr.astype(np.int64)))


def _assemble(rec: W12Record, nib: np.ndarray) -> np.ndarray:
    a = rec.ae.astype(np.int64)
    s, E, mh = a >> 7, (a >> 3) & 0xF, a & 0x7
    e = rec.base.astype(np.int64)[:, None] + E
    u = (s << 15) | (e << 7) | (mh << 4) | nib
    u[_escape_rows(rec), rec.esc_col.astype(np.int64)] = rec.esc_val
    return u.astype(np.uint16)


def decode(rec: W12Record) -> np.ndarray:
    """Exact bfloat16 bits back from the planes, then every escape overwritten (lossless)."""
    return _assemble(rec, _unpack_lo(rec.lo, rec.k))


def q8_view_bits(rec: W12Record, midpoint: bool = False) -> np.ndarray:
    """Weights the Q pass sees: the 8-bit view with B = 0 (R8), or with B = 8 (midpoint, R8m);
    escapes exact."""
    return _assemble(rec, np.full((rec.n, rec.k), 8 if midpoint else 0, dtype=np.int64))


def validate(rec: W12Record) -> None:
    """Raise ValidationError unless ``rec`` is in canonical form."""
    n, k = rec.n, rec.k

    def need(cond, msg):
        if not cond:
            raise ValidationError(msg)

    need(rec.base.shape == (n,) and rec.base.dtype == np.uint8, "base shape/dtype")
    need(rec.ae.shape == (n, k) and rec.ae.dtype == np.uint8, "ae shape/dtype")
    need(rec.lo.shape == (n, lo_row_bytes(k)) and rec.lo.dtype == np.uint8, "lo shape/dtype")
    need(rec.esc_ptr.shape == (n + 1,) and rec.esc_ptr.dtype == np.uint32, "esc_ptr shape/dtype")
    need(rec.esc_col.dtype == np.uint32 and rec.esc_val.dtype == np.uint16, "escape dtypes")
    ptr = rec.esc_ptr.astype(np.int64)
    need(ptr[0] == 0, "esc_ptr[0] != 0")
    need(bool(np.all(np.diff(ptr) >= 0)), "esc_ptr not monotone")
    need(ptr[-1] == rec.esc_col.shape[0] == rec.esc_val.shape[0], "escape array lengths")
    need(bool(np.all((rec.base >= BASE_MIN) & (rec.base <= BASE_MAX))), "base outside 1..239")
    col = rec.esc_col.astype(np.int64)
    need(bool(np.all(col < k)), "escape column out of range")
    rows = _escape_rows(rec)
    if col.size > 1:
        same_row = rows[1:] == rows[:-1]
        need(bool(np.all(col[1:][same_row] > col[:-1][same_row])), "escape columns not ascending")
    need(bool(np.all(rec.ae[rows, col] == 0)), "escaped slot has nonzero AE")
    need(bool(np.all(_unpack_lo(rec.lo, k)[rows, col] == 0)), "escaped slot has nonzero B")
    if k % 8:
        byte, shift = lo_position(np.arange(k, 8 * ((k + 7) // 8)))
        pad = (rec.lo.astype(np.int64)[:, byte] >> shift) & 0xF
        need(bool(np.all(pad == 0)), "B padding nibbles nonzero")
    _, ev, _ = bf16_fields(rec.esc_val)
    b = rec.base.astype(np.int64)[rows]
    need(bool(np.all((ev < b) | (ev > b + WINDOW - 1))), "escaped value lies inside the window")
    base2, _ = choose_window(decode(rec))
    need(bool(np.array_equal(base2, rec.base)), "base is not the window rule's choice")


# ----------------------------------------------------------------------------
# float64 GEMMs (y = x W^T, PyTorch Linear shapes) and the error bound
# ----------------------------------------------------------------------------
ROW_CHUNK = 8192


def gemm64(x_bits, w_bits) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * W[n, k] in float64 (every bf16 x bf16 product is exact)."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
    y = np.empty((x.shape[0], w.shape[0]), dtype=np.float64)
    for r0 in range(0, w.shape[0], ROW_CHUNK):
        y[:, r0:r0 + ROW_CHUNK] = x @ bf16_to_f64(w[r0:r0 + ROW_CHUNK]).T
    return y


def abs_bound64(x_bits, w_bits) -> np.ndarray:
    """sum_k |x[m, k] * W[n, k]| in float64: the scale of the error bound."""
    x = np.abs(bf16_to_f64(np.atleast_2d(x_bits)))
    w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
    y = np.empty((x.shape[0], w.shape[0]), dtype=np.float64)
    for r0 in range(0, w.shape[0], ROW_CHUNK):
        y[:, r0:r0 + ROW_CHUNK] = x @ np.abs(bf16_to_f64(w[r0:r0 + ROW_CHUNK])).T
    return y


def _by_rows(rec: W12Record, fn):
    parts = [fn(rec.rows(r0, min(rec.n, r0 + ROW_CHUNK))) for r0 in range(0, rec.n, ROW_CHUNK)]
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, rec.k), np.uint16)


def w12_gemm64(x_bits, rec: W12Record) -> np.ndarray:
    """The exact pass: x times the decoded (= original) weights, float64."""
    return gemm64(x_bits, _by_rows(rec, decode))


def q8_gemm64(x_bits, rec: W12Record, midpoint: bool = False) -> np.ndarray:
    """The Q pass: x times the 8-bit-view weights (B = 0, or 8 with ``midpoint``; escapes exact),
    float64."""
    return gemm64(x_bits, _by_rows(rec, lambda r: q8_view_bits(r, midpoint)))


def top1(y) -> np.ndarray:
    """argmax over n for each row m; ties go to the lowest n (R11)."""
    return np.argmax(np.asarray(y), axis=1)


def gemm64_f(x_bits, w64) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * W[n, k] in float64 for a float64 weight matrix."""
    return bf16_to_f64(np.atleast_2d(x_bits)) @ np.asarray(w64, dtype=np.float64).T


def abs_bound64_f(x_bits, w64) -> np.ndarray:
    """sum_k |x[m, k] * W[n, k]| in float64 for a float64 weight matrix."""
    return np.abs(bf16_to_f64(np.atleast_2d(x_bits))) @ np.abs(np.asarray(w64, dtype=np.float64)).T


# ----------------------------------------------------------------------------
# A separate 8-bit copy for the Q pass (summary page, Main Findings: the port to
# the RTX PRO 6000 reads an INT6/INT8 copy of the weights in the Q pass instead
# of the zero-copy 8-bit view).  The pages give no quantiser; reading R16:
#   * per output row n, M_n = the largest |w| among the row's in-window weights
#     (2^(base_n - 127), the window's smallest magnitude, for a row that has
#     none), and the row scale s_n = float32(M_n) / 127 in float32;
#   * an in-window weight becomes q = round-half-even(float32(w) / s_n), the
#     division in float32, clamped to [-127, 127];
#   * escaped weights (the record's exact escape list) hold q = 0 and stay exact
#     through the same escape list the exact pass uses;
#   * the weight the Q pass sees is s_n * q (in-window) or the escape value.
# ----------------------------------------------------------------------------
@dataclass
class I8Copy:
    """The 8-bit Q-pass copy of a W12 record (R16)."""
    n: int
    k: int
    q: np.ndarray         # int8    [n, k]
    scale: np.ndarray     # float32 [n]


def escaped_mask(rec: W12Record) -> np.ndarray:
    """True at every (n, k) listed in the record's escape list."""
    mask = np.zeros((rec.n, rec.k), dtype=bool)
    mask[_escape_rows(rec), rec.esc_col.astype(np.int64)] = True
    return mask


def i8_copy(rec: W12Record) -> I8Copy:
    """Quantise the record's in-window weights to int8 with one float32 scale per row (R16)."""
    w = decode(rec)
    esc = escaped_mask(rec)
    mag = np.abs(bf16_to_f64(w))
    mag[esc] = 0.0
    floor = np.ldexp(1.0, rec.base.astype(np.int64) - 127)
    big = np.maximum(mag.max(axis=1) if rec.k else floor, floor)
    scale = (big.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    wf = bf16_to_f64(w).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        ratio = (wf / scale[:, None]).astype(np.float32)
    ratio[esc] = 0.0
    q = np.clip(np.rint(ratio), -127, 127).astype(np.int8)
    return I8Copy(rec.n, rec.k, q, scale)


def i8_weights64(rec: W12Record, cp: I8Copy) -> np.ndarray:
    """The weights the Q pass sees with the 8-bit copy: s_n * q, escapes exact (float64)."""
    w = cp.scale.astype(np.float64)[:, None] * cp.q.astype(np.float64)
    w[_escape_rows(rec), rec.esc_col.astype(np.int64)] = bf16_to_f64(rec.esc_val)
    return w


def i8_gemm64(x_bits, rec: W12Record, cp: I8Copy) -> np.ndarray:
    """The Q pass on the 8-bit copy, float64."""
    return gemm64_f(x_bits, i8_weights64(rec, cp))


# ----------------------------------------------------------------------------
# SiLU(gate) * up on a gate+up product (summary page, Main Findings: W12 also
# speeds up plain autoregressive decoding, where the gate and up projections
# feed SiLU(gate) * up).  Readings R17:
#   * the gate and up weights [I, k] are stored as one record whose rows
#     interleave in groups of 8: rows 16 t .. 16 t + 7 are gate rows
#     8 t .. 8 t + 7 and rows 16 t + 8 .. 16 t + 15 are up rows 8 t .. 8 t + 7
#     (I a multiple of 8), so both halves of one output sit in one 16-row tile;
#   * h[m, i] = silu(g) * u with g = y[m, gate row of i], u = y[m, up row of i]
#     and silu(z) = z / (1 + exp(-z)).
# ----------------------------------------------------------------------------
SILU_GROUP = 8


def interleave_rows(gate_bits, up_bits) -> np.ndarray:
    """The stacked weight of R17: groups of 8 gate rows and 8 up rows, alternating."""
    g = np.atleast_2d(np.asarray(gate_bits))
    u = np.atleast_2d(np.asarray(up_bits))
    if g.shape != u.shape or g.shape[0] % SILU_GROUP:
        raise ValueError("gate and up must have the same shape, rows a multiple of 8")
    i, k = g.shape
    out = np.empty((2 * i, k), dtype=g.dtype)
    for t in range(i // SILU_GROUP):
        out[16 * t:16 * t + 8] = g[8 * t:8 * t + 8]
        out[16 * t + 8:16 * t + 16] = u[8 * t:8 * t + 8]
    return out


def silu_rows(i: int):
    """(gate rows, up rows) of the interleaved product for outputs 0 .. i-1 (R17)."""
    j = np.arange(i)
    gate = 16 * (j // SILU_GROUP) + j % SILU_GROUP
    return gate, gate + SILU_GROUP


def silu64(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in float64 (exp overflow gives the limit -0)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_mul64(y_gu) -> np.ndarray:
    """h[m, i] = silu(y[m, gate row of i]) * y[m, up row of i] from the interleaved product."""
    y = np.atleast_2d(np.asarray(y_gu, dtype=np.float64))
    gate, up = silu_rows(y.shape[1] // 2)
    return silu64(y[:, gate]) * y[:, up]


# |d silu / dz| is at most 1.0998 (its maximum, near z = 2.4); 1.1 bounds it.
SILU_SLOPE = 1.1


def silu_mul_bound(y64, absum, rel=1e-3) -> np.ndarray:
    """Error bound of a SiLU(gate) * up output whose gate and up values each carry the GEMM bound
    B = rel * sum|x w|: |silu(g') u' - silu(g) u| <= 1.1 B_g (|u| + B_u) + |silu(g)| B_u, plus
    2^-20 |h| for the float32 evaluation of silu and the product."""
    y = np.atleast_2d(np.asarray(y64, dtype=np.float64))
    b = rel * np.atleast_2d(np.asarray(absum, dtype=np.float64))
    gate, up = silu_rows(y.shape[1] // 2)
    g, u, bg, bu = y[:, gate], y[:, up], b[:, gate], b[:, up]
    h = silu64(g) * u
    return SILU_SLOPE * bg * (np.abs(u) + bu) + np.abs(silu64(g)) * bu + 2.0 ** -20 * np.abs(h)


# ----------------------------------------------------------------------------
# Size accounting (summary page, Main Findings: 12.01-12.02 bits per weight)
# ----------------------------------------------------------------------------
# ----------------------------------------------------------------------------
# Device storage order of the planes (R15)
# ----------------------------------------------------------------------------
TILE_ROWS = 16
TILE_COLS = 128


def padded_rows(n: int) -> int:
    return TILE_ROWS * ((n + TILE_ROWS - 1) // TILE_ROWS)


def to_storage(rec: W12Record):
    """(ae_s, lo_s): the AE and B planes as flat uint8 arrays in the tiled storage order."""
    n, k = rec.n, rec.k
    if k % TILE_COLS:
        raise ValueError("the tiled storage order needs k % 128 == 0")
    npad = padded_rows(n)
    ae = np.zeros((npad, k), dtype=np.uint8)
    ae[:n] = rec.ae
    lo = np.zeros((npad, k // 2), dtype=np.uint8)
    lo[:n] = rec.lo
    tr, tk = npad // TILE_ROWS, k // TILE_COLS
    # ae[tile_r, r, tile_k, g, h, j] -> ae_s[tile_r, tile_k, h, g, r, j]
    a6 = ae.reshape(tr, TILE_ROWS, tk, 4, 2, 16)
    ae_s = a6.transpose(0, 2, 4, 3, 1, 5).reshape(-1)
    # lo[tile_r, r, tile_k, g, b] -> lo_s[tile_r, tile_k, g, r, b]
    l5 = lo.reshape(tr, TILE_ROWS, tk, 4, 16)
    lo_s = l5.transpose(0, 2, 3, 1, 4).reshape(-1)
    return np.ascontiguousarray(ae_s), np.ascontiguousarray(lo_s)


def from_storage(ae_s, lo_s, n: int, k: int):
    """Inverse of ``to_storage``: row-major (ae [n, k], lo [n, k/2]); padding rows dropped."""
    npad = padded_rows(n)
    tr, tk = npad // TILE_ROWS, k // TILE_COLS
    ae = np.asarray(ae_s, dtype=np.uint8).reshape(tr, tk, 2, 4, TILE_ROWS, 16).transpose(0, 4, 1, 3, 2, 5)
    lo = np.asarray(lo_s, dtype=np.uint8).reshape(tr, tk, 4, TILE_ROWS, 16).transpose(0, 3, 1, 2, 4)
    return ae.reshape(npad, k)[:n].copy(), lo.reshape(npad, k // 2)[:n].copy()


def bf16_to_storage(w_bits) -> np.ndarray:
    """Dense bf16 W in the same tile order (the baseline's layout): inside a tile, the 8 values of
    row r at columns 32g + 8q .. +8 sit at element offset 512*q + 8*(r + 16*g)."""
    w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
    n, k = w.shape
    npad = padded_rows(n)
    wp = np.zeros((npad, k), dtype=np.uint16)
    wp[:n] = w
    tr, tk = npad // TILE_ROWS, k // TILE_COLS
    # w[tile_r, r, tile_k, g, q, e] -> s[tile_r, tile_k, q, g, r, e]
    return np.ascontiguousarray(wp.reshape(tr, TILE_ROWS, tk, 4, 4, 8).transpose(0, 2, 4, 3, 1, 5).reshape(-1))


def record_nbytes(rec: W12Record) -> int:
    return int(rec.base.nbytes + rec.ae.nbytes + rec.lo.nbytes + rec.esc_ptr.nbytes
               + rec.esc_col.nbytes + rec.esc_val.nbytes)


def bits_per_weight(rec: W12Record) -> float:
    return 8.0 * record_nbytes(rec) / (rec.n * rec.k)
