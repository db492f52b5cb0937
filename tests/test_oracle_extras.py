"""Pins of the oracle's two next-step readings: the separate 8-bit Q-pass copy (R16) and
SiLU(gate) * up on an interleaved gate+up product (R17).

R16 (summary page, Main Findings: an INT6/INT8 Q-pass copy on the RTX PRO 6000):
* the row scale equals a literal pure-Python maximum over the in-window weights (read from the
  input weights and the brute-force window, not from the record) divided by 127 in float32;
* every code is the exact nearest integer to w / s (Fractions), except where the float32
  division can move a near-tie; escapes hold 0; the row maximum maps to +-127;
* the Q-pass GEMM on the copy equals an exact rational GEMM of s * q (escapes exact).
R17 (summary page, Main Findings: W12 in plain decoding, where gate and up feed SiLU * up):
* the interleave places gate and up rows at literal positions;
* silu agrees with scipy's logistic function times z, and with its identities;
* silu_mul64 picks the gate and up outputs of each index; the bound accepts float32 results of
  perturbed gate/up values within their GEMM bounds and rejects a wrong pairing.
Planted mistakes in these functions must fail a pin.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
import oracle.w12 as ow
from lossless_bit_weight_02_amd import synth
from tests import bruteforce as bf


def _weights(seed, n, k, scale=0.02):
    rng = np.random.default_rng(seed)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * scale).astype(np.float32))
    w[rng.random((n, k)) < 0.02] = 0                         # zeros: escapes
    return w


def _with_far_escape(w):
    """Row 0 gets a value 2^40 above the rest (outside any window holding the others): an escape
    larger than every in-window weight, which the scale must ignore."""
    w = w.copy()
    w[0, 3] = 0x6F00
    return w


def _f32_exact(v) -> Fraction:
    return Fraction(float(np.float32(v)))


# ---------------------------------------------------------------- R16: the 8-bit copy
def test_i8_scale_is_literal_max_over_window():
    w = _with_far_escape(_weights(1, 6, 40))
    cp = oracle.i8_copy(oracle.encode(w))
    for n in range(w.shape[0]):
        row = [int(u) for u in w[n]]
        b, _ = bf.best_window(row)
        inside = [bf.bf16_fraction(u) for u in row if 1 <= bf.bf16_exponent(u) <= 254
                  and b <= bf.bf16_exponent(u) <= b + 15]
        big = max(abs(v) for v in inside) if inside else Fraction(2) ** (b - 127)
        want = np.float32(float(big)) / np.float32(127.0)
        assert cp.scale[n] == want, n


def test_i8_codes_are_nearest_integers():
    w = _with_far_escape(_weights(2, 8, 64))
    rec = oracle.encode(w)
    cp = oracle.i8_copy(rec)
    esc = set(zip(*np.nonzero(oracle.escaped_mask(rec))))
    near_ties = 0
    for n in range(w.shape[0]):
        s = _f32_exact(cp.scale[n])
        row_max = 0
        for kk in range(w.shape[1]):
            q = int(cp.q[n, kk])
            if (n, kk) in esc:
                assert q == 0
                continue
            r = bf.bf16_fraction(int(w[n, kk])) / s
            lo = r.numerator // r.denominator
            frac = r - lo
            if abs(frac - Fraction(1, 2)) < Fraction(127, 2 ** 23):   # float32 division may tip it
                near_ties += 1
                assert q in (lo, lo + 1)
                continue
            want = lo + 1 if frac > Fraction(1, 2) else lo
            assert q == max(-127, min(127, want)), (n, kk, float(r), q)
            row_max = max(row_max, abs(q))
        assert row_max == 127
    assert near_ties <= 2


def test_i8_gemm_equals_exact_rational():
    w = _with_far_escape(_weights(3, 5, 24))
    rec = oracle.encode(w)
    cp = oracle.i8_copy(rec)
    rng = np.random.default_rng(4)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, 24)).astype(np.float32))
    got = oracle.i8_gemm64(x, rec, cp)
    esc = oracle.escaped_mask(rec)
    for m in range(3):
        for n in range(5):
            s = _f32_exact(cp.scale[n])
            acc = Fraction(0)
            for kk in range(24):
                xv = bf.bf16_fraction(int(x[m, kk]))
                wv = bf.bf16_fraction(int(w[n, kk])) if esc[n, kk] else s * int(cp.q[n, kk])
                acc += xv * wv
            assert abs(got[m, n] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))


def test_i8_weights_within_half_step():
    w, _, _ = synth.config_weight("tiny")
    rec = oracle.encode(w)
    cp = oracle.i8_copy(rec)
    wq = oracle.i8_weights64(rec, cp)
    wv = oracle.bf16_to_f64(w)
    esc = oracle.escaped_mask(rec)
    step = cp.scale.astype(np.float64)[:, None] * np.ones_like(wv)
    assert np.array_equal(wq[esc], wv[esc])
    assert np.all(np.abs(wq - wv)[~esc] <= step[~esc] * (0.5 + 2.0 ** -16))
    assert cp.q.dtype == np.int8 and int(np.abs(cp.q.astype(np.int64)).max()) <= 127


# ---------------------------------------------------------------- R17: SiLU(gate) * up
def test_interleave_literal_positions():
    g = np.arange(16 * 3).reshape(16, 3)
    u = 1000 + np.arange(16 * 3).reshape(16, 3)
    out = oracle.interleave_rows(g, u)
    want = [g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7], u[0], u[1], u[2], u[3], u[4], u[5],
            u[6], u[7], g[8], g[9], g[10], g[11], g[12], g[13], g[14], g[15], u[8], u[9], u[10],
            u[11], u[12], u[13], u[14], u[15]]
    assert np.array_equal(out, np.array(want))
    gate, up = oracle.silu_rows(16)
    assert gate.tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 16, 17, 18, 19, 20, 21, 22, 23]
    assert up.tolist() == [8, 9, 10, 11, 12, 13, 14, 15, 24, 25, 26, 27, 28, 29, 30, 31]
    with pytest.raises(ValueError):
        oracle.interleave_rows(g[:12], u[:12])


def test_silu_against_logistic_and_identities():
    z = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-8, -1e-8, 700.0, -700.0, -800.0]])
    got = oracle.silu64(z)
    want = z * expit(z)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-300)
    assert oracle.silu64(np.array([0.0]))[0] == 0.0
    assert np.allclose(oracle.silu64(-z[:601]), oracle.silu64(z[:601]) - z[:601], rtol=1e-12, atol=1e-12)
    assert oracle.silu64(np.array([-800.0]))[0] == 0.0          # exp overflow: the limit


def test_silu_mul_picks_pairs_and_bound_behaves():
    rng = np.random.default_rng(7)
    m, i = 3, 24
    y = rng.standard_normal((m, 2 * i)) * 3
    h = oracle.silu_mul64(y)
    for j in range(i):
        gr = 16 * (j // 8) + j % 8
        g, u = y[:, gr], y[:, gr + 8]
        assert np.allclose(h[:, j], g * expit(g) * u, rtol=1e-14)
    absum = np.abs(y) * 50                        # any positive scale for the GEMM bound
    bound = oracle.silu_mul_bound(y, absum)
    # gate and up each moved by up to their GEMM bound, then evaluated in float32
    b = 1e-3 * absum
    yp = (y + b * rng.uniform(-1, 1, y.shape)).astype(np.float32)
    gate, up = oracle.silu_rows(i)
    g32, u32 = yp[:, gate], yp[:, up]
    h32 = (g32 / (np.float32(1) + np.exp(-g32)) * u32).astype(np.float64)
    assert np.all(np.abs(h32 - h) <= bound)
    # swapping gate and up is caught
    swapped = oracle.silu64(y[:, up]) * y[:, gate]
    assert np.any(np.abs(swapped - h) > bound)


# ---------------------------------------------------------------- planted mistakes
def _fails(fn, *args):
    try:
        fn(*args)
    except Exception:
        return True
    return False


def test_mutant_scale_over_all_weights(monkeypatch):
    def i8_all(rec):
        cp = ow.I8Copy.__new__(ow.I8Copy)
        w = ow.decode(rec)
        mag = np.abs(ow.bf16_to_f64(w))
        mag[~np.isfinite(mag)] = 0
        scale = (mag.max(axis=1).astype(np.float32) / np.float32(127)).astype(np.float32)
        wf = ow.bf16_to_f64(w).astype(np.float32)
        q = np.clip(np.rint(wf / scale[:, None]), -127, 127).astype(np.int8)
        q[ow.escaped_mask(rec)] = 0
        return ow.I8Copy(rec.n, rec.k, q, scale)
    monkeypatch.setattr(oracle, "i8_copy", i8_all)
    assert _fails(test_i8_scale_is_literal_max_over_window)


def test_mutant_truncating_codes(monkeypatch):
    orig = ow.i8_copy

    def trunc(rec):
        cp = orig(rec)
        w = ow.bf16_to_f64(ow.decode(rec)).astype(np.float32)
        q = np.clip(np.trunc(w / cp.scale[:, None]), -127, 127).astype(np.int8)
        q[ow.escaped_mask(rec)] = 0
        return ow.I8Copy(cp.n, cp.k, q, cp.scale)
    monkeypatch.setattr(oracle, "i8_copy", trunc)
    assert _fails(test_i8_codes_are_nearest_integers)


def test_mutant_i8_gemm_drops_escapes(monkeypatch):
    def no_esc(rec, cp):
        return cp.scale.astype(np.float64)[:, None] * cp.q.astype(np.float64)
    monkeypatch.setattr(ow, "i8_weights64", no_esc)
    assert _fails(test_i8_gemm_equals_exact_rational)


def test_mutant_interleave_groups_of_16(monkeypatch):
    def rows16(i):
        j = np.arange(i)
        gate = 32 * (j // 16) + j % 16
        return gate, gate + 16
    monkeypatch.setattr(oracle, "silu_rows", rows16)
    monkeypatch.setattr(ow, "silu_rows", rows16)
    assert _fails(test_interleave_literal_positions)
    assert _fails(test_silu_mul_picks_pairs_and_bound_behaves)


def test_mutant_silu_sign(monkeypatch):
    def bad(z):
        z = np.asarray(z, dtype=np.float64)
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(z))
    monkeypatch.setattr(oracle, "silu64", bad)
    monkeypatch.setattr(ow, "silu64", bad)
    assert _fails(test_silu_against_logistic_and_identities)
    assert _fails(test_silu_mul_picks_pairs_and_bound_behaves)
