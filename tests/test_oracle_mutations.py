"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each one.

Each mutant replaces one oracle function for the duration of a test; the pins from the other
test modules are then run against it and at least one must fail.
"""
import numpy as np
import pytest

import oracle
import oracle.w12 as ow
from tests import test_oracle_format as tf
from tests import test_oracle_gemm as tg


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(ow, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _fails(fn, *args):
    try:
        fn(*args)
    except Exception:  # AssertionError, shape errors, ValidationError ...
        return True
    return False


def test_mutant_tie_to_largest_base(monkeypatch, golden_dir):
    orig_cov, orig_hist = ow.window_coverage, ow.exponent_histogram

    def choose_last(w_bits):
        w = np.atleast_2d(np.asarray(w_bits, dtype=np.uint16))
        cov = orig_cov(orig_hist(w))[:, ow.BASE_MIN:ow.BASE_MAX + 1]
        pick = cov.shape[1] - 1 - np.argmax(cov[:, ::-1], axis=1)
        return (pick + ow.BASE_MIN).astype(np.uint8), w.shape[1] - cov.max(axis=1)

    _patch(monkeypatch, "choose_window", choose_last)
    assert _fails(tf.test_worked_examples, golden_dir)
    assert _fails(tf.test_window_matches_literal_bruteforce)


def test_mutant_swapped_nibble_order(monkeypatch, golden_dir):
    def swapped(k_index):
        k_index = np.asarray(k_index, dtype=np.int64)
        g, i = k_index // 8, k_index % 8
        return 4 * g + (i // 2), 4 * (i % 2)          # even k low nibble, odd k high nibble

    _patch(monkeypatch, "lo_position", swapped)
    # encode and decode stay mutually consistent, so the round trip alone cannot see this ...
    tf.test_exhaustive_roundtrip("shuffled_256x256")
    # ... but the hand-worked layout does
    assert _fails(tf.test_worked_examples, golden_dir)


def test_mutant_dropped_sign(monkeypatch):
    orig = ow.bf16_fields

    def no_sign(bits):
        s, e, m = orig(bits)
        return s * 0, e, m

    _patch(monkeypatch, "bf16_fields", no_sign)
    assert _fails(tf.test_exhaustive_roundtrip, "natural_256x256")


def test_mutant_window_off_by_one(monkeypatch, golden_dir):
    monkeypatch.setattr(ow, "WINDOW", 15)
    assert _fails(tf.test_window_matches_direct_count_tiny)


def test_mutant_transposed_gemm(monkeypatch):
    def transposed(x_bits, w_bits):
        return ow.bf16_to_f64(np.atleast_2d(x_bits)) @ ow.bf16_to_f64(np.atleast_2d(w_bits))

    _patch(monkeypatch, "gemm64", transposed)
    assert _fails(tg.test_gemm64_equals_exact_rational, 2, 6, 6)
    assert _fails(tg.test_gemm64_equals_exact_rational, 1, 5, 7)


def test_mutant_dropped_last_term(monkeypatch):
    orig = ow.gemm64

    def short(x_bits, w_bits):
        x = np.array(np.atleast_2d(x_bits), copy=True)
        x[:, -1] = 0
        return orig(x, w_bits)

    _patch(monkeypatch, "gemm64", short)
    assert _fails(tg.test_gemm64_equals_exact_rational, 3, 4, 9)


def test_mutant_q8_midpoint(monkeypatch):
    orig = ow._assemble

    def midpoint(rec, nib):
        return orig(rec, nib + 8)

    monkeypatch.setattr(ow, "q8_view_bits",
                        lambda rec, mid=False: midpoint(rec, np.zeros((rec.n, rec.k), np.int64)))
    monkeypatch.setattr(oracle, "q8_view_bits", ow.q8_view_bits)
    assert _fails(tg.test_q8_view_is_arithmetic_truncation)


def test_mutant_placeholder_not_cleared(monkeypatch):
    """An encoder that leaves the escaped value's own bits in the planes is caught by validate()."""
    orig_encode = ow.encode

    def leaky(w_bits):
        rec = orig_encode(w_bits)
        rows = np.repeat(np.arange(rec.n), np.diff(rec.esc_ptr.astype(np.int64)))
        rec.ae[rows, rec.esc_col.astype(np.int64)] = (rec.esc_val >> 8).astype(np.uint8) | 1
        return rec

    _patch(monkeypatch, "encode", leaky)
    assert _fails(tf.test_config_roundtrip_tiny)


def test_mutant_q8_midpoint_wrong_direction(monkeypatch):
    """A midpoint view that moves toward zero (B = 8 subtracted instead of added) is caught."""
    orig = ow._assemble

    def view(rec, mid=False):
        if not mid:
            return orig(rec, np.zeros((rec.n, rec.k), np.int64))
        u = orig(rec, np.zeros((rec.n, rec.k), np.int64)).astype(np.int64)
        return np.where((u & 0x7F) >= 8, u - 8, u).astype(np.uint16)

    monkeypatch.setattr(ow, "q8_view_bits", view)
    monkeypatch.setattr(oracle, "q8_view_bits", ow.q8_view_bits)
    assert _fails(tg.test_q8_midpoint_view_is_truncation_plus_half_a_step)
