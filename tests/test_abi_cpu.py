"""Host-only checks of the C ABI: libw12.so loads, exports every symbol include/w12.h declares,
and rejects bad arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from lossless_bit_weight_02_amd import w12

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w12.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w12_[a-z0-9_]+)\s*\(", text)))


def _lib():
    if not os.path.exists(w12.LIB_PATH):
        pytest.skip("libw12.so not built")
    return w12.lib()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for want in ("w12_encode", "w12_decode", "w12_gemm", "w12_q8_gemm"):
        assert want in names


def test_every_declared_symbol_is_exported():
    L = _lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert name in w12.EXPORTS, f"binding does not marshal {name}"


def test_abi_version_and_status_codes_match_header():
    L = _lib()
    text = open(HEADER).read()
    assert L.w12_abi_version() == int(re.search(r"#define W12_ABI_VERSION (\d+)", text).group(1))
    for name in ("OK", "ERR_ARG", "ERR_SHAPE", "ERR_ALIGN", "ERR_CAPACITY", "ERR_RANGE", "ERR_HIP"):
        m = re.search(rf"#define W12_{name}\s+\(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == getattr(w12, f"W12_{name}"), name


def _rec(n=64, k=128, **over):
    s = w12._W12Weight(n, k, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 10)
    for key, v in over.items():
        setattr(s, key, v)
    return s


def test_argument_errors_are_host_side():
    L = _lib()
    n_esc = ctypes.c_uint64(0)
    assert L.w12_encode(None, None, None, None) == w12.W12_ERR_ARG
    assert b"NULL" in L.w12_last_error()
    # k not a multiple of 128
    assert L.w12_encode(0x1000, ctypes.byref(_rec(k=96)), ctypes.byref(n_esc), None) == w12.W12_ERR_SHAPE
    # non-positive sizes
    assert L.w12_decode(ctypes.byref(_rec(n=0)), 0x1000, None) == w12.W12_ERR_ARG
    assert L.w12_gemm(0x1000, 0, ctypes.byref(_rec()), 0x1000, 0, None) == w12.W12_ERR_ARG
    # misaligned planes / x
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec(ae=0x2001)), 0x1000, 0, None) == w12.W12_ERR_ALIGN
    assert L.w12_gemm(0x1008, 1, ctypes.byref(_rec()), 0x1000, 0, None) == w12.W12_ERR_ALIGN
    # unknown flags
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1000, 7, None) == w12.W12_ERR_ARG
    # q8 does not need the B plane, the exact pass does
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec(lo=None)), 0x1000, 0, None) == w12.W12_ERR_ARG
    # escape arrays missing while esc_cap > 0
    assert L.w12_decode(ctypes.byref(_rec(esc_col=None)), 0x1000, None) == w12.W12_ERR_ARG
    # dense baseline
    assert L.w12_bf16_gemm(0x1000, 1, None, 8, 128, 0x1000, 0, None) == w12.W12_ERR_ARG
    assert L.w12_bf16_gemm(0x1000, 1, 0x1000, 8, 64, 0x1000, 0, None) == w12.W12_ERR_SHAPE
    assert L.w12_bf16_to_tiles(None, 8, 128, 0x1000, None) == w12.W12_ERR_ARG
    assert L.w12_bf16_to_tiles(0x1000, 8, 200, 0x1000, None) == w12.W12_ERR_SHAPE
    assert L.w12_read_probe(0x1000, 20, 0x1000, None) == w12.W12_ERR_SHAPE
    # huge sizes: n >= 2^31, k > 2^24 (kernels use 32-bit buffer offsets)
    assert L.w12_decode(ctypes.byref(_rec(n=1 << 40)), 0x1000, None) == w12.W12_ERR_RANGE
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec(k=(1 << 24) + 128)), 0x1000, 0, None) == w12.W12_ERR_RANGE
    assert L.w12_bf16_gemm(0x1000, 1, 0x1000, 8, (1 << 24) + 128, 0x1000, 0, None) == w12.W12_ERR_RANGE


def test_concat_rows_argument_errors_are_host_side():
    """w12_concat_rows rejects bad part lists before any device access (fake device pointers)."""
    L = _lib()
    n_esc = ctypes.c_uint64(0)

    def parts(*ns, k=128):
        return (w12._W12Weight * len(ns))(*[_rec(n=n, k=k) for n in ns])

    assert L.w12_concat_rows(None, 1, ctypes.byref(_rec()), ctypes.byref(n_esc), None) == w12.W12_ERR_ARG
    assert L.w12_concat_rows(parts(16), 0, ctypes.byref(_rec(n=16)), ctypes.byref(n_esc), None) == w12.W12_ERR_ARG
    assert L.w12_concat_rows(parts(16), 65, ctypes.byref(_rec(n=16)), ctypes.byref(n_esc), None) == w12.W12_ERR_ARG
    # a part other than the last is not whole 16-row tiles
    assert L.w12_concat_rows(parts(20, 16), 2, ctypes.byref(_rec(n=36)), ctypes.byref(n_esc),
                             None) == w12.W12_ERR_SHAPE
    assert b"multiple of 16" in L.w12_last_error()
    # parts disagree on k
    mixed = (w12._W12Weight * 2)(_rec(n=16, k=128), _rec(n=16, k=256))
    assert L.w12_concat_rows(mixed, 2, ctypes.byref(_rec(n=32)), ctypes.byref(n_esc), None) == w12.W12_ERR_SHAPE
    # out->n is not the parts' total
    assert L.w12_concat_rows(parts(16, 5), 2, ctypes.byref(_rec(n=20)), ctypes.byref(n_esc), None) == w12.W12_ERR_ARG
    # misaligned part plane
    bad = (w12._W12Weight * 2)(_rec(n=16), _rec(n=16, ae=0x2004))
    assert L.w12_concat_rows(bad, 2, ctypes.byref(_rec(n=32)), ctypes.byref(n_esc), None) == w12.W12_ERR_ALIGN


def test_top1_argument_errors_are_host_side():
    L = _lib()
    assert L.w12_q8_top1(0x1000, 1, ctypes.byref(_rec()), None, 0x1000, 0, None) == w12.W12_ERR_ARG
    assert L.w12_gemm_top1(0x1000, 0, ctypes.byref(_rec()), 0x1000, 0x1000, 0, None) == w12.W12_ERR_ARG
    assert L.w12_gemm_top1(0x1000, 1, ctypes.byref(_rec()), 0x1002, 0x1000, 0, None) == w12.W12_ERR_ALIGN
    assert L.w12_q8_top1(0x1000, 1, ctypes.byref(_rec(k=100)), 0x1000, 0x1000, 0, None) == w12.W12_ERR_SHAPE
    # the Q pass does not need the B plane, the exact pass does
    assert L.w12_gemm_top1(0x1000, 1, ctypes.byref(_rec(lo=None)), 0x1000, 0x1000, 0, None) == w12.W12_ERR_ARG
    # flags: only the Q pass has a midpoint variant; path flags do not apply
    assert L.w12_gemm_top1(0x1000, 1, ctypes.byref(_rec()), 0x1000, 0x1000, w12.Q8_MIDPOINT, None) == w12.W12_ERR_ARG
    assert L.w12_q8_top1(0x1000, 1, ctypes.byref(_rec()), 0x1000, 0x1000, 1, None) == w12.W12_ERR_ARG


def test_midpoint_flag_only_on_the_q_pass():
    L = _lib()
    # the exact pass has no midpoint variant: the flag is an unknown flag there (host-side)
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1000, w12.Q8_MIDPOINT, None) == w12.W12_ERR_ARG
    assert L.w12_bf16_gemm(0x1000, 1, 0x1000, 8, 128, 0x1000, w12.Q8_MIDPOINT, None) == w12.W12_ERR_ARG
    # on the Q pass it combines with a path; other bits stay unknown
    assert L.w12_q8_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1000, w12.Q8_MIDPOINT | 0x4, None) == w12.W12_ERR_ARG
    text = open(HEADER).read()
    assert int(re.search(r"#define W12_Q8_MIDPOINT (0x[0-9a-fA-F]+)u", text).group(1), 16) == w12.Q8_MIDPOINT


def test_bf16_output_flag_host_checks():
    """W12_OUT_BF16: the header's value is the binding's; with it y needs only 2-byte alignment,
    an odd address is refused before anything runs, and it does not combine with top-1 calls."""
    L = _lib()
    text = open(HEADER).read()
    assert int(re.search(r"#define W12_OUT_BF16 (0x[0-9a-fA-F]+)u", text).group(1), 16) == w12.OUT_BF16
    for fl in (w12.OUT_BF16, w12.OUT_BF16 | 1, w12.OUT_BF16 | 2):
        assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1001, fl, None) == w12.W12_ERR_ALIGN
        assert L.w12_q8_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1001, fl | w12.Q8_MIDPOINT, None) == w12.W12_ERR_ALIGN
        assert L.w12_bf16_gemm(0x1000, 1, 0x1000, 8, 128, 0x1001, fl, None) == w12.W12_ERR_ALIGN
    # without the flag y stays a float array (4-byte alignment)
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1002, 0, None) == w12.W12_ERR_ALIGN
    # the exact pass still has no midpoint variant; top-1 calls write no y
    assert L.w12_gemm(0x1000, 1, ctypes.byref(_rec()), 0x1000, w12.OUT_BF16 | w12.Q8_MIDPOINT, None) == w12.W12_ERR_ARG
    assert L.w12_q8_top1(0x1000, 1, ctypes.byref(_rec()), 0x1000, 0x1000, w12.OUT_BF16, None) == w12.W12_ERR_ARG
