"""CPU oracle for the W12 lossless 12-bit weight format (test infrastructure).

This package is test infrastructure, not part of the product.  Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library and the
HIP library's Python binding never imports it.

Everything here is plain numpy (integer bit manipulation and float64 sums),
written to be checked by eye against the SpecPilot pages (arXiv 2611.02501):
the figure-captions page, Fig. 5 (W12 planes, window, escape list) and
Fig. 7 (8-bit view read by the Q pass), and the summary page's "Main
Findings" (12.01-12.02 bits per weight, escape fraction 7.3e-5).
"""
from .w12 import (  # noqa: F401
    W12Record, bf16_fields, exponent_histogram, window_coverage, choose_window,
    encode, decode, q8_view_bits, validate, ValidationError, bf16_to_f64,
    gemm64, w12_gemm64, q8_gemm64, abs_bound64, top1, record_nbytes,
    bits_per_weight, lo_row_bytes, lo_position, to_storage, from_storage,
    bf16_to_storage, padded_rows, TILE_ROWS, TILE_COLS,
    gemm64_f, abs_bound64_f, I8Copy, escaped_mask, i8_copy, i8_weights64, i8_gemm64,
    SILU_GROUP, interleave_rows, silu_rows, silu64, silu_mul64, silu_mul_bound,
)
