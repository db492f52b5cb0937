"""Row-chunked runs of the CPU oracle in worker processes (test infrastructure).

W12 windows and escape lists are per output row, so the oracle's record of W is the row-wise
concatenation of the records of its row chunks (escape offsets shifted by the escapes before
each chunk).  The workers are spawned fresh (no GPU state), import only numpy and the oracle,
and each returns plain arrays.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import dataclasses

import numpy as np

import oracle

ROWS_PER_TASK = 4096


def _encode_chunk(w_chunk):
    r = oracle.encode(w_chunk)
    return r.base, r.ae, r.lo, r.esc_ptr, r.esc_col, r.esc_val


def _gemm_chunk(args):
    x_bits, w_chunk, view = args
    if view in ("q8", "q8m"):
        w_chunk = oracle.q8_view_bits(oracle.encode(w_chunk), midpoint=view == "q8m")
    return oracle.gemm64(x_bits, w_chunk), oracle.abs_bound64(x_bits, w_chunk)


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def make_pool() -> ProcessPoolExecutor:
    return ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"),
                               initializer=_one_blas_thread)


def _chunks(n: int):
    return [(r, min(n, r + ROWS_PER_TASK)) for r in range(0, n, ROWS_PER_TASK)]


def encode(w_bits: np.ndarray, pool: ProcessPoolExecutor) -> oracle.W12Record:
    """oracle.encode(w_bits), computed over row chunks."""
    n, k = w_bits.shape
    parts = list(pool.map(_encode_chunk, [w_bits[a:b] for a, b in _chunks(n)]))
    base = np.concatenate([p[0] for p in parts])
    ae = np.concatenate([p[1] for p in parts])
    lo = np.concatenate([p[2] for p in parts])
    ptr = [np.zeros(1, np.uint32)]
    off = 0
    for p in parts:
        ptr.append((p[3][1:].astype(np.uint64) + off).astype(np.uint32))
        off += int(p[3][-1])
    esc_ptr = np.concatenate(ptr)
    esc_col = np.concatenate([p[4] for p in parts])
    esc_val = np.concatenate([p[5] for p in parts])
    return oracle.W12Record(n, k, base, ae, lo, esc_ptr, esc_col, esc_val)


def gemm(x_bits: np.ndarray, w_bits: np.ndarray, pool: ProcessPoolExecutor, view: str = "exact"):
    """(y64, sum |x w|) for y = x W^T over all rows of W; view "q8" uses the oracle's 8-bit view,
    "q8m" its midpoint view."""
    n = w_bits.shape[0]
    parts = list(pool.map(_gemm_chunk, [(x_bits, w_bits[a:b], view) for a, b in _chunks(n)]))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def _i8_chunk(args):
    """(scale, codes in the storage order, y64, sum |x w|) of the 8-bit Q-pass copy of one row
    chunk (a whole number of 16-row tiles, so the chunks' storage orders concatenate)."""
    x_bits, w_chunk = args
    ref = oracle.encode(w_chunk)
    cp = oracle.i8_copy(ref)
    q_s = oracle.to_storage(dataclasses.replace(ref, ae=cp.q.view(np.uint8)))[0].view(np.int8)
    wq = oracle.i8_weights64(ref, cp)
    return cp.scale, q_s, oracle.gemm64_f(x_bits, wq), oracle.abs_bound64_f(x_bits, wq)


def i8_chunks(x_bits: np.ndarray, w_bits: np.ndarray, pool: ProcessPoolExecutor):
    """_i8_chunk over the row chunks of W, in order."""
    return list(pool.map(_i8_chunk, [(x_bits, w_bits[a:b]) for a, b in _chunks(w_bits.shape[0])]))
