"""Helpers for the GPU parity tests: device transfer and the element-wise bound check."""
import sys

import numpy as np

import oracle


def say(msg: str):
    """Print what is about to run on the GPU (flushed, so a crash still names the case)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, device="cuda:0"):
    import torch
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def to_host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def record_numpy(rec) -> dict:
    """The GPU record's arrays as stored (planes in the tiled storage order)."""
    return rec.to_numpy()


def oracle_storage(rec: oracle.W12Record) -> dict:
    """The oracle's record in the same storage form."""
    ae_s, lo_s = oracle.to_storage(rec)
    return dict(n=rec.n, k=rec.k, base=rec.base, ae_s=ae_s, lo_s=lo_s, esc_ptr=rec.esc_ptr,
                esc_col=rec.esc_col, esc_val=rec.esc_val)


def logical_record(d: dict) -> oracle.W12Record:
    """A stored record back in the oracle's row-major form."""
    ae, lo = oracle.from_storage(d["ae_s"], d["lo_s"], d["n"], d["k"])
    return oracle.W12Record(d["n"], d["k"], d["base"], ae, lo, d["esc_ptr"], d["esc_col"],
                            d["esc_val"])


def assert_records_equal(got: dict, want, what=""):
    if isinstance(want, oracle.W12Record):
        want = oracle_storage(want)
    assert got["n"] == want["n"] and got["k"] == want["k"]
    for name in ("base", "ae_s", "lo_s", "esc_ptr", "esc_col", "esc_val"):
        a, b = got[name], want[name]
        assert a.shape == b.shape, f"{what}: {name} shape {a.shape} != {b.shape}"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{what}: {name} differs at {bad[:5].tolist()} "
                                 f"({len(bad)} positions)")


def check_gemm(y_gpu: np.ndarray, x_bits, w_bits, what="", rel=1e-3):
    """|y - y64| <= rel * sum|x w| for finite oracle values; non-finite oracle values must be
    matched in kind (NaN with NaN, +-Inf with the same Inf).  Returns the worst error / bound."""
    return check_y(y_gpu, oracle.gemm64(x_bits, w_bits), oracle.abs_bound64(x_bits, w_bits), what, rel)


def check_y(y_gpu: np.ndarray, y64: np.ndarray, absum: np.ndarray, what="", rel=1e-3):
    """check_gemm against a precomputed oracle product y64 and sum |x w| (same shapes)."""
    y = np.asarray(y_gpu, dtype=np.float64)
    bound = rel * absum
    fin = np.isfinite(y64)
    nan = np.isnan(y64)
    inf = ~fin & ~nan
    assert y.shape == y64.shape, f"{what}: shape {y.shape} != {y64.shape}"
    assert np.all(np.isnan(y[nan])), f"{what}: NaN expected"
    assert np.array_equal(y[inf], y64[inf]), f"{what}: Inf mismatch"
    err = np.abs(y[fin] - y64[fin])
    ok = err <= bound[fin]
    if not np.all(ok):
        idx = np.argwhere(fin)[~ok][:5]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} elements outside the bound, first "
                             f"{idx.tolist()} y={y[tuple(idx.T)]} ref={y64[tuple(idx.T)]} "
                             f"bound={bound[tuple(idx.T)]}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound[fin] > 0, err / bound[fin], 0.0)
    return float(r.max()) if r.size else 0.0


def check_top1(y_gpu: np.ndarray, y64: np.ndarray, absum: np.ndarray, what="", rel=1e-3):
    """Top-1 over the last axis: the GPU's argmax must be a maximum of y64 within the error bound
    (a tie within the bound may resolve either way).  Returns the number of exact agreements."""
    g = np.argmax(np.asarray(y_gpu, dtype=np.float64), axis=-1)
    o = oracle.top1(y64)
    agree = 0
    for m in range(y64.shape[0]):
        a, b = int(g[m]), int(o[m])
        if a == b:
            agree += 1
            continue
        slack = rel * (absum[m, a] + absum[m, b])
        assert y64[m, a] >= y64[m, b] - slack, (f"{what}: row {m}: GPU argmax {a} "
                                                f"(y64 {y64[m, a]}) vs oracle {b} (y64 {y64[m, b]})")
    return agree


def check_y_bf16(y16, y32: np.ndarray, y64: np.ndarray, absum: np.ndarray, what="", rel=1e-3):
    """A bfloat16 output (W12_OUT_BF16) against the float output of the same call and the oracle:
    bit for bit the float output rounded to nearest even (torch's rounding on the CPU, NaN where
    NaN), and within the GEMM bound plus half a bfloat16 unit in the last place (relative 2^-8)."""
    import torch
    want = torch.from_numpy(np.ascontiguousarray(y32)).to(torch.bfloat16)
    got = y16.cpu()
    assert tuple(got.shape) == tuple(want.shape), f"{what}: shape {tuple(got.shape)}"
    wn, gn = torch.isnan(want.float()), torch.isnan(got.float())
    assert torch.equal(wn, gn), f"{what}: NaN positions differ"
    assert torch.equal(want.view(torch.int16)[~wn], got.view(torch.int16)[~gn]), \
        f"{what}: bfloat16 output is not the rounded float output"
    y = got.float().numpy().astype(np.float64)
    b = rel * absum
    fin = np.isfinite(y64)
    err = np.abs(y[fin] - y64[fin])
    ok = err <= b[fin] + 2.0 ** -8 * (np.abs(y64[fin]) + b[fin])
    assert np.all(ok), f"{what}: {np.count_nonzero(~ok)} elements outside the bound"
