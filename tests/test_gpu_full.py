"""GPU parity at the full workload sizes, in the launch configurations bench.py times.

gate+up [34816, 5120] (every M of its config, both kernel families, and 48, 128 and 256 rows of
x, so the three- and eight-tile matrix-core kernels run with every wave busy), the LM-head-shaped
Q pass [152064, 5120] at M=16 with top-1 and at 48 and 128 rows (several rounds of tiles per wave),
and three layers (0, 31, 63) of the 64-layer 27B-class stack.
The oracle runs over row chunks in spawned worker processes (tests/oracle_pool.py), so every
output element and every stored byte is compared, not a sample.
"""
import numpy as np
import pytest

from lossless_bit_weight_02_amd import synth
from tests import oracle_pool
from tests.gpu_util import (assert_records_equal, check_top1, check_y, check_y_bf16, record_numpy,
                            say, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_weight_02_amd import w12
    w12.lib()  # fails loudly if the library is missing


@pytest.fixture(scope="module")
def pool():
    ex = oracle_pool.make_pool()
    yield ex
    ex.shutdown()


def _w12():
    from lossless_bit_weight_02_amd import w12
    return w12


def _codec(w, what, pool):
    """GPU encode byte-identical to the oracle's record, GPU decode bit-exact; returns the record."""
    w12 = _w12()
    dw = to_dev(w)
    say(f"{what}: encode {w.shape}")
    rec = w12.encode(dw)
    say(f"{what}: oracle encode (row chunks)")
    ref = oracle_pool.encode(w, pool)
    assert_records_equal(record_numpy(rec), ref, what)
    say(f"{what}: decode")
    back = w12.decode(rec)
    assert torch.equal(back.view(torch.int16), dw.view(torch.int16)), f"{what}: decode not bit-exact"
    del back
    return rec, dw


def test_gate_up_full(pool):
    """Config gate+up: codec, exact GEMM at M = 1, 2, 4, 8, 16, 32, 64 on the three kernel families
    (the streaming kernel in passes of 32 rows), the Q pass at M=16 and the dense baseline at M=1
    and 32 -- every output element."""
    w12 = _w12()
    w, spec, tid = synth.config_weight("gate_up")
    rec, dw = _codec(w, "gate_up", pool)
    x = synth.gen_x(64, spec.k, tensor_id=tid)
    say("gate_up: oracle GEMM M=64 (all rows)")
    y64, absum = oracle_pool.gemm(x, w, pool)
    for m in (1, 2, 4, 8, 16, 32, 64):
        for path in ("gemv", "mfma", "stream"):
            say(f"gate_up: gemm m={m} path={path}")
            y = w12.gemm(to_dev(x[:m]), rec, path=path).cpu().numpy()
            check_y(y, y64[:m], absum[:m], f"gate_up w12 m={m} {path}")
    say("gate_up: oracle Q-pass GEMM M=16")
    yq64, qabs = oracle_pool.gemm(x[:16], w, pool, view="q8")
    for path in ("gemv", "mfma", "stream"):
        say(f"gate_up: q8_gemm m=16 path={path}")
        yq = w12.q8_gemm(to_dev(x[:16]), rec, path=path).cpu().numpy()
        check_y(yq, yq64, qabs, f"gate_up q8 m=16 {path}")
    bt = w12.bf16_tiles(dw)
    for m, path in ((1, "gemv"), (32, "mfma"), (32, "stream")):
        say(f"gate_up: bf16_gemm m={m} path={path}")
        yb = w12.bf16_gemm(to_dev(x[:m]), bt, path=path).cpu().numpy()
        check_y(yb, y64[:m], absum[:m], f"gate_up bf16 m={m} {path}")


def test_lm_head_q_pass_top1(pool):
    """Config LM head [152064, 5120], M=16: Q pass (truncated and midpoint views) and exact pass on
    every output, on the automatic path (the streaming kernel, three tiles per wave) and the
    matrix cores; the top-1 token of each row within the error bound (a near-tie may resolve
    either way) and the top-1 entry points equal to the argmax of the same kernel's outputs."""
    w12 = _w12()
    w, spec, tid = synth.config_weight("lm_head")
    rec, dw = _codec(w, "lm_head", pool)
    del dw
    x = synth.gen_x(16, spec.k, tensor_id=tid)
    xd = to_dev(x)
    say("lm_head: q8_gemm m=16")
    yq = w12.q8_gemm(xd, rec).cpu().numpy()
    say("lm_head: oracle Q-pass GEMM (all rows)")
    yq64, qabs = oracle_pool.gemm(x, w, pool, view="q8")
    check_y(yq, yq64, qabs, "lm_head q8")
    agree_q = check_top1(yq, yq64, qabs, "lm_head q8 top-1")
    say("lm_head: gemm m=16")
    y = w12.gemm(xd, rec).cpu().numpy()
    say("lm_head: oracle exact GEMM (all rows)")
    y64, absum = oracle_pool.gemm(x, w, pool)
    check_y(y, y64, absum, "lm_head exact")
    agree = check_top1(y, y64, absum, "lm_head exact top-1")
    say(f"lm_head: top-1 exact agreement q8 {agree_q}/16, exact {agree}/16")
    # the top-1 entry points run the streaming kernel where the automatic path runs it in one row
    # group (both passes here, three tiles per wave), so they must pick exactly the argmax of its
    # full outputs (ties to the lowest index) and report exactly that value
    say("lm_head: matrix-core gemm m=16 (q8, exact); automatic q8 midpoint")
    yq_mf = w12.q8_gemm(xd, rec, path="mfma").cpu().numpy()
    y_mf = w12.gemm(xd, rec, path="mfma").cpu().numpy()
    yqm = w12.q8_gemm(xd, rec, midpoint=True).cpu().numpy()
    check_y(yq_mf, yq64, qabs, "lm_head q8 matrix cores")
    check_y(y_mf, y64, absum, "lm_head exact matrix cores")
    say("lm_head: oracle midpoint-view GEMM (all rows)")
    yqm64, qmabs = oracle_pool.gemm(x, w, pool, view="q8m")
    check_y(yqm, yqm64, qmabs, "lm_head q8 midpoint")
    for name, fn, yy in (("q8", w12.q8_top1, yq), ("exact", w12.gemm_top1, y),
                         ("q8 midpoint", lambda xx, rr: w12.q8_top1(xx, rr, midpoint=True), yqm)):
        say(f"lm_head: {name} top-1 entry point")
        idx, val = (t.cpu().numpy() for t in fn(xd, rec))
        want = np.argmax(yy, axis=1)
        assert np.array_equal(idx, want), name
        assert np.array_equal(val.view(np.uint32), yy[np.arange(16), want].view(np.uint32)), name


@pytest.mark.parametrize("layer", [0, 31, 63])
def test_stack_layer(pool, layer):
    """Config 27B stack, layers 0, 31 and 63 (all seven projections): codec and the exact GEMM at
    M = 1 and 32 in the bench's launch configuration (GEMV at 1, MFMA at 32)."""
    w12 = _w12()
    cfg = synth.CONFIGS["stack"]
    for p in range(len(synth.STACK_PROJ)):
        tid, label, spec = cfg.weights[layer * len(synth.STACK_PROJ) + p]
        w = synth.gen_weight(spec, 0, tid)
        rec, dw = _codec(w, label, pool)
        del dw
        x = synth.gen_x(32, spec.k, tensor_id=tid)
        y64, absum = oracle_pool.gemm(x, w, pool)
        for m in (1, 32):
            say(f"{label}: gemm m={m}")
            y = w12.gemm(to_dev(x[:m]), rec).cpu().numpy()
            check_y(y, y64[:m], absum[:m], f"{label} w12 m={m}")


def _formats(w12, rec, bt):
    """(name, call, oracle view) of the four GEMMs on one record: exact pass, both Q-pass views and
    the dense baseline."""
    return (("w12", lambda x, **kw: w12.gemm(x, rec, **kw), "exact"),
            ("q8", lambda x, **kw: w12.q8_gemm(x, rec, **kw), "q8"),
            ("q8 midpoint", lambda x, **kw: w12.q8_gemm(x, rec, midpoint=True, **kw), "q8m"),
            ("bf16", lambda x, **kw: w12.bf16_gemm(x, bt, **kw), "exact"))


def test_gate_up_many_rows(pool):
    """gate+up [34816, 5120] at 48 rows of x (three-tile kernel: 2176 tiles, every wave of the chip
    busy), 128 rows (one eight-tile pass: 9 busy waves per workgroup) and 256 rows (two passes), on
    the automatic path bench.py times: exact pass, both Q-pass views and the baseline, float and
    bfloat16 outputs, every element against the oracle."""
    w12 = _w12()
    w, spec, tid = synth.config_weight("gate_up")
    dw = to_dev(w)
    say("gate_up many rows: encode")
    rec = w12.encode(dw)
    bt = w12.bf16_tiles(dw)
    del dw
    x = synth.gen_x(256, spec.k, tensor_id=tid)
    ref = {}
    for view in ("exact", "q8", "q8m"):
        say(f"gate_up many rows: oracle GEMM M=256 ({view})")
        ref[view] = oracle_pool.gemm(x, w, pool, view=view)
    for m in (48, 128, 256):
        xd = to_dev(x[:m])
        for name, fn, view in _formats(w12, rec, bt):
            y64, absum = ref[view]
            say(f"gate_up: {name} m={m} float out")
            y = fn(xd).cpu().numpy()
            check_y(y, y64[:m], absum[:m], f"gate_up {name} m={m}")
            say(f"gate_up: {name} m={m} bfloat16 out")
            y16 = fn(xd, out_bf16=True)
            check_y_bf16(y16, y, y64[:m], absum[:m], f"gate_up {name} m={m} bf16 out")


@pytest.mark.parametrize("m", [48, 128])
def test_lm_head_many_rows(pool, m):
    """LM head [152064, 5120] (9504 tiles: four rounds of tiles per wave) at 48 rows of x (the
    three-tile kernel) and 128 rows (the eight-tile kernel): exact pass and Q pass, every element
    against the oracle."""
    w12 = _w12()
    w, spec, tid = synth.config_weight("lm_head")
    dw = to_dev(w)
    say(f"lm_head m={m}: encode")
    rec = w12.encode(dw)
    del dw
    x = synth.gen_x(m, spec.k, tensor_id=tid)
    xd = to_dev(x)
    for name, fn, view in (("w12", w12.gemm, "exact"), ("q8", w12.q8_gemm, "q8")):
        say(f"lm_head: {name} m={m}")
        y = fn(xd, rec).cpu().numpy()
        say(f"lm_head: oracle GEMM m={m} ({view})")
        y64, absum = oracle_pool.gemm(x, w, pool, view=view)
        check_y(y, y64, absum, f"lm_head {name} m={m}")
