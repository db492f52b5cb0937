"""GPU parity of the separate 8-bit Q-pass copy (w12_i8_build, w12_i8_gemm, w12_i8_top1) against
the oracle's reading R16 (summary page, Main Findings: an INT8 copy read by the Q pass).

Bars: the copy (codes in storage order and per-row scales) byte-identical to the oracle's; Q-pass
outputs within 1e-3 * sum_k |x[m,k] (s q)[n,k]| of the float64 oracle, per element; one-hot x
returns float32(s q) and every escape exactly; top-1 a maximum within the bound, and exactly the
argmax of the same pass's outputs on a shape too large to split.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from lossless_bit_weight_02_amd import synth
from tests.gpu_util import check_y, check_y_bf16, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_weight_02_amd import w12
    w12.lib()


def _w12():
    from lossless_bit_weight_02_amd import w12
    return w12


def _weights(n, k, seed, p_zero=0.01, p_out=5e-4):
    rng = np.random.default_rng(seed)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < p_zero] = 0
    w[rng.random((n, k)) < p_out] = 0x4400
    return w


def _copy_check(w_bits, what):
    """Encode on the GPU, build the copy there, compare it with the oracle's; return
    (record, copy, oracle record, oracle copy)."""
    w12 = _w12()
    say(f"i8 build {what} {w_bits.shape}")
    rec = w12.encode(to_dev(w_bits))
    cp = w12.i8_build(rec)
    ref = oracle.encode(w_bits)
    ocp = oracle.i8_copy(ref)
    got = cp.to_numpy()
    want_q = oracle.to_storage(dataclasses.replace(ref, ae=ocp.q.view(np.uint8)))[0].view(np.int8)
    assert np.array_equal(got["scale"].view(np.uint32), ocp.scale.view(np.uint32)), f"{what}: scales"
    if not np.array_equal(got["q_s"], want_q):
        bad = np.argwhere(got["q_s"] != want_q)
        raise AssertionError(f"{what}: codes differ at {bad[:5].tolist()} ({len(bad)} positions)")
    return rec, cp, ref, ocp


def _gemm_check(x_bits, cp, ref, ocp, what, paths=("gemv", "mfma", "auto")):
    w12 = _w12()
    wq = oracle.i8_weights64(ref, ocp)
    y64 = oracle.gemm64_f(x_bits, wq)
    absum = oracle.abs_bound64_f(x_bits, wq)
    x = to_dev(x_bits)
    for path in paths:
        say(f"i8 gemm {what} m={x_bits.shape[0]} path={path}")
        y = w12.i8_gemm(x, cp, path=path).cpu().numpy()
        check_y(y, y64, absum, f"{what} i8 {path}")
    return y64, absum


def test_i8_tiny_config():
    w, spec, tid = synth.config_weight("tiny")
    rec, cp, ref, ocp = _copy_check(w, "tiny")
    x = synth.gen_x(16, spec.k, tensor_id=tid)
    for m in (1, 3, 8, 16):
        _gemm_check(x[:m], cp, ref, ocp, "tiny")


@pytest.mark.parametrize("n,k,ms", [
    (300, 1152, (1, 2, 5, 8, 17, 32, 40, 64, 100)),   # every kernel family, ragged tiles (passes
                                                       # of 32 above 32 rows on 19 tiles)
    (6160, 256, (40, 64, 100)),                        # 385 tiles: the three/four-tile kernel
    (64, 5120, (1, 16, 32)),                           # split k (few tiles)
    (320, 17408, (1, 32)),                             # split k, long rows
    (1037, 640, (4, 33)),
])
def test_i8_shapes(n, k, ms):
    w = _weights(n, k, n + k)
    rec, cp, ref, ocp = _copy_check(w, f"{n}x{k}")
    x = synth.gen_x(max(ms), k, tensor_id=n)
    for m in ms:
        _gemm_check(x[:m], cp, ref, ocp, f"{n}x{k}")


def test_i8_edge_rows():
    """Rows with a far escape above the window, all-zero rows (no in-window weight: the scale is
    the window floor / 127 and every code 0), an Inf weight and a constant row."""
    k = 256
    rng = np.random.default_rng(3)
    w = synth.f32_to_bf16_bits((rng.standard_normal((40, k)) * 0.02).astype(np.float32))
    w[0, 5] = 0x6F00                      # 2^95: outside the row's window
    w[1] = 0                              # nothing in the window
    w[2, 7] = 0x7F80                      # +Inf: an escape
    w[3] = 0x3F80                         # constant 1.0
    w[4, :64] = 0x0001                    # subnormals
    rec, cp, ref, ocp = _copy_check(w, "edge rows")
    x = synth.gen_x(4, k, tensor_id=9)
    w12 = _w12()
    wq = oracle.i8_weights64(ref, ocp)
    for path in ("gemv", "mfma"):
        y = w12.i8_gemm(to_dev(x), cp, path=path).cpu().numpy().astype(np.float64)
        y64 = oracle.gemm64_f(x, wq)
        assert np.all(np.isinf(y[:, 2]) & (np.sign(y[:, 2]) == np.sign(y64[:, 2])))
        keep = np.arange(40) != 2
        check_y(y[:, keep], y64[:, keep], oracle.abs_bound64_f(x, wq)[:, keep], f"edge rows {path}")


def test_i8_one_hot_exact():
    """x = e_k returns float32(s_n q[n, k]) for in-window weights and the exact value for
    escapes, on both kernel families."""
    w = _weights(48, 512, 11)
    rec, cp, ref, ocp = _copy_check(w, "one-hot")
    w12 = _w12()
    esc = oracle.escaped_mask(ref)
    for kk in (0, 1, 31, 32, 127, 128, 300, 511):
        x = np.zeros((16, 512), dtype=np.uint16)
        x[:, kk] = 0x3F80
        want = (ocp.scale * ocp.q[:, kk].astype(np.float32)).astype(np.float32)
        want = np.where(esc[:, kk], oracle.bf16_to_f64(w[:, kk]).astype(np.float32), want)
        for path, m in (("gemv", 1), ("mfma", 16)):
            y = w12.i8_gemm(to_dev(x[:m]), cp, path=path).cpu().numpy()
            assert np.array_equal(y[0].view(np.uint32), want.view(np.uint32)), (kk, path)


def test_i8_top1_and_bf16_out():
    w = _weights(4000, 1024, 21)
    rec, cp, ref, ocp = _copy_check(w, "top1")
    w12 = _w12()
    x_bits = synth.gen_x(40, 1024, tensor_id=21)
    x = to_dev(x_bits)
    wq = oracle.i8_weights64(ref, ocp)
    y64, absum = oracle.gemm64_f(x_bits, wq), oracle.abs_bound64_f(x_bits, wq)
    say("i8 top1")
    idx, val = (t.cpu().numpy() for t in w12.i8_top1(x, cp))
    for j in range(40):
        a = int(idx[j])
        assert y64[j, a] >= y64[j].max() - 1e-3 * (absum[j, a] + absum[j, np.argmax(y64[j])])
        assert abs(val[j] - y64[j, a]) <= 1e-3 * absum[j, a]
    for m, path in ((1, "gemv"), (16, "mfma"), (40, "mfma")):
        say(f"i8 bf16 out m={m} {path}")
        y = w12.i8_gemm(x[:m], cp, path=path).cpu().numpy()
        y16 = w12.i8_gemm(x[:m], cp, path=path, out_bf16=True)
        check_y_bf16(y16, y, y64[:m], absum[:m], f"i8 bf16 out m={m} {path}")


def test_i8_full_lm_head():
    """LM head [152064, 5120] at M=16 (the Q-pass config): the copy byte-identical to the oracle's,
    every output within the bound (automatic path and matrix cores), top-1 exactly the argmax of
    the automatic path's full outputs (the family the top-1 entry point runs)."""
    from tests import oracle_pool
    w12 = _w12()
    w, spec, tid = synth.config_weight("lm_head")
    say("lm_head i8: encode + build")
    rec = w12.encode(to_dev(w))
    cp = w12.i8_build(rec)
    x_bits = synth.gen_x(16, spec.k, tensor_id=tid)
    x = to_dev(x_bits)
    y = w12.i8_gemm(x, cp).cpu().numpy()
    y_mf = w12.i8_gemm(x, cp, path="mfma").cpu().numpy()
    idx, val = (t.cpu().numpy() for t in w12.i8_top1(x, cp))
    got = cp.to_numpy()
    ex = oracle_pool.make_pool()
    try:
        say("lm_head i8: oracle copy and GEMM over row chunks")
        parts = oracle_pool.i8_chunks(x_bits, w, ex)
    finally:
        ex.shutdown()
    scale = np.concatenate([p[0] for p in parts])
    q_s = np.concatenate([p[1] for p in parts])
    y64 = np.concatenate([p[2] for p in parts], axis=1)
    absum = np.concatenate([p[3] for p in parts], axis=1)
    assert np.array_equal(got["scale"].view(np.uint32), scale.view(np.uint32))
    assert np.array_equal(got["q_s"], q_s)
    check_y(y, y64, absum, "lm_head i8")
    check_y(y_mf, y64, absum, "lm_head i8 matrix cores")
    want = np.argmax(y, axis=1)
    assert np.array_equal(idx, want)
    assert np.array_equal(val.view(np.uint32), y[np.arange(16), want].view(np.uint32))

