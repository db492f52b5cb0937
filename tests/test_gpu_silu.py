"""GPU parity of the SiLU(gate) * up epilogue (w12_gemm_silu_mul) and of the row-interleaved
gate+up record it reads (w12_interleave_rows), against the oracle's reading R17 (summary page,
Main Findings: W12 in plain decoding, where the gate and up projections feed SiLU(gate) * up).

Bars: the interleaved record byte-identical to the oracle's encoding of the interleaved matrix;
every h within 1.1 B_g (|u| + B_u) + |silu(g)| B_u + 2^-20 |h| of the float64 oracle (B the GEMM
bound of each input row); bfloat16 h exactly the rounding of the float h and within that bound
plus half a bfloat16 unit in the last place.
"""
import numpy as np
import pytest

import oracle
from lossless_bit_weight_02_amd import synth
from tests.gpu_util import assert_records_equal, record_numpy, say, to_dev

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


def _weights(i, k, seed):
    rng = np.random.default_rng(seed)
    g = synth.f32_to_bf16_bits((rng.standard_normal((i, k)) * 0.03).astype(np.float32))
    u = synth.f32_to_bf16_bits((rng.standard_normal((i, k)) * 0.03).astype(np.float32))
    for w in (g, u):
        w[rng.random((i, k)) < 0.01] = 0
        w[rng.random((i, k)) < 3e-4] = 0x4300
    return g, u


def check_h(h, y64, absum, what):
    h = np.asarray(h, dtype=np.float64)
    want = oracle.silu_mul64(y64)
    bound = oracle.silu_mul_bound(y64, absum)
    assert h.shape == want.shape, f"{what}: shape {h.shape} != {want.shape}"
    err = np.abs(h - want)
    ok = err <= bound
    if not np.all(ok):
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} outputs outside the bound, first "
                             f"{idx.tolist()} h={h[tuple(idx.T)]} want={want[tuple(idx.T)]}")


def check_h_bf16(h16, h32, y64, absum, what):
    want = torch.from_numpy(np.ascontiguousarray(h32)).to(torch.bfloat16)
    got = h16.cpu()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16)), f"{what}: not the rounded float h"
    h = got.float().numpy().astype(np.float64)
    ref = oracle.silu_mul64(y64)
    bound = oracle.silu_mul_bound(y64, absum)
    assert np.all(np.abs(h - ref) <= bound + 2.0 ** -8 * (np.abs(ref) + bound)), f"{what}: outside the bound"


def _interleaved(gate_bits, up_bits, what):
    """GPU interleave of the two GPU records, byte-compared with the oracle's encoding of the
    interleaved matrix; returns (record, interleaved bits)."""
    w12 = _w12()
    say(f"interleave {what}")
    gr, ur = w12.encode(to_dev(gate_bits)), w12.encode(to_dev(up_bits))
    rec = w12.interleave_rows(gr, ur)
    wi = oracle.interleave_rows(gate_bits, up_bits)
    assert_records_equal(record_numpy(rec), oracle.encode(wi), f"interleave {what}")
    return rec, wi


@pytest.mark.parametrize("i,k,ms,paths", [
    (40, 256, (1, 2, 5, 8), ("gemv", "auto")),             # GEMV, ragged tile count
    (200, 1152, (1, 16, 20, 32, 40, 64, 100), ("mfma", "auto")),   # 25 tiles: passes of 32 above 32
    (3080, 256, (40, 64, 100, 128), ("mfma", "auto")),     # 385 tiles: three/four- and eight-tile
    (32, 5120, (1, 16, 32), ("gemv", "mfma")),             # split k (few tiles)
    (160, 17408, (1, 32), ("gemv", "mfma")),               # split k, long rows
    (64, 6144, (8,), ("gemv",)),                           # GEMV over two k slices (float sums)
])
def test_silu_mul_shapes(i, k, ms, paths):
    w12 = _w12()
    g, u = _weights(i, k, i + k)
    rec, wi = _interleaved(g, u, f"{i}x{k}")
    x = synth.gen_x(max(ms), k, tensor_id=i)
    y64, absum = oracle.gemm64(x, wi), oracle.abs_bound64(x, wi)
    for m in ms:
        xd = to_dev(x[:m])
        for path in paths:
            what = f"silu {i}x{k} m={m} {path}"
            say(what)
            h = w12.gemm_silu_mul(xd, rec, path=path).cpu().numpy()
            check_h(h, y64[:m], absum[:m], what)
            h16 = w12.gemm_silu_mul(xd, rec, path=path, out_bf16=True)
            check_h_bf16(h16, h, y64[:m], absum[:m], what + " bf16")


def test_silu_mul_equals_pairs_of_gemm():
    """The epilogue applies silu(g) * u in float to the very outputs w12_gemm computes on the same
    record and path: recomputing it from those outputs with torch in float32 stays within a few
    float32 rounding steps (the exp of the device library and of torch may differ slightly)."""
    w12 = _w12()
    g, u = _weights(96, 1024, 5)
    rec, wi = _interleaved(g, u, "pairs")
    x = to_dev(synth.gen_x(32, 1024, tensor_id=5))
    gate, up = oracle.silu_rows(96)
    for m, path in ((1, "gemv"), (32, "mfma")):
        y = w12.gemm(x[:m], rec, path=path)
        want = torch.nn.functional.silu(y[:, gate]) * y[:, up]
        h = w12.gemm_silu_mul(x[:m], rec, path=path)
        assert torch.allclose(h, want, rtol=1e-5, atol=1e-30), path


def test_interleave_errors():
    w12 = _w12()
    g, u = _weights(24, 128, 1)
    gr, ur = w12.encode(to_dev(g)), w12.encode(to_dev(u[:16]))
    with pytest.raises(w12.W12Error) as ei:
        w12.interleave_rows(gr, ur)
    assert ei.value.status == w12.W12_ERR_SHAPE
    odd = w12.encode(to_dev(g[:8]))                      # n = 8: not a multiple of 16 for the GEMM
    with pytest.raises(w12.W12Error) as ei:
        w12.gemm_silu_mul(to_dev(synth.gen_x(1, 128, tensor_id=1)), odd)
    assert ei.value.status == w12.W12_ERR_SHAPE


def test_silu_mul_full_gate_up():
    """The configs' gate+up shape as the two [17408, 5120] halves of the MLP, interleaved, at
    M = 1 and 32 (the bench's rows): every output against the oracle."""
    from tests import oracle_pool
    w12 = _w12()
    w, spec, tid = synth.config_weight("gate_up")
    half = w.shape[0] // 2
    gr, ur = w12.encode(to_dev(w[:half])), w12.encode(to_dev(w[half:]))
    say("full gate+up: interleave")
    rec = w12.interleave_rows(gr, ur)
    del gr, ur
    wi = oracle.interleave_rows(w[:half], w[half:])
    x = synth.gen_x(32, spec.k, tensor_id=tid)
    hs = {}
    for m in (1, 32):
        say(f"full gate+up silu m={m}")
        hs[m] = w12.gemm_silu_mul(to_dev(x[:m]), rec).cpu().numpy()
    ex = oracle_pool.make_pool()
    try:
        say("full gate+up: oracle record and GEMM")
        ref = oracle_pool.encode(wi, ex)
        assert_records_equal(record_numpy(rec), ref, "full interleave")
        y64, absum = oracle_pool.gemm(x, wi, ex)
    finally:
        ex.shutdown()
    for m in (1, 32):
        check_h(hs[m], y64[:m], absum[:m], f"full gate+up silu m={m}")
