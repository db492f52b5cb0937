"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: encode and decode byte-identical / bit-exact; GEMM outputs within
1e-3 * sum_k |x[m,k] W[n,k]| of the float64 oracle, per element.
"""
import numpy as np
import pytest

import oracle
from lossless_bit_weight_02_amd import synth
from tests.gpu_util import (assert_records_equal, check_gemm, record_numpy, say, to_dev,
                            to_host_bits)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_weight_02_amd import w12
    w12.lib()  # fails loudly if the library is missing


def _w12():
    from lossless_bit_weight_02_amd import w12
    return w12


def _encode_check(w_bits, what):
    w12 = _w12()
    say(f"encode {what} {w_bits.shape}")
    rec = w12.encode(to_dev(w_bits))
    got = record_numpy(rec)
    assert_records_equal(got, oracle.encode(w_bits), what)
    say(f"decode {what}")
    back = to_host_bits(w12.decode(rec))
    assert np.array_equal(back, w_bits), f"{what}: decode not bit-exact"
    return rec


# ------------------------------------------------------------------------------------------------
# encode / decode
# ------------------------------------------------------------------------------------------------
def test_codec_tiny():
    w, _, _ = synth.config_weight("tiny")
    _encode_check(w, "tiny")


def test_codec_attn():
    w, _, _ = synth.config_weight("attn")
    _encode_check(w, "attn 5120x5120")


@pytest.mark.parametrize("layout", ["natural", "shuffled"])
def test_codec_all_65536_patterns(layout):
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if layout == "shuffled":
        a = np.random.default_rng(1).permutation(a)
    _encode_check(a.reshape(256, 256), f"all bf16 patterns ({layout})")
    _encode_check(a.reshape(64, 1024), f"all bf16 patterns 64x1024 ({layout})")


def test_codec_edge_rows():
    k = 128
    rows = [np.zeros(k, np.uint16),                                   # all zero -> base 1, all escape
            np.full(k, 0x8000, np.uint16),                            # all -0
            np.full(k, 0x7FC0, np.uint16),                            # all NaN
            np.tile(np.array([0x7F80, 0xFF80, 0x0001, 0x8001], np.uint16), k // 4),  # Inf/subnormal
            np.full(k, 0x3F80, np.uint16),                            # constant
            (np.arange(k, dtype=np.uint16) << 7) | 0x5,                # exponents 0..95 (wide row)
            ]
    w = np.stack(rows)
    _encode_check(w, "edge rows")


def test_codec_ragged_rows_and_min_k():
    rng = np.random.default_rng(4)
    for n, k in ((1, 128), (3, 128), (17, 256), (37, 384), (129, 640), (255, 1152)):
        w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        w[rng.random((n, k)) < 0.01] = 0
        _encode_check(w, f"random {n}x{k}")


def test_encode_capacity_protocol():
    """A too-small esc_cap returns W12_ERR_CAPACITY with the escape total; the binding then sizes
    the arrays exactly and encodes again."""
    import ctypes
    w12 = _w12()
    w, _, _ = synth.config_weight("tiny")
    dev_w = to_dev(w)
    n, k = w.shape
    npad = w12.padded_rows(n)
    base = torch.empty(n, dtype=torch.uint8, device="cuda")
    ae = torch.empty(npad * k, dtype=torch.uint8, device="cuda")
    lo = torch.empty(npad * k // 2, dtype=torch.uint8, device="cuda")
    ptr = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    col = torch.empty(4, dtype=torch.int32, device="cuda")
    val = torch.empty(4, dtype=torch.int16, device="cuda")
    s = w12._W12Weight(n, k, base.data_ptr(), ae.data_ptr(), lo.data_ptr(), ptr.data_ptr(),
                       col.data_ptr(), val.data_ptr(), 4)
    n_esc = ctypes.c_uint64(0)
    say("encode with esc_cap=4")
    st = w12.lib().w12_encode(dev_w.data_ptr(), ctypes.byref(s), ctypes.byref(n_esc),
                              torch.cuda.current_stream().cuda_stream)
    ref = oracle.encode(w)
    assert st == w12.W12_ERR_CAPACITY
    assert n_esc.value == ref.n_esc
    assert np.array_equal(base.cpu().numpy(), ref.base)
    assert np.array_equal(ptr.cpu().numpy().view(np.uint32), ref.esc_ptr)
    rec = w12.encode(dev_w, esc_guess=3)
    assert_records_equal(record_numpy(rec), ref, "re-encode after capacity")


def test_encode_deterministic():
    w12 = _w12()
    w, _, _ = synth.config_weight("attn", rows=(0, 1024))
    dw = to_dev(w)
    say("encode twice")
    a, b = record_numpy(w12.encode(dw)), record_numpy(w12.encode(dw))
    assert_records_equal(a, b, "two encodes")


def test_encode_errors():
    w12 = _w12()
    bad = torch.zeros((4, 192), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w12.W12Error) as ei:
        w12.encode(bad)
    assert ei.value.status == w12.W12_ERR_SHAPE


# ------------------------------------------------------------------------------------------------
# GEMMs
# ------------------------------------------------------------------------------------------------
def _gemm_case(w_bits, x_bits, what, paths=("gemv", "mfma"), rec=None, rows=None):
    """Exact pass, Q pass and the dense baseline on both kernel families."""
    w12 = _w12()
    if rec is None:
        rec = w12.encode(to_dev(w_bits))
    ref = oracle.encode(w_bits if rows is None else w_bits)
    q8w = oracle.q8_view_bits(ref)
    x = to_dev(x_bits)
    dw = w12.bf16_tiles(to_dev(w_bits))
    worst = {}
    for path in paths:
        say(f"gemm {what} m={x_bits.shape[0]} path={path}")
        y = w12.gemm(x, rec, path=path).cpu().numpy()
        worst[("w12", path)] = check_gemm(y, x_bits, w_bits, f"{what} w12 {path}")
        say(f"q8_gemm {what} path={path}")
        yq = w12.q8_gemm(x, rec, path=path).cpu().numpy()
        worst[("q8", path)] = check_gemm(yq, x_bits, q8w, f"{what} q8 {path}")
        say(f"bf16_gemm {what} path={path}")
        yb = w12.bf16_gemm(x, dw, path=path).cpu().numpy()
        worst[("bf16", path)] = check_gemm(yb, x_bits, w_bits, f"{what} bf16 {path}")
    return worst


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65])
def test_gemm_tiny_all_m(m):
    w, spec, tid = synth.config_weight("tiny")
    x = synth.gen_x(m, spec.k, tensor_id=tid)
    _gemm_case(w, x, "tiny")


def test_gemm_attn_m1():
    w, spec, tid = synth.config_weight("attn")
    x = synth.gen_x(1, spec.k, tensor_id=tid)
    _gemm_case(w, x, "attn 5120x5120")


def _seeded_shapes(count, seed):
    """Shapes drawn once from a fixed seed: ragged n, k a multiple of 128, m up to 260 (so the
    GEMV, the one- and two-tile matrix-core kernels, split k and, above 32 rows on these few-tile
    shapes, passes of 32 rows and the dense baseline's streaming kernel all occur)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        n = int(rng.integers(1, 900))
        k = 128 * int(rng.integers(1, 24))
        m = int(rng.choice([int(rng.integers(1, 9)), int(rng.integers(9, 65)), int(rng.integers(65, 261))]))
        out.append((n, k, m))
    return out


@pytest.mark.parametrize("n,k,m", _seeded_shapes(16, 2027))
def test_gemm_seeded_shapes_auto_path(n, k, m):
    """The automatic kernel choice on seeded shapes: exact pass, Q pass (both views) and the dense
    baseline against the oracle; zeros and far outliers make escapes in most tiles."""
    rng = np.random.default_rng(n * 131 + k * 7 + m)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[rng.random((n, k)) < 5e-4] = 0x4400
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    _gemm_case(w, x, f"seeded {n}x{k}", paths=("auto",))
    w12 = _w12()
    rec = w12.encode(to_dev(w))
    say(f"q8_gemm midpoint seeded {n}x{k} m={m}")
    y = w12.q8_gemm(to_dev(x), rec, midpoint=True).cpu().numpy()
    check_gemm(y, x, oracle.q8_view_bits(oracle.encode(w), midpoint=True), f"seeded {n}x{k} q8 midpoint")


@pytest.mark.parametrize("n,k,m", [(1, 128, 1), (37, 256, 3), (129, 384, 16), (300, 1152, 8),
                                   (300, 1152, 40), (77, 4224, 1), (64, 9216, 8), (50, 640, 2),
                                   (33, 128, 64), (16, 3968, 5), (1000, 2176, 33), (8, 128, 100)])
def test_gemm_ragged(n, k, m):
    rng = np.random.default_rng(n * 7 + k + m)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    _gemm_case(w, x, f"ragged {n}x{k}")


@pytest.mark.parametrize("n,k,ms", [(17989, 384, (1,)), (33609, 128, (1, 2, 4))])
def test_gemv_many_rounds(n, k, ms):
    """More 16-row tiles than the persistent GEMV grid holds workgroups (1125 and 2101 tiles), so
    workgroups take several tiles and the last round is partly idle; the last tile is ragged (5
    and 9 rows)."""
    rng = np.random.default_rng(n + k)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w12 = _w12()
    rec = w12.encode(to_dev(w))
    for m in ms:
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        _gemm_case(w, x, f"many rounds {n}x{k}", paths=("gemv",), rec=rec)


def test_gemm_one_hot_exact():
    """x = e_k must return column k of W exactly, escapes included, on both kernel families."""
    w12 = _w12()
    w, spec, _ = synth.config_weight("tiny")
    rec = w12.encode(to_dev(w))
    cols = [0, 1, 7, 8, 100, 255, 256, 511]
    x = np.zeros((len(cols), spec.k), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80
    want = oracle.bf16_to_f64(w[:, cols]).T
    for path in ("gemv", "mfma"):
        say(f"one-hot path={path}")
        y = w12.gemm(to_dev(x), rec, path=path).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, want), path
        yq = w12.q8_gemm(to_dev(x), rec, path=path).cpu().numpy().astype(np.float64)
        assert np.array_equal(yq, oracle.bf16_to_f64(oracle.q8_view_bits(oracle.encode(w))[:, cols]).T)


def test_gemm_special_values():
    """NaN / Inf weights propagate; zero, subnormal and -0 weights are exact escapes; an
    all-escape row returns only the placeholder residue allowed by the bound's absolute floor."""
    w12 = _w12()
    k = 128
    rng = np.random.default_rng(9)
    w = synth.f32_to_bf16_bits((rng.standard_normal((8, k)) * 0.05).astype(np.float32))
    w[0, 5] = 0x7F80          # +Inf
    w[1, 9] = 0x7FC1          # NaN
    w[2, :] = 0               # all zero
    w[3, ::2] = 0x0001        # subnormals
    w[4, 3] = 0x8000          # -0
    w[5, :] = 0x3F80          # constant
    w[6, 10] = 0x7F00         # 2^127 (escape, finite)
    w[7, :] = ((np.arange(k) % 40 + 100) << 7).astype(np.uint16)  # wide row: many escapes
    rec = w12.encode(to_dev(w))
    ref = oracle.encode(w)
    assert_records_equal(record_numpy(rec), ref, "special")
    x_all = synth.f32_to_bf16_bits(rng.standard_normal((100, k)).astype(np.float32) * 1e-3)
    # 100 rows: passes of 32 rows on this one-tile record; the same rows stacked over 6152 more
    # (385 tiles) run the eight-tile matrix-core kernel, whose escapes are patched in the epilogue
    w_big = np.concatenate([w, synth.f32_to_bf16_bits((rng.standard_normal((6152, k)) * 0.05).astype(np.float32))])
    rec_big = w12.encode(to_dev(w_big))
    for path, m, rr, ww in (("gemv", 3, rec, w), ("mfma", 3, rec, w), ("mfma", 100, rec, w),
                            ("mfma", 100, rec_big, w_big)):
        say(f"special values path={path} m={m} n={ww.shape[0]}")
        x = x_all[:m]
        y_all = w12.gemm(to_dev(x), rr, path=path).cpu().numpy().astype(np.float64)
        if ww.shape[0] > 8:
            check_gemm(y_all[:, 8:], x, ww[8:], f"special values stacked rows {path} m={m}")
        y = y_all[:, :8]
        y64 = oracle.gemm64(x, w)
        assert np.isinf(y[:, 0]).all() and np.array_equal(np.sign(y[:, 0]), np.sign(y64[:, 0]))
        assert np.isnan(y[:, 1]).all()
        floor = k * np.abs(oracle.bf16_to_f64(x)).max() * 2.0 ** (int(ref.base[2]) - 127) * 2.0 ** -24
        assert np.all(np.abs(y[:, 2]) <= floor)
        check_gemm(y[:, 3:], x, w[3:], f"special rows 3.. {path} m={m}")


def test_gemm_deterministic():
    w12 = _w12()
    w, spec, tid = synth.config_weight("attn", rows=(0, 2048))
    rec = w12.encode(to_dev(w))
    for m, path in ((1, "gemv"), (32, "mfma")):
        x = to_dev(synth.gen_x(m, spec.k, tensor_id=tid))
        say(f"determinism m={m}")
        a = w12.gemm(x, rec, path=path).cpu().numpy()
        b = w12.gemm(x, rec, path=path).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("n,k,ms,p_zero", [(64, 5120, (1, 3, 8, 16, 32), 0.01),
                                           (320, 17408, (1, 32), 0.001),
                                           (48, 5120, (1, 16, 32), 0.05),
                                           (200, 6144, (2, 20), 0.01)])
def test_gemm_split_k(n, k, ms, p_zero):
    """Shapes with few tiles and long rows run as several k ranges whose partial sums are added by
    a second kernel (k and v projections: 4 tiles of 40 blocks; down projection: 20 tiles of 136
    blocks; 5% zeros put ~4000 escapes in a tile, past the matrix-core kernel's LDS copy, so
    ranges also read escapes from memory)."""
    rng = np.random.default_rng(n + k + len(ms))
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < p_zero] = 0
    w12 = _w12()
    rec = _encode_check(w, f"split {n}x{k}")
    for m in ms:
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        _gemm_case(w, x, f"split {n}x{k}", rec=rec)


def test_gemm_split_k_one_hot_exact():
    """x = e_c on a split shape returns column c of W exactly for columns at the edges of the k
    ranges and for escaped columns, on both kernel families."""
    w12 = _w12()
    n, k = 64, 5120
    rng = np.random.default_rng(3)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[:, 1024] = 0
    w[5, 2047] = 0x4500                       # outlier far above the row's window
    rec = w12.encode(to_dev(w))
    cols = [0, 127, 128, 1023, 1024, 1025, 2047, 2048, 3071, 3072, 4095, 4096, 5119]
    for path, group in (("gemv", 8), ("mfma", len(cols))):
        for i in range(0, len(cols), group):
            cs = cols[i:i + group]
            x = np.zeros((len(cs), k), np.uint16)
            for j, c in enumerate(cs):
                x[j, c] = 0x3F80
            say(f"split one-hot path={path} cols={cs}")
            y = w12.gemm(to_dev(x), rec, path=path).cpu().numpy().astype(np.float64)
            assert np.array_equal(y, oracle.bf16_to_f64(w[:, cs]).T), (path, cs)


@pytest.mark.parametrize("ns,k", [((48, 16, 37), 256), ((16,), 128), ((64, 32, 32, 128), 640)])
def test_concat_rows_equals_encode_of_stacked(ns, k):
    """The record built from the parts' records equals, byte for byte, the encoder's record of the
    stacked matrix; the fused GEMM then matches the oracle."""
    w12 = _w12()
    rng = np.random.default_rng(sum(ns) + k)
    parts = []
    for n in ns:
        w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02 * rng.uniform(0.1, 3)).astype(np.float32))
        w[rng.random((n, k)) < 0.02] = 0
        parts.append(w)
    stacked = np.concatenate(parts, axis=0)
    recs = [w12.encode(to_dev(w)) for w in parts]
    say(f"concat {ns} k={k}")
    fused = w12.concat_rows(recs)
    assert fused.n_esc == sum(r.n_esc for r in recs)
    assert_records_equal(record_numpy(fused), oracle.encode(stacked), f"concat {ns}")
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, k)).astype(np.float32))
    for path in ("gemv", "mfma"):
        y = w12.gemm(to_dev(x), fused, path=path).cpu().numpy()
        check_gemm(y, x, stacked, f"concat gemm {path}")
    # capacity protocol: too few escape slots in `out` -> W12_ERR_CAPACITY with the total reported
    import ctypes
    total = fused.n_esc
    if total > 0:
        small = w12.W12Weight(fused.n, k, torch.empty_like(fused.base), torch.empty_like(fused.ae),
                              torch.empty_like(fused.lo), torch.empty_like(fused.esc_ptr),
                              torch.empty(total, dtype=torch.int32, device="cuda")[:total - 1],
                              torch.empty(total, dtype=torch.int16, device="cuda")[:total - 1])
        arr = (w12._W12Weight * len(recs))(*[r.c_struct() for r in recs])
        n_esc = ctypes.c_uint64(0)
        st = w12.lib().w12_concat_rows(arr, len(recs), ctypes.byref(small.c_struct()), ctypes.byref(n_esc),
                                       torch.cuda.current_stream().cuda_stream)
        assert st == w12.W12_ERR_CAPACITY and n_esc.value == total


@pytest.mark.parametrize("n,k,ms", [(300, 1152, (1, 5, 16)), (4099, 640, (17, 40)), (64, 5120, (16,))])
def test_top1_within_bound(n, k, ms):
    """w12_q8_top1 / w12_gemm_top1 pick, per row of x, an output that is a maximum of the exact
    product within the error bound, and report its value within the bound (ragged last tile,
    passes of 32 rows for m = 40)."""
    w12 = _w12()
    rng = np.random.default_rng(n + k)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    rec = w12.encode(to_dev(w))
    q8w = oracle.q8_view_bits(oracle.encode(w))
    q8m = oracle.q8_view_bits(oracle.encode(w), midpoint=True)
    for m in ms:
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        for fn, ref_w, what in ((w12.q8_top1, q8w, "q8"), (w12.gemm_top1, w, "exact"),
                                (lambda xx, rr: w12.q8_top1(xx, rr, midpoint=True), q8m, "q8 midpoint")):
            say(f"top1 {what} n={n} k={k} m={m}")
            idx, val = (t.cpu().numpy() for t in fn(to_dev(x), rec))
            y64 = oracle.gemm64(x, ref_w)
            bound = 1e-3 * oracle.abs_bound64(x, ref_w)
            rows = np.arange(m)
            assert np.all((idx >= 0) & (idx < n))
            # the chosen output is within the bound of the true maximum, and its value is right
            assert np.all(y64[rows, idx] + bound[rows, idx] >= y64.max(axis=1) - bound.max(axis=1)), what
            assert np.all(np.abs(val - y64[rows, idx]) <= bound[rows, idx]), what


def test_top1_ties_go_to_the_lowest_row():
    """Planted exact ties: with x = e_c every output is one weight, exactly; rows 3, 10 and 200 hold
    the column's largest value (row 100 a larger one in column 300, which the Q pass may or may
    not see, depending on its window), so the top-1 is the lowest row holding the maximum of the
    pass's own weights (oracle views), on both passes."""
    w12 = _w12()
    n, k = 256, 512
    rng = np.random.default_rng(5)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    cols = [0, 77, 300, 511]
    for c in cols:
        w[:, c] = synth.f32_to_bf16_bits(np.full(n, 0.01, np.float32))
        w[[3, 10, 200], c] = 0x3F80                                      # 1.0, three times
    w[100, 300] = 0x3F8F                                                 # 1.1171875
    rec = w12.encode(to_dev(w))
    x = np.zeros((len(cols), k), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80
    q8w = oracle.q8_view_bits(oracle.encode(w))
    for fn, ref in ((w12.q8_top1, q8w), (w12.gemm_top1, w)):
        vals = oracle.bf16_to_f64(ref[:, cols]).T                         # [len(cols), n], exact
        want_idx = np.argmax(vals, axis=1)                                # first maximum
        assert want_idx[0] == 3 and want_idx[1] == 3 and want_idx[3] == 3
        idx, val = (t.cpu().numpy() for t in fn(to_dev(x), rec))
        assert np.array_equal(idx, want_idx), fn.__name__
        assert np.array_equal(val.astype(np.float64), vals[np.arange(len(cols)), want_idx]), fn.__name__
    assert w12.gemm_top1(to_dev(x), rec)[0].cpu().numpy()[2] == 100


@pytest.mark.parametrize("m", [3, 16, 24])
def test_top1_streaming_route(m):
    """On a shape where the automatic path takes the streaming kernel (8192 rows: 2 tiles per CU),
    the top-1 entry points run it too (outputs into the workspace, then a chunked scan): per row
    exactly the first maximum of the automatic path's full outputs and its value, bit for bit, on
    planted exact ties as well, and within the bound of the oracle's maximum."""
    w12 = _w12()
    n, k = 8192, 512
    rng = np.random.default_rng(31 + m)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[[7, 4000, 8191], 5] = 0x4000                     # 2.0 three times: an exact tie for x = e_5
    rec = w12.encode(to_dev(w))
    q8w = oracle.q8_view_bits(oracle.encode(w))
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    x[0] = 0
    x[0, 5] = 0x3F80
    xd = to_dev(x)
    rows = np.arange(m)
    for name, top1, full, ref_w in (("q8", w12.q8_top1, w12.q8_gemm, q8w), ("exact", w12.gemm_top1, w12.gemm, w)):
        say(f"top1 streaming route {name} m={m}")
        y = full(xd, rec).cpu().numpy()
        idx, val = (t.cpu().numpy() for t in top1(xd, rec))
        want = np.argmax(y, axis=1)
        assert np.array_equal(idx, want), name
        assert np.array_equal(val.view(np.uint32), y[rows, want].view(np.uint32)), name
        if name == "exact":
            assert idx[0] == 7
        y64 = oracle.gemm64(x, ref_w)
        bound = 1e-3 * oracle.abs_bound64(x, ref_w)
        assert np.all(y64[rows, idx] + bound[rows, idx] >= y64.max(axis=1) - bound.max(axis=1)), name


def test_top1_streaming_route_row_groups():
    """The streaming top-1 mode on a shape that runs in two row groups (200003 rows: 12501 tiles,
    more than three per wave at 4 rows; ragged last tile): per row exactly the first maximum of
    the automatic path's full outputs and its value, bit for bit, and within the bound of the
    oracle's maximum."""
    w12 = _w12()
    n, k, m = 200003, 128, 4
    rng = np.random.default_rng(77)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[[11, 150000, 200002], 3] = 0x4000                # an exact tie for x = e_3 across the groups
    rec = w12.encode(to_dev(w))
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    x[1] = 0
    x[1, 3] = 0x3F80
    xd = to_dev(x)
    rows = np.arange(m)
    say("top1 streaming route, row groups")
    y = w12.gemm(xd, rec).cpu().numpy()
    idx, val = (t.cpu().numpy() for t in w12.gemm_top1(xd, rec))
    want = np.argmax(y, axis=1)
    assert np.array_equal(idx, want)
    assert np.array_equal(val.view(np.uint32), y[rows, want].view(np.uint32))
    assert idx[1] == 11
    y64 = oracle.gemm64(x, w)
    bound = 1e-3 * oracle.abs_bound64(x, w)
    assert np.all(y64[rows, idx] + bound[rows, idx] >= y64.max(axis=1) - bound.max(axis=1))


def test_graph_capture_replays_match_eager():
    """Split-k GEMMs (workspace), the three kernel families (the streaming kernel with float and
    bfloat16 outputs), the Q pass and the top-1 entry points (the matrix cores' and the streaming
    kernel's top-1 modes) captured in one HIP graph on a fresh stream (its workspace is allocated
    inside the capture):
    every replay, with eager work and cleared outputs in between, equals the eager launches bit
    for bit."""
    w12 = _w12()
    rng = np.random.default_rng(11)
    n, k = 320, 17408                                   # splits at 1 and at 16 rows
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.001] = 0
    rec = w12.encode(to_dev(w))
    x1 = to_dev(synth.f32_to_bf16_bits(rng.standard_normal((1, k)).astype(np.float32)))
    x16 = to_dev(synth.f32_to_bf16_bits(rng.standard_normal((16, k)).astype(np.float32)))
    outs = [torch.empty((1, n), dtype=torch.float32, device="cuda"),
            torch.empty((16, n), dtype=torch.float32, device="cuda"),
            torch.empty((16, n), dtype=torch.float32, device="cuda"),
            torch.empty((16, n), dtype=torch.float32, device="cuda"),
            torch.empty((16, n), dtype=torch.bfloat16, device="cuda")]
    t1 = (torch.empty(16, dtype=torch.int32, device="cuda"), torch.empty(16, dtype=torch.float32, device="cuda"))
    # 400 tiles: the automatic path and the top-1 entry points take the streaming kernel at 16 rows
    n2, k2 = 6400, 256
    w2 = synth.f32_to_bf16_bits((rng.standard_normal((n2, k2)) * 0.02).astype(np.float32))
    w2[rng.random((n2, k2)) < 0.01] = 0
    rec2 = w12.encode(to_dev(w2))
    x16b = to_dev(synth.f32_to_bf16_bits(rng.standard_normal((16, k2)).astype(np.float32)))
    t2 = tuple(torch.empty(16, dtype=d, device="cuda") for d in (torch.int32, torch.float32))
    t3 = tuple(torch.empty(16, dtype=d, device="cuda") for d in (torch.int32, torch.float32))

    def run():
        w12.gemm(x1, rec, path="gemv", out=outs[0])
        w12.gemm(x16, rec, path="mfma", out=outs[1])
        w12.q8_gemm(x16, rec, out=outs[2])
        w12.gemm(x16, rec, path="stream", out=outs[3])
        w12.gemm(x16, rec, path="stream", out=outs[4])
        w12.q8_top1(x16, rec, out=t1)
        w12.q8_top1(x16b, rec2, out=t2)
        w12.gemm_top1(x16b, rec2, out=t3)

    run()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs] + [t.clone() for t in t1 + t2 + t3]
    y2 = w12.gemm(x16b, rec2).cpu().numpy()
    assert np.array_equal(t3[0].cpu().numpy(), np.argmax(y2, axis=1))
    check_gemm(outs[0].cpu().numpy(), to_host_bits(x1), w, "graph eager gemv")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs + list(t1 + t2 + t3):
            o.zero_()
        torch.mm(torch.ones(64, 64, device="cuda"), torch.ones(64, 64, device="cuda"))   # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs + list(t1 + t2 + t3)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, i)


@pytest.mark.parametrize("n,k,ms", [(256, 512, (1, 4, 16, 33)), (64, 5120, (1, 16, 32)), (4099, 640, (2, 17)),
                                    (300, 1152, (8,))])
def test_q8_midpoint_gemm(n, k, ms):
    """w12_q8_gemm with W12_Q8_MIDPOINT against the oracle's midpoint view (in-window weights
    bits & 0xFFF0 | 0x8, escapes exact), both kernel families, split-k and ragged shapes; and
    one-hot exactness (every output is exactly one midpoint weight)."""
    w12 = _w12()
    rng = np.random.default_rng(n * 3 + k)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    rec = w12.encode(to_dev(w))
    qm = oracle.q8_view_bits(oracle.encode(w), midpoint=True)
    for m in ms:
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        for path in ("gemv", "mfma"):
            say(f"q8 midpoint n={n} k={k} m={m} path={path}")
            y = w12.q8_gemm(to_dev(x), rec, path=path, midpoint=True).cpu().numpy()
            check_gemm(y, x, qm, f"q8 midpoint {path}")
    cols = [0, k // 2 + 3, k - 1]
    x = np.zeros((len(cols), k), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80
    for path in ("gemv", "mfma"):
        y = w12.q8_gemm(to_dev(x), rec, path=path, midpoint=True).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, oracle.bf16_to_f64(qm[:, cols]).T), path


@pytest.mark.parametrize("n,k,m", [(4099, 640, 128), (300, 1152, 200), (64, 5120, 100), (16, 128, 65),
                                   (6151, 384, 100), (6151, 384, 200)])
def test_gemm_more_than_64_rows(n, k, m):
    """More than 32 rows of x on the matrix cores: shapes of fewer than 1.5 tiles per CU in passes
    of 32 rows (split k); 385 tiles and more on the eight-tile kernel, 65..128 rows per weight read
    (escapes patched in the epilogue, from LDS and, past its 384 entries in the crowded first
    tile, from memory), passes of 128 above that; every format against the oracle."""
    rng = np.random.default_rng(n + k + m)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[rng.random((n, k)) < 1e-3] = 0x4480                                # outliers far above the window
    if n >= 6144:
        w[:16][rng.random((16, k)) < 0.5] = 0                            # a crowded tile: ~3000 escapes
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    _gemm_case(w, x, f"m>64 {n}x{k}", paths=("mfma",))
    w12 = _w12()
    rec = w12.encode(to_dev(w))
    y = w12.q8_gemm(to_dev(x), rec, midpoint=True).cpu().numpy()
    check_gemm(y, x, oracle.q8_view_bits(oracle.encode(w), midpoint=True), f"m>64 {n}x{k} q8 midpoint")


def test_gemm_more_than_64_rows_one_hot_exact():
    """x = e_c for 100 columns (escaped ones included) through the eight-tile path (385 tiles): every
    output is exactly one weight, on the exact pass and both Q passes."""
    w12 = _w12()
    n, k = 6160, 256
    rng = np.random.default_rng(21)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.02] = 0
    w[5, 17] = 0x4500
    w[9, 200] = 0x0001                                                   # subnormal escape
    rec = w12.encode(to_dev(w))
    ref = oracle.encode(w)
    cols = sorted(set(rng.choice(k, 97, replace=False).tolist()) | {17, 200, 0})[:100]
    x = np.zeros((len(cols), k), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80
    xd = to_dev(x)
    for fn, wv in ((lambda: w12.gemm(xd, rec, path="mfma"), w),
                   (lambda: w12.q8_gemm(xd, rec, path="mfma"), oracle.q8_view_bits(ref)),
                   (lambda: w12.q8_gemm(xd, rec, path="mfma", midpoint=True), oracle.q8_view_bits(ref, midpoint=True))):
        y = fn().cpu().numpy().astype(np.float64)
        assert np.array_equal(y, oracle.bf16_to_f64(wv[:, cols]).T)


def _check_bf16_out(y16, y32, x_bits, w_bits, what):
    """y16 (bfloat16 output) is the float output of the same call rounded to nearest even
    (torch's rounding on the CPU: bit for bit, NaN for NaN); with an oracle weight, also within the
    GEMM bound plus half a bfloat16 unit in the last place."""
    import torch
    want = torch.from_numpy(np.ascontiguousarray(y32)).to(torch.bfloat16)
    got = y16.cpu()
    wn, gn = torch.isnan(want.float()), torch.isnan(got.float())
    assert torch.equal(wn, gn), f"{what}: NaN positions differ"
    assert torch.equal(want.view(torch.int16)[~wn], got.view(torch.int16)[~gn]), \
        f"{what}: bfloat16 output is not the rounded float output"
    if w_bits is None:
        return
    y = got.float().numpy().astype(np.float64)
    y64 = oracle.gemm64(x_bits, w_bits)
    b = 1e-3 * oracle.abs_bound64(x_bits, w_bits)
    fin = np.isfinite(y64)
    err = np.abs(y[fin] - y64[fin])
    # round to nearest with 8 significant bits: relative error at most 2^-8
    assert np.all(err <= b[fin] + 2.0 ** -8 * (np.abs(y64[fin]) + b[fin])), f"{what}: outside the bound"


@pytest.mark.parametrize("n,k,m,path,oracle_check", [
    (300, 1152, 1, "auto", True),          # GEMV
    (300, 1152, 3, "gemv", True),
    (100, 6144, 8, "gemv", True),          # GEMV over two k slices: float sum in the workspace
    (64, 9216, 1, "gemv", True),           # GEMV split k: ordered sum rounds
    (320, 2048, 16, "mfma", True),         # matrix-core split k
    (24593, 256, 20, "mfma", False),       # matrix-core, one k range: the epilogue rounds (n % 4 = 1:
                                           # 2-byte stores)
    (300, 1152, 40, "mfma", True),         # passes of 32 rows (few tiles)
    (6160, 256, 40, "mfma", True),         # three activation tiles (385 tiles)
    (6160, 256, 100, "mfma", True),        # eight activation tiles (385 tiles)
    (50752, 128, 16, "mfma", False),       # full rounds (8-byte stores) + the split tail launch
])
def test_gemm_bf16_output(n, k, m, path, oracle_check):
    """W12_OUT_BF16 on every store site, for the exact pass, both Q-pass views and the baseline."""
    import torch
    w12 = _w12()
    rng = np.random.default_rng(n + 3 * k + m)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[rng.random((n, k)) < 5e-4] = 0x4400
    w[0, 0] = 0x7F80                                                       # +Inf weight: Inf output
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    rec = w12.encode(to_dev(w))
    xd = to_dev(x)
    dw = w12.bf16_tiles(to_dev(w))
    ref = oracle.encode(w) if oracle_check else None
    cases = [("w12", lambda **kw: w12.gemm(xd, rec, path=path, **kw), w),
             ("q8", lambda **kw: w12.q8_gemm(xd, rec, path=path, **kw),
              oracle.q8_view_bits(ref) if oracle_check else None),
             ("q8 midpoint", lambda **kw: w12.q8_gemm(xd, rec, path=path, midpoint=True, **kw),
              oracle.q8_view_bits(ref, midpoint=True) if oracle_check else None),
             ("bf16", lambda **kw: w12.bf16_gemm(xd, dw, path=path, **kw), w)]
    for name, fn, wv in cases:
        what = f"bf16 out {name} {n}x{k} m={m} path={path}"
        say(what)
        y32 = fn().cpu().numpy()
        y16 = fn(out_bf16=True)
        assert y16.dtype == torch.bfloat16 and tuple(y16.shape) == (m, n)
        _check_bf16_out(y16, y32, x, wv if oracle_check else None, what)


def test_gemm_bf16_output_gemv_k_slices():
    """The GEMV with bfloat16 outputs when its x rows need two k slices and the split-k partial
    sums would not fit the workspace (8 rows of x, k = 6144, n = 2^20 + 16: 2 x 8 x n floats >
    64 MiB), so the slices add in float in the workspace before one rounding: bit for bit against
    the rounded float output of the same path."""
    import torch
    w12 = _w12()
    n, k, m = (1 << 20) + 16, 6144, 8
    g = torch.Generator(device="cuda:0").manual_seed(11)
    w = torch.randn((n, k), device="cuda:0", dtype=torch.bfloat16, generator=g).mul_(0.02)   # 12.9 GB
    x = torch.randn((m, k), device="cuda:0", dtype=torch.float32, generator=g).to(torch.bfloat16)
    rec = w12.encode(w)
    del w
    torch.cuda.empty_cache()
    for name, fn in (("w12", lambda **kw: w12.gemm(x, rec, path="gemv", **kw)),
                     ("q8", lambda **kw: w12.q8_gemm(x, rec, path="gemv", **kw))):
        say(f"bf16 out gemv k slices {name} n={n}")
        y32 = fn().cpu().numpy()
        y16 = fn(out_bf16=True)
        _check_bf16_out(y16, y32, None, None, f"gemv k slices {name}")
    del rec
    torch.cuda.empty_cache()


def test_binding_rejects_bad_arguments():
    """The binding checks x and caller-provided outputs before anything is launched: a float or
    wrongly shaped x, an output of the wrong shape, dtype, device or layout raise; a strided x is
    copied contiguous and gives the same result; an x with no rows gives an empty output."""
    import torch
    w12 = _w12()
    rng = np.random.default_rng(5)
    n, k = 64, 256
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = synth.f32_to_bf16_bits(rng.standard_normal((4, k)).astype(np.float32))
    rec = w12.encode(to_dev(w))
    bt = w12.bf16_tiles(to_dev(w))
    xd = to_dev(x)
    calls = (lambda xx, **kw: w12.gemm(xx, rec, **kw), lambda xx, **kw: w12.q8_gemm(xx, rec, **kw),
             lambda xx, **kw: w12.bf16_gemm(xx, bt, **kw))
    dev = xd.device
    for fn in calls:
        with pytest.raises(TypeError):
            fn(xd.float())
        with pytest.raises(ValueError):
            fn(xd[:, :128])                                        # k mismatch
        with pytest.raises(ValueError):
            fn(xd.cpu())                                           # not on the GPU
        with pytest.raises(ValueError):
            fn(xd, out=torch.empty((4, n - 1), dtype=torch.float32, device=dev))
        with pytest.raises(ValueError):
            fn(xd, out=torch.empty((4, n), dtype=torch.float16, device=dev))
        with pytest.raises(ValueError):
            fn(xd, out=torch.empty((n, 4), dtype=torch.float32, device=dev).t())
        with pytest.raises(ValueError):
            fn(xd, out=torch.empty((4, n), dtype=torch.float32))  # host memory
        y = fn(xd)
        wide = torch.zeros((4, 2 * k), dtype=torch.bfloat16, device=dev)
        wide[:, ::2] = xd
        assert torch.equal(fn(wide[:, ::2]), y)                    # strided x: same result
        assert fn(xd[:0]).shape == (0, n)
    for fn in (w12.q8_top1, w12.gemm_top1):
        with pytest.raises(ValueError):
            fn(xd, rec, out=(torch.empty(4, dtype=torch.int64, device=dev),
                             torch.empty(4, dtype=torch.float32, device=dev)))
        with pytest.raises(ValueError):
            fn(xd, rec, out=(torch.empty(4, dtype=torch.int32, device=dev),
                             torch.empty(3, dtype=torch.float32, device=dev)))
        with pytest.raises(ValueError):
            fn(xd[:, :128], rec)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n,k,ms", [
    (300, 1152, (1, 2, 3, 8)),            # 19 tiles: every tile shared by several CUs
    (4000, 1024, (1, 2, 4, 5, 8, 13)),    # 250 tiles; 13 rows: the 16-row instance, rows 13..15 zero
    (20487, 512, (1, 3, 7)),              # 1281 tiles: 5-6 per CU, ragged last tile
    (40000, 128, (1, 6)),                 # 2500 tiles of one block each: 9-10 per CU
    (3000, 5120, (1, 2, 8)),              # 188 tiles of 40 blocks: no tile inside one CU
    (8192, 5120, (9, 13, 16, 21, 32)),    # 16 rows: 4 k phases; 21 and 32 rows: 5 phases of 8 blocks
    (4000, 10240, (16,)),                 # 5 phases of 16 blocks
    (1024, 5120, (1, 17, 32)),            # 64 tiles (a k/v projection): each tile over 4 CUs
    (2000, 2048, (33, 40, 64)),           # 33..64 rows: the 64-row instance, ranges over 3 tiles
    (70003, 256, (1, 4, 16, 32)),         # 4376 tiles: 1 and 32 rows two row groups; 4 and 16
                                          # rows one group, up to three tiles finalised per wave
])
def test_stream_path(n, k, ms):
    """The streaming kernel (W12_PATH_STREAM) on every format, 1..64 rows per pass (x staged in
    k phases when it does not fit the LDS whole; a tile's blocks shared by several waves of its CU,
    their sums added in wave order; shapes with more tiles than waves on the chip in row groups),
    against the oracle; bfloat16 outputs the rounding of the float outputs; a second call gives the
    same bits."""
    import torch
    w12 = _w12()
    rng = np.random.default_rng(n + k)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[rng.random((n, k)) < 3e-4] = 0x4400
    x = synth.f32_to_bf16_bits(rng.standard_normal((max(ms), k)).astype(np.float32))
    rec = w12.encode(to_dev(w))
    ref = oracle.encode(w)
    cp = w12.i8_build(rec)
    wq8, wq8m = oracle.q8_view_bits(ref), oracle.q8_view_bits(ref, midpoint=True)
    wi8 = oracle.i8_weights64(ref, oracle.i8_copy(ref))
    dw = w12.bf16_tiles(to_dev(w))
    for m in ms:
        xd = to_dev(x[:m])
        for name, fn, wv in (("w12", lambda **kw: w12.gemm(xd, rec, path="stream", **kw), w),
                             ("q8", lambda **kw: w12.q8_gemm(xd, rec, path="stream", **kw), wq8),
                             ("q8m", lambda **kw: w12.q8_gemm(xd, rec, path="stream", midpoint=True, **kw), wq8m),
                             ("bf16", lambda **kw: w12.bf16_gemm(xd, dw, path="stream", **kw), w),
                             ("i8", lambda **kw: w12.i8_gemm(xd, cp, path="stream", **kw), None)):
            what = f"stream {name} {n}x{k} m={m}"
            say(what)
            y = fn().cpu().numpy()
            if wv is None:
                from tests.gpu_util import check_y
                check_y(y, oracle.gemm64_f(x[:m], wi8), oracle.abs_bound64_f(x[:m], wi8), what)
            else:
                check_gemm(y, x[:m], wv, what)
            if m in (1, 3, 32):
                y16 = fn(out_bf16=True)
                _check_bf16_out(y16, y, x[:m], None, what + " bf16")
            if name == "w12":
                assert np.array_equal(fn().cpu().numpy().view(np.uint32), y.view(np.uint32)), \
                    f"{what}: a second call differs"


@pytest.mark.parametrize("n,k,ms", [
    (197000, 128, (4, 16)),               # 12313 tiles: two row groups of up to 3 tiles per wave
    (66000, 2816, (8, 16)),               # 4125 tiles; 16 rows: two k phases of 11 blocks
    (40000, 640, (40, 64)),               # 2500 tiles, 64-row instance: up to 2 tiles per wave
    (70000, 128, (33,)),                  # 4375 tiles: two row groups of up to 2 tiles per wave
    (100000, 128, (24,)),                 # 6250 tiles at 24 rows: two row groups of up to 2 tiles
])
def test_stream_several_tiles_per_wave(n, k, ms):
    """The streaming kernel on shapes with more tiles than waves on the chip (3..16 rows: up to
    three tiles finalised per wave; 17..64 rows: up to two), every wave walking the escapes of all
    its tiles phase by phase: W12 and the dense baseline against the oracle product (the plain
    definition), bfloat16 outputs the rounding of the float outputs, a second call the same bits."""
    w12 = _w12()
    rng = np.random.default_rng(n + k)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.01] = 0
    w[rng.random((n, k)) < 3e-4] = 0x4400
    x = synth.f32_to_bf16_bits(rng.standard_normal((max(ms), k)).astype(np.float32))
    wd = to_dev(w)
    rec = w12.encode(wd)
    dw = w12.bf16_tiles(wd)
    del wd
    for m in ms:
        xd = to_dev(x[:m])
        for name, fn in (("w12", lambda **kw: w12.gemm(xd, rec, path="stream", **kw)),
                         ("bf16", lambda **kw: w12.bf16_gemm(xd, dw, path="stream", **kw))):
            what = f"stream {name} {n}x{k} m={m}"
            say(what)
            y = fn().cpu().numpy()
            check_gemm(y, x[:m], w, what)
            _check_bf16_out(fn(out_bf16=True), y, x[:m], None, what + " bf16")
            assert np.array_equal(fn().cpu().numpy().view(np.uint32), y.view(np.uint32)), \
                f"{what}: a second call differs"


def test_stream_one_hot_and_special_values():
    """One-hot x returns every weight exactly through the streaming kernel (escapes included), and
    Inf / NaN weights give Inf / NaN outputs."""
    w12 = _w12()
    rng = np.random.default_rng(8)
    n, k = 2048, 384
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 0.02] = 0
    w[5, 100] = 0x4700                     # far outside the window: an escape
    rec = w12.encode(to_dev(w))
    for kk in (0, 100, 127, 128, 255, 383):
        x = np.zeros((3, k), dtype=np.uint16)
        x[:, kk] = 0x3F80
        y = w12.gemm(to_dev(x), rec, path="stream").cpu().numpy().astype(np.float64)
        assert np.array_equal(y[0], oracle.bf16_to_f64(w[:, kk])), kk
        assert np.array_equal(y[2], y[0])
    w2 = w.copy()
    w2[7, 9] = 0x7F80
    w2[8, 9] = 0x7FC0
    rec2 = w12.encode(to_dev(w2))
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, k)).astype(np.float32))
    y = w12.gemm(to_dev(x), rec2, path="stream").cpu().numpy()
    assert np.all(np.isinf(y[:, 7])) and np.all(np.isnan(y[:, 8]))
    check_gemm(np.delete(y, [7, 8], axis=1), x, np.delete(w2, [7, 8], axis=0), "stream special")


def test_release_workspace_on_a_side_stream():
    """w12_release_workspace: a split-k GEMM on a stream of its own (W [1024, 2048] at 32 rows
    splits k, so its partial sums use that stream's workspace) is right before and after the
    stream's workspace is freed (the next call allocates a new one); releasing a stream that has
    none, or twice, is a no-op."""
    w12 = _w12()
    rng = np.random.default_rng(77)
    w = synth.f32_to_bf16_bits((rng.standard_normal((1024, 2048)) * 0.02).astype(np.float32))
    w[rng.random(w.shape) < 0.01] = 0
    x = synth.f32_to_bf16_bits(rng.standard_normal((32, 2048)).astype(np.float32))
    rec = w12.encode(to_dev(w))
    xd = to_dev(x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(2):
        with torch.cuda.stream(side):
            say(f"side-stream split GEMM, call {rep}")
            y = w12.gemm(xd, rec, path="mfma")
        side.synchronize()
        check_gemm(y.cpu().numpy(), x, w, f"side stream call {rep}")
        w12.release_workspace(side)
        w12.release_workspace(side)
    fresh = torch.cuda.Stream()
    w12.release_workspace(fresh)
    torch.cuda.synchronize()
