"""The allocation-free entry point w12_gemm_noalloc against w12_gemm.

w12_gemm_noalloc runs the same kernels as w12_gemm with the library's fixed per-GPU scratch in
place of the per-stream workspace, so on every shape whose scratch use fits the fixed size the two
must give bit-identical outputs.  Calls come in a row on one record, each next one with fewer rows
of x, so a call that read what the previous one left in the scratch would show.  Cases: the
eight-tile pass (100 rows: x transposed into the scratch), the split-k matrix-core pass (32 rows
on W [1024, 5120] and [5120, 17408]: partial sums in the scratch), the split-k GEMV (1 row on
[5120, 17408]), a GEMV with no scratch and the streaming kernel (32, 16 and 4 rows on
[8192, 5120]); float and bfloat16 outputs; plus the oracle bound on
one case and the up-front refusal of a call that cannot fit.
"""
import numpy as np
import pytest

import oracle
from lossless_bit_weight_02_amd import synth
from tests.gpu_util import check_gemm, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_weight_02_amd import w12
    w12.lib()


def _weight(n, k, seed):
    rng = np.random.default_rng(seed)
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w[rng.random((n, k)) < 1e-3] = 0                      # escapes (zeros)
    w[rng.random((n, k)) < 1e-4] = 0x4400                 # escapes (outliers)
    return w


@pytest.mark.parametrize("n,k,ms,seed", [
    (1024, 5120, (100, 32, 1), 1),        # eight-tile pass, split-k matrix cores, GEMV
    (5120, 17408, (32, 1), 2),            # split-k matrix cores, split-k GEMV
    (8192, 5120, (32, 16, 4), 3),         # the streaming kernel (no scratch)
])
def test_noalloc_matches_gemm(n, k, ms, seed):
    from lossless_bit_weight_02_amd import w12
    w = _weight(n, k, seed)
    x = synth.gen_x(max(ms), k, tensor_id=seed)
    rec = w12.encode(to_dev(w))
    for out_dtype in (torch.float32, torch.bfloat16):
        for m in ms:
            what = f"noalloc {n}x{k} m={m} {out_dtype}"
            say(what)
            xd = to_dev(x[:m])
            want = w12.gemm(xd, rec, out_bf16=out_dtype == torch.bfloat16)
            got = torch.full((m, n), float("nan"), dtype=out_dtype, device=xd.device)
            w12.gemm_noalloc(xd, rec, got)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                               want.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)), what
    say(f"noalloc {n}x{k} oracle bound m={ms[-1]}")
    xd = to_dev(x[:ms[0]])
    got = torch.empty((ms[0], n), dtype=torch.float32, device=xd.device)
    w12.gemm_noalloc(xd, rec, got)
    check_gemm(got.cpu().numpy(), x[:ms[0]], w, f"noalloc {n}x{k} m={ms[0]}")


def test_noalloc_refuses_what_does_not_fit():
    """bfloat16 outputs of 8 rows on the GEMV path over two k slices need 8 x n floats of scratch;
    with n = 2^19 + 16 that is more than the fixed 16 MiB, so the call is refused before anything
    runs (the record is zero-filled, so even a wrong launch would read only valid memory)."""
    from lossless_bit_weight_02_amd import w12
    n, k, m = (1 << 19) + 16, 6144, 8
    dev = torch.device("cuda:0")
    npad = w12.padded_rows(n)
    rec = w12.W12Weight(n, k, torch.ones(n, dtype=torch.uint8, device=dev),
                        torch.zeros(npad * k, dtype=torch.uint8, device=dev),
                        torch.zeros(npad * k // 2, dtype=torch.uint8, device=dev),
                        torch.zeros(n + 1, dtype=torch.int32, device=dev),
                        torch.zeros(1, dtype=torch.int32, device=dev)[:0],
                        torch.zeros(1, dtype=torch.int16, device=dev)[:0])
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=dev)
    y = torch.zeros((m, n), dtype=torch.bfloat16, device=dev)
    say("noalloc refusal")
    with pytest.raises(w12.W12Error) as ei:
        w12.gemm_noalloc(x, rec, y, path="gemv")
    assert ei.value.status == w12.W12_ERR_RANGE
    assert b"scratch" in w12.lib().w12_last_error()
    # the same call with float outputs needs no scratch and runs
    yf = torch.full((m, n), 1.0, dtype=torch.float32, device=dev)
    w12.gemm_noalloc(x, rec, yf, path="gemv")
    torch.cuda.synchronize()
    assert torch.count_nonzero(yf).item() == 0
    del rec, x, y, yf
    torch.cuda.empty_cache()
