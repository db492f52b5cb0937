"""CPU checks of the seeded input generators (no W12 arithmetic involved)."""
import numpy as np
import pytest

from lossless_bit_weight_02_amd import synth

torch = pytest.importorskip("torch")


def test_torch_bf16_rounding_matches_numpy_rne():
    """torch's float32 -> bfloat16 cast and synth.f32_to_bf16_bits round alike (nearest, ties to
    even), on random values and on exact halfway cases."""
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(1 << 16) * 10.0 ** rng.uniform(-6, 3, 1 << 16)).astype(np.float32)
    halfway = ((rng.integers(0, 0x7F00, 4096, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    for v in (a, halfway):
        want = synth.f32_to_bf16_bits(v)
        got = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want)


def test_gen_weight_torch_distribution_and_determinism():
    spec = synth.WeightSpec(n=512, k=1024, p_out=2e-3, out_pow=6, p_zero=1e-2)
    w = synth.gen_weight_torch(spec, 0, 5)
    assert w.dtype == torch.bfloat16 and tuple(w.shape) == (512, 1024)
    again = synth.gen_weight_torch(spec, 0, 5)
    assert torch.equal(w.view(torch.int16), again.view(torch.int16))
    other = synth.gen_weight_torch(spec, 0, 6)
    assert not torch.equal(w.view(torch.int16), other.view(torch.int16))
    f = w.float()
    zero_frac = float((f == 0).float().mean())
    assert 0.008 < zero_frac < 0.012
    # per-row spread (robust to the outliers): median |w| / 0.6745 estimates s_n, whose median
    # over rows is 0.02
    sd = f.abs().median(dim=1).values / 0.6745
    assert 0.015 < float(sd.median()) < 0.026
    # outliers: 2^6 times the row scale shows up in about p_out of the entries
    big = (f.abs() > 8 * sd[:, None]).float().mean()
    assert 1e-3 < float(big) < 3e-3


def test_gen_weight_torch_loguniform():
    spec = synth.WeightSpec(n=256, k=512, scale="loguniform", s_lo=1e-3, s_hi=1e-1,
                            p_out=1e-4, out_pow=8, p_zero=0.01)
    f = synth.gen_weight_torch(spec, 0, 1000).float()
    sd = f.abs().median(dim=1).values / 0.6745
    assert float(sd.min()) > 7e-4 and float(sd.max()) < 0.13
