"""Seeded synthetic inputs for the W12 hot path.

This module is shared by the HIP path's callers (tests, bench) and by the
oracle's callers.  It holds none of the W12 method's arithmetic: it draws
random numbers and rounds float32 to bfloat16, nothing else.

Stand-in for trained weights.  The SpecPilot pages measure W12 on trained
checkpoints (Qwen3.8-27B and other dense models; SpecPilot summary page,
"Main Findings", W12 compression bullet).  None is available here, so every
weight is drawn from the distribution below, with the projection shapes of a
27B-class dense model:

* each output row n has a scale s_n;
* w[n, k] = float32(z * s_n) with z ~ N(0, 1) drawn in float32;
* with probability p_out an entry is multiplied by 2**out_pow (outliers);
* with probability p_zero an entry is set to exactly 0 (applied last);
* the float32 value is rounded to bfloat16 with round-to-nearest-even.

Rows are generated in chunks of ``CHUNK`` rows.  Chunk c of tensor t under
seed S uses ``numpy.random.default_rng([S, t, c])`` and draws, in order:
the per-row scale randomness, z [rows, K] float32, u_out [rows, K] float32,
u_zero [rows, K] float32.  The activations x [M, K] of tensor t use
``default_rng([S, t, X_STREAM])``: N(0, 1) float32 rounded to bfloat16.  The
first rows of a larger M are the rows of a smaller one.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096
X_STREAM = 0x5EED_0001
DEVICE_STREAM = 0x5EED_0002


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw u16 bits.

    Inputs here are finite; NaN is not expected and not special-cased.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class WeightSpec:
    """Distribution and shape of one synthetic weight tensor W [n, k]."""
    n: int
    k: int
    scale: str = "lognormal"      # "lognormal" or "loguniform"
    median: float = 0.02           # lognormal: s_n = median * exp(sigma * N(0,1))
    sigma: float = 0.5
    s_lo: float = 1e-3             # loguniform: s_n = 10 ** U(log10 s_lo, log10 s_hi)
    s_hi: float = 1e-1
    p_out: float = 7.3e-5
    out_pow: int = 6
    p_zero: float = 1e-3


@dataclass(frozen=True)
class Config:
    name: str
    weights: tuple            # tuple of (tensor_id, label, WeightSpec)
    ms: tuple                 # activation row counts used with this config
    ops: tuple = ()
    note: str = ""


def _tiny_spec():
    return WeightSpec(n=256, k=512, scale="loguniform", s_lo=1e-3, s_hi=1e-1,
                      p_out=1e-4, out_pow=8, p_zero=0.01)


def _proj(n, k):
    return WeightSpec(n=n, k=k)


# tensor ids: single-tensor configs use 1000 + index; the stack uses 8*layer + proj.
STACK_PROJ = (("q", 6144, 5120), ("k", 1024, 5120), ("v", 1024, 5120),
              ("o", 5120, 6144), ("gate", 17408, 5120), ("up", 17408, 5120),
              ("down", 5120, 17408))
STACK_LAYERS = 64

CONFIGS = {
    "tiny": Config("tiny", ((1000, "W", _tiny_spec()),), (1,), ("encode", "decode", "gemv")),
    "attn": Config("attn", ((1001, "W", _proj(5120, 5120)),), (1,), ("encode", "decode", "gemm")),
    "gate_up": Config("gate_up", ((1002, "W", _proj(34816, 5120)),), (1, 4, 8, 16, 32, 64),
                      ("gemm_both_paths",), "gate rows then up rows, one matrix"),
    "lm_head": Config("lm_head", ((1003, "W", _proj(152064, 5120)),), (16,), ("q8", "gemm", "top1")),
    "stack": Config("stack", tuple((8 * l + p, f"layer{l}.{nm}", _proj(n, k))
                                   for l in range(STACK_LAYERS)
                                   for p, (nm, n, k) in enumerate(STACK_PROJ)),
                    (1, 32), ("encode_all", "gemm_sweep")),
}


def _chunk(spec: WeightSpec, seed: int, tensor_id: int, c: int) -> np.ndarray:
    r0 = c * CHUNK
    rows = min(CHUNK, spec.n - r0)
    rng = np.random.default_rng([seed, tensor_id, c])
    if spec.scale == "lognormal":
        s = spec.median * np.exp(spec.sigma * rng.standard_normal(rows))
    elif spec.scale == "loguniform":
        s = 10.0 ** rng.uniform(np.log10(spec.s_lo), np.log10(spec.s_hi), rows)
    else:
        raise ValueError(spec.scale)
    z = rng.standard_normal((rows, spec.k), dtype=np.float32)
    u_out = rng.random((rows, spec.k), dtype=np.float32)
    u_zero = rng.random((rows, spec.k), dtype=np.float32)
    w = z * s.astype(np.float32)[:, None]
    w[u_out < np.float32(spec.p_out)] *= np.float32(2.0 ** spec.out_pow)
    w[u_zero < np.float32(spec.p_zero)] = np.float32(0.0)
    return f32_to_bf16_bits(w)


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_weight(spec: WeightSpec, seed: int = 0, tensor_id: int = 0,
               rows: tuple | None = None, threads: int | None = None) -> np.ndarray:
    """bfloat16 bits of W [n, k] (or of rows [r0, r1) when ``rows`` is given)."""
    r0, r1 = (0, spec.n) if rows is None else rows
    if not (0 <= r0 <= r1 <= spec.n):
        raise ValueError("row range out of bounds")
    out = np.empty((r1 - r0, spec.k), dtype=np.uint16)
    c0, c1 = r0 // CHUNK, (r1 + CHUNK - 1) // CHUNK

    def work(c):
        blk = _chunk(spec, seed, tensor_id, c)
        a, b = max(r0, c * CHUNK), min(r1, c * CHUNK + blk.shape[0])
        out[a - r0:b - r0] = blk[a - c * CHUNK:b - c * CHUNK]

    n_thr = threads or _threads()
    if c1 - c0 <= 1 or n_thr == 1:
        for c in range(c0, c1):
            work(c)
    else:
        with ThreadPoolExecutor(max_workers=n_thr) as ex:
            list(ex.map(work, range(c0, c1)))
    return out


def gen_x(m: int, k: int, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    """bfloat16 bits of activations x [m, k], N(0,1)."""
    rng = np.random.default_rng([seed, tensor_id, X_STREAM])
    z = rng.standard_normal((m, k), dtype=np.float32)
    return f32_to_bf16_bits(z)


def config_weight(name: str, seed: int = 0, index: int = 0, rows=None):
    cfg = CONFIGS[name]
    tid, label, spec = cfg.weights[index]
    return gen_weight(spec, seed, tid, rows), spec, tid


def device_seed(seed: int, tensor_id: int) -> int:
    """63-bit seed of tensor ``tensor_id`` for torch's generator (from numpy's SeedSequence)."""
    st = np.random.SeedSequence([seed, tensor_id, DEVICE_STREAM]).generate_state(1, np.uint64)[0]
    return int(st) & ((1 << 63) - 1)


def gen_weight_torch(spec: WeightSpec, seed: int = 0, tensor_id: int = 0, device="cpu"):
    """W [n, k] as a torch bfloat16 tensor, drawn on ``device`` with torch's own generator.

    Same distribution and steps as ``gen_weight`` (per-row scale, z ~ N(0,1) float32, outliers
    multiplied by 2**out_pow, zeros last, round to nearest even), but a different random stream:
    torch's generator seeded with ``device_seed(seed, tensor_id)``.  It serves workloads too large
    to draw on the host in reasonable time (the 64-layer stack holds 2.18e10 weights).
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(device_seed(seed, tensor_id))
    n, k = spec.n, spec.k
    if spec.scale == "lognormal":
        s = spec.median * torch.exp(spec.sigma * torch.randn(n, generator=g, device=device,
                                                             dtype=torch.float64))
    elif spec.scale == "loguniform":
        lo, hi = np.log10(spec.s_lo), np.log10(spec.s_hi)
        s = 10.0 ** (lo + (hi - lo) * torch.rand(n, generator=g, device=device, dtype=torch.float64))
    else:
        raise ValueError(spec.scale)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    w *= s.to(torch.float32)[:, None]
    u = torch.rand((n, k), generator=g, device=device, dtype=torch.float32)
    w[u < spec.p_out] *= float(2.0 ** spec.out_pow)
    torch.rand((n, k), generator=g, device=device, dtype=torch.float32, out=u)
    w[u < spec.p_zero] = 0.0
    del u
    return w.to(torch.bfloat16)
