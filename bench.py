#!/usr/bin/env python3
"""Benchmark of the W12 hot path on one MI355X.

Metric: W12 GEMM effective HBM GB/s (algorithmic bytes / kernel time) at M=1 and M=32, and the
speedup over the same-build BF16 kernel.  Workload: the fused MLP gate+up projection of a
27B-class dense model, W bf16 [34816, 5120] (synthetic weights, see
lossless_bit_weight_02_amd/synth.py), activations x bf16 [M, 5120].

One step = one pass of the whole path over one batch of R weight matrices (R copies of the
gate+up weight, >= 1.1 GB per format, so every launch streams from HBM and not from the 256 MB
Infinity Cache):
  encode x R (window choice + plane packing + escape CSR, one host sync each) -> decode x R ->
  cached read of 512 MiB (writes back the dirty lines the encoder and decoder left in the
  caches; the streaming kernels' non-temporal loads do not, and a GEMM launched right after the
  decoder pays several microseconds for that write-back) -> read probe over 2 GiB (measured
  ceiling) -> exact W12 GEMM M=1 (GEMV) x 2R -> exact W12 GEMM M=32 x R -> Q-pass GEMM on the
  8-bit view M=16 x R -> same-build BF16 GEMM M=1 x 2R and M=32 x R (M = 16 and 32 on the
  automatic path: the streaming kernel for W12 and Q8, the matrix cores for BF16).
Each op's back-to-back launches are bracketed by one pair of HIP events on the stream they run
on; the per-launch time is the elapsed time / launches (the M=1 groups launch every copy twice,
so the gap around an event pair weighs less).

Beside the step (context, outside `value` and `ms_per_step`): an M sweep on gate+up (GEMV, MFMA and
streaming families, W12 and BF16, W12 with bfloat16 outputs at M = 1, 32, 128) and the vendor library's
bf16 GEMM; the attention projection [5120, 5120]
at M=1; the LM-head-like [152064, 5120] Q pass at M=16 (truncated and midpoint views, exact pass,
top-1 entry points, BF16, top-1 agreement); and the 64-layer 27B-class stack at M=1 and M=32,
per projection and in the qkv / gate_up layout.  These are timed as captured HIP graphs whose
replays are checked bit for bit against eager launches; their outputs are sampled into the CPU
oracle leg.

Prints one JSON line.  `--gpus N` with N > 1 exits: the kernels here run on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor peak
MFMA_BF16_PEAK_TFS = 2500.0      # dense bf16
K_HIDDEN = 5120
N_GATE_UP = 34816
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w12_gemv_m1_gate_up_traffic.md")
KERNEL_SOURCES = ["lossless_bit_weight_02_amd/csrc/gemv.hip", "lossless_bit_weight_02_amd/csrc/block.hpp",
                  "lossless_bit_weight_02_amd/csrc/w12_device.hpp"]


def w12_bytes(n, k, n_esc, m):
    """Algorithmic bytes of one exact W12 GEMM: planes, base, esc_ptr, escapes, x and y."""
    return n * k * 1.5 + n + 4 * (n + 1) + 6 * n_esc + 2 * m * k + 4 * m * n


def q8_bytes(n, k, n_esc, m):
    return n * k * 1.0 + n + 4 * (n + 1) + 6 * n_esc + 2 * m * k + 4 * m * n


def bf16_bytes(n, k, m):
    return n * k * 2.0 + 2 * m * k + 4 * m * n


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the M=1 W12 GEMV from the committed rocprofv3 --pmc summary, or
    None if there is none or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def time_eager(fns, stream, reps):
    """Mean seconds per pass over the launch list `fns`, launched one by one from Python (host
    launch overhead included), timed with HIP events on `stream`."""
    import torch
    for f in fns:
        f()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(reps):
        for f in fns:
            f()
    eb.record(stream)
    torch.cuda.synchronize()
    return ea.elapsed_time(eb) * 1e-3 / reps


def capture_graph(fns, outs):
    """Capture the launch list in one HIP graph and check its replays against the eager result:
    every output is cleared, the graph replayed, and the output compared bit for bit, three
    times, with eager work in between.  Returns the graph."""
    import torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            if not torch.equal(o.view(torch.int32), w.view(torch.int32)):
                raise SystemExit("graph replay differs from the eager launches")
    return g


def time_graph(g, stream, reps):
    """Mean seconds per replay of a captured HIP graph (HIP events on `stream`)."""
    import torch
    g.replay()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(reps):
        g.replay()
    eb.record(stream)
    torch.cuda.synchronize()
    return ea.elapsed_time(eb) * 1e-3 / reps


def to_dev_bits(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def attn_bench(dev, stream, min_rot_bytes, reps):
    """Attention projection W [5120, 5120] at M=1: W12 GEMV and the same-build BF16 GEMV over R
    copies (>= min_rot_bytes per format, so every launch reads HBM), launched one by one and as
    one captured HIP graph.  At ~5 us per launch the host's launch rate, not the kernel, sets the
    eager time, so the graph figure is the kernel's.  Returns (results, parity samples)."""
    import torch
    from lossless_bit_weight_02_amd import synth, w12

    w_bits, spec, tid = synth.config_weight("attn")
    n, k = spec.n, spec.k
    x_bits = synth.gen_x(1, k, tensor_id=tid)
    w = to_dev_bits(w_bits, dev)
    rec = w12.encode(w)
    rot = max(2, int(np.ceil(min_rot_bytes / rec.nbytes())))
    recs = [rec] + [rec.clone() for _ in range(rot - 1)]
    tiles = [w12.bf16_tiles(w)]
    tiles += [w12.Bf16Tiles(n, k, tiles[0].data.clone()) for _ in range(rot - 1)]
    del w
    x = to_dev_bits(x_bits, dev)
    y = [torch.empty((1, n), dtype=torch.float32, device=dev) for _ in range(rot)]
    yb = [torch.empty((1, n), dtype=torch.float32, device=dev) for _ in range(rot)]
    w12_fns = [lambda r=r: w12.gemm(x, recs[r], path="gemv", out=y[r]) for r in range(rot)]
    bf_fns = [lambda r=r: w12.bf16_gemm(x, tiles[r], path="gemv", out=yb[r]) for r in range(rot)]
    out = {"n": n, "k": k, "m": 1, "rotation_copies": rot, "escapes": rec.n_esc}
    b_w12, b_bf = w12_bytes(n, k, rec.n_esc, 1), bf16_bytes(n, k, 1)
    for name, fns, outs, byt in (("w12", w12_fns, y, b_w12), ("bf16", bf_fns, yb, b_bf)):
        t_e = time_eager(fns, stream, reps) / rot
        g = capture_graph(fns, outs)
        t_g = time_graph(g, stream, reps) / rot
        out[f"{name}_us_graph"] = round(t_g * 1e6, 3)
        out[f"{name}_gbs_graph"] = round(byt / t_g / 1e9, 1)
        out[f"{name}_us_eager"] = round(t_e * 1e6, 3)
        del g
    out["w12_frac_hbm_graph"] = round(b_w12 / (out["w12_us_graph"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    out["speedup_vs_bf16_graph"] = round(out["bf16_us_graph"] / out["w12_us_graph"], 4)
    samples = [("attn w12 m=1", x_bits, w_bits, y[0].cpu().numpy())]
    return out, samples


def lm_head_bench(dev, stream, reps):
    """LM-head-like W [152064, 5120] at M=16: the Q pass on the 8-bit view (truncated and midpoint)
    and on the separate 8-bit copy, and the exact pass, as full outputs (automatic path, and the
    matrix-core path that the top-1 entry points run) and as top-1 per row (no logits written),
    and the same-build BF16 kernel; each timed as a captured HIP graph of
    back-to-back launches (the 1.17 GB record streams from HBM on every launch).  Reports each Q
    pass's top-1 agreement with the exact pass on these inputs and over 1024 rows of x.
    Weights drawn on the GPU (synth.gen_weight_torch)."""
    import torch
    from lossless_bit_weight_02_amd import synth, w12

    tid, _, spec = synth.CONFIGS["lm_head"].weights[0]
    n, k, m = spec.n, spec.k, 16
    w = synth.gen_weight_torch(spec, 0, tid, dev)
    rec = w12.encode(w)
    tiles = w12.bf16_tiles(w)
    keep = w[:128].view(torch.int16).cpu().numpy().view(np.uint16)
    del w
    # the separate 8-bit copy (one more byte per weight of memory), built on the device
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    cp = w12.i8_build(rec)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_build = ev0.elapsed_time(ev1) * 1e-3
    x_bits = synth.gen_x(m, k, tensor_id=tid)
    x = to_dev_bits(x_bits, dev)
    yq = torch.empty((m, n), dtype=torch.float32, device=dev)
    ye = torch.empty_like(yq)
    yb = torch.empty_like(yq)
    ym = torch.empty_like(yq)
    yq_mf = torch.empty_like(yq)
    ye_mf = torch.empty_like(yq)
    ym_mf = torch.empty_like(yq)
    tq = (torch.empty(m, dtype=torch.int32, device=dev), torch.empty(m, dtype=torch.float32, device=dev))
    te = (torch.empty(m, dtype=torch.int32, device=dev), torch.empty(m, dtype=torch.float32, device=dev))
    tm = (torch.empty(m, dtype=torch.int32, device=dev), torch.empty(m, dtype=torch.float32, device=dev))
    yi = torch.empty_like(yq)
    ti = (torch.empty(m, dtype=torch.int32, device=dev), torch.empty(m, dtype=torch.float32, device=dev))
    i8_byt = n * k + 4 * n + 4 * (n + 1) + 6 * rec.n_esc + 2 * m * k + 4 * m * n
    cases = (("q8_m16", lambda: w12.q8_gemm(x, rec, out=yq), [yq], q8_bytes(n, k, rec.n_esc, m)),
             ("q8_midpoint_m16", lambda: w12.q8_gemm(x, rec, out=ym, midpoint=True), [ym],
              q8_bytes(n, k, rec.n_esc, m)),
             ("w12_m16", lambda: w12.gemm(x, rec, out=ye), [ye], w12_bytes(n, k, rec.n_esc, m)),
             # the matrix-core path, for comparison (the automatic path and the top-1 entry
             # points run the streaming kernel at this size)
             ("q8_m16_mfma", lambda: w12.q8_gemm(x, rec, out=yq_mf, path="mfma"), [yq_mf],
              q8_bytes(n, k, rec.n_esc, m)),
             ("q8_midpoint_m16_mfma", lambda: w12.q8_gemm(x, rec, out=ym_mf, midpoint=True, path="mfma"), [ym_mf],
              q8_bytes(n, k, rec.n_esc, m)),
             ("w12_m16_mfma", lambda: w12.gemm(x, rec, out=ye_mf, path="mfma"), [ye_mf],
              w12_bytes(n, k, rec.n_esc, m)),
             ("q8_top1_m16", lambda: w12.q8_top1(x, rec, out=tq), list(tq),
              q8_bytes(n, k, rec.n_esc, m) - 4 * m * n + 8 * m),
             ("q8_midpoint_top1_m16", lambda: w12.q8_top1(x, rec, out=tm, midpoint=True), list(tm),
              q8_bytes(n, k, rec.n_esc, m) - 4 * m * n + 8 * m),
             ("w12_top1_m16", lambda: w12.gemm_top1(x, rec, out=te), list(te),
              w12_bytes(n, k, rec.n_esc, m) - 4 * m * n + 8 * m),
             ("i8_copy_m16", lambda: w12.i8_gemm(x, cp, out=yi), [yi], i8_byt),
             ("i8_copy_top1_m16", lambda: w12.i8_top1(x, cp, out=ti), list(ti), i8_byt - 4 * m * n + 8 * m),
             ("bf16_m16", lambda: w12.bf16_gemm(x, tiles, out=yb), [yb], bf16_bytes(n, k, m)))
    out = {"n": n, "k": k, "m": m, "escapes": rec.n_esc, "launches_per_graph": 8,
           "i8_copy_bytes": cp.nbytes(), "i8_copy_build_us": round(t_build * 1e6, 1)}
    for i, (name, fn, outs, byt) in enumerate(cases):
        g = capture_graph([fn] * 8, outs)
        if i == 0:
            time_graph(g, stream, 4 * reps)   # warm-up: the first timed graph ran ~3% slow
        t = time_graph(g, stream, reps) / 8
        del g
        out[f"{name}_us"] = round(t * 1e6, 2)
        out[f"{name}_gbs"] = round(byt / t / 1e9, 1)
    out["q8_frac_hbm"] = round(out["q8_m16_gbs"] / HBM_PEAK_GBS, 4)
    out["w12_frac_hbm"] = round(out["w12_m16_gbs"] / HBM_PEAK_GBS, 4)
    out["i8_copy_frac_hbm"] = round(out["i8_copy_m16_gbs"] / HBM_PEAK_GBS, 4)
    out["q8_speedup_vs_bf16"] = round(out["bf16_m16_us"] / out["q8_m16_us"], 4)
    out["i8_copy_speedup_vs_bf16"] = round(out["bf16_m16_us"] / out["i8_copy_m16_us"], 4)
    out["w12_speedup_vs_bf16"] = round(out["bf16_m16_us"] / out["w12_m16_us"], 4)
    iq, ie = tq[0].cpu().numpy(), te[0].cpu().numpy()
    out["top1_agreement_q8_vs_exact"] = f"{int((iq == ie).sum())}/{m}"
    im = ym.argmax(dim=1).cpu().numpy()
    out["top1_agreement_q8_midpoint_vs_exact"] = f"{int((im == ie).sum())}/{m}"
    scale = float(ye.abs().mean())
    out["q8_mean_abs_err_rel"] = round(float((yq - ye).abs().mean()) / scale, 6)
    out["q8_midpoint_mean_abs_err_rel"] = round(float((ym - ye).abs().mean()) / scale, 6)
    out["i8_copy_mean_abs_err_rel"] = round(float((yi - ye).abs().mean()) / scale, 6)
    # top-1 agreement with the exact pass over many rows of x (passes of 32 through the top-1
    # entry points; the first 16 rows are the timed x)
    rows = 1024
    xa = to_dev_bits(synth.gen_x(rows, k, tensor_id=tid), dev)
    agree = {"q8": 0, "q8_midpoint": 0, "i8_copy": 0}
    for r0 in range(0, rows, 32):
        xr = xa[r0:r0 + 32]
        ie32 = w12.gemm_top1(xr, rec)[0]
        for name, fn in (("q8", lambda: w12.q8_top1(xr, rec)), ("q8_midpoint", lambda: w12.q8_top1(xr, rec, midpoint=True)),
                         ("i8_copy", lambda: w12.i8_top1(xr, cp))):
            agree[name] += int((fn()[0] == ie32).sum())
    for name, v in agree.items():
        out[f"top1_agreement_{name}_vs_exact_{rows}_rows"] = f"{v}/{rows}"
    # the top-1 entry points against the first maximum of the full outputs of the same kernel
    # (the automatic path's: the streaming kernel in one row group at this size), and their
    # values bit for bit
    def same_top1(t, yy):
        want = yy.cpu().numpy().argmax(axis=1)
        got_v = t[1].cpu().numpy()
        return bool(np.array_equal(t[0].cpu().numpy(), want)
                    and np.array_equal(got_v.view(np.uint32), yy.cpu().numpy()[np.arange(m), want].view(np.uint32)))
    out["top1_matches_full_outputs"] = (same_top1(tq, yq) and same_top1(te, ye) and same_top1(tm, ym)
                                        and same_top1(ti, yi))
    samples = [("lm_head q8 m=16 (rows 0..127)", x_bits, keep, yq[:, :128].cpu().numpy(), "q8"),
               ("lm_head w12 m=16 (rows 0..127)", x_bits, keep, ye[:, :128].cpu().numpy()),
               ("lm_head q8 midpoint m=16 (rows 0..127)", x_bits, keep, ym[:, :128].cpu().numpy(), "q8m"),
               ("lm_head i8 copy m=16 (rows 0..127)", x_bits, keep, yi[:, :128].cpu().numpy(), "i8")]
    return out, samples


def silu_bench(w_bits, x_bits, dev, stream, rot):
    """The gate+up shape as an MLP's two [17408, 5120] halves, row-interleaved
    (w12_interleave_rows), at M = 1 and 32: the exact pass with the SiLU(gate) * up epilogue
    (h [m, 17408]: half the output bytes) against the plain exact pass on the same record, over
    `rot` copies so every launch reads HBM.  Returns (results, parity samples)."""
    import torch
    from lossless_bit_weight_02_amd import w12

    half = w_bits.shape[0] // 2
    n, k = w_bits.shape
    to_dev = lambda bits: to_dev_bits(bits, dev)
    gr, ur = w12.encode(to_dev(w_bits[:half])), w12.encode(to_dev(w_bits[half:]))
    rec0 = w12.interleave_rows(gr, ur)
    del gr, ur
    recs = [rec0] + [rec0.clone() for _ in range(rot - 1)]
    out = {"n": n, "k": k, "i": half}
    samples = []
    for m in (1, 32):
        xm = to_dev(x_bits[:m])
        ys = torch.empty((m, n), dtype=torch.float32, device=dev)
        hs = torch.empty((m, half), dtype=torch.float32, device=dev)
        for name, fn in (("w12", lambda r: w12.gemm(xm, recs[r], out=ys)),
                         ("w12_silu_mul", lambda r: w12.gemm_silu_mul(xm, recs[r], out=hs))):
            fn(0)
            reps = 2 * rot
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record(stream)
            for r in range(reps):
                fn(r % rot)
            eb.record(stream)
            torch.cuda.synchronize()
            t = ea.elapsed_time(eb) * 1e-3 / reps
            byt = w12_bytes(n, k, rec0.n_esc, m) - (2 * m * n if name == "w12_silu_mul" else 0)
            out[f"{name}_m{m}_us"] = round(t * 1e6, 2)
            out[f"{name}_m{m}_gbs"] = round(byt / t / 1e9, 1)
        # the first 64 outputs read interleaved rows 0..127: gate rows 0..63 and up rows 0..63
        wi = np.empty((128, k), dtype=np.uint16)
        for t in range(8):
            wi[16 * t:16 * t + 8] = w_bits[8 * t:8 * t + 8]
            wi[16 * t + 8:16 * t + 16] = w_bits[half + 8 * t:half + 8 * t + 8]
        samples.append((f"silu_mul m={m} (outputs 0..63)", x_bits[:m], wi, hs[:, :64].cpu().numpy(), "silu"))
    return out, samples


def stack_bench(dev, stream, layers, reps, sample_layer):
    """The 27B-class dense stack: `layers` layers of {q, k, v, o, gate, up, down} (tensor id
    8*layer + projection).  Every matrix is drawn on the GPU (synth.gen_weight_torch), encoded,
    decoded and compared bit for bit with its source, and tiled for the BF16 baseline; then one
    pass over all matrices at M=1 and at M=32 (automatic path) is timed launched one by one
    (wall time, host gaps included) and as one captured HIP graph (~kernel-sum time).
    Returns (results, parity samples of `sample_layer`: its first 128 rows per projection)."""
    import torch
    from lossless_bit_weight_02_amd import synth, w12

    cfg = synth.CONFIGS["stack"]
    n_proj = len(synth.STACK_PROJ)
    entries = cfg.weights[:layers * n_proj]
    recs, tiles, keep = [], [], {}
    t0 = time.perf_counter()
    t_enc = 0.0
    n_esc = 0
    weights = 0
    for i, (tid, label, spec) in enumerate(entries):
        w = synth.gen_weight_torch(spec, 0, tid, dev)
        torch.cuda.synchronize()
        te = time.perf_counter()
        rec = w12.encode(w)
        torch.cuda.synchronize()
        t_enc += time.perf_counter() - te
        back = w12.decode(rec)
        if not torch.equal(back.view(torch.int16), w.view(torch.int16)):
            raise SystemExit(f"stack {label}: decode(encode(W)) is not bit-exact")
        del back
        tiles.append(w12.bf16_tiles(w))
        if i // n_proj == sample_layer:
            keep[i] = w[:128].view(torch.int16).cpu().numpy().view(np.uint16)
        del w
        recs.append(rec)
        n_esc += rec.n_esc
        weights += spec.n * spec.k
    t_build = time.perf_counter() - t0
    xs = {}
    for p, (nm, n, k) in enumerate(synth.STACK_PROJ):
        if k not in xs:
            xb = synth.gen_x(32, k, tensor_id=p)
            xs[k] = (xb, to_dev_bits(xb, dev))
    out = {"layers": layers, "matrices": len(entries), "weights": weights, "escapes": n_esc,
           "escape_fraction": round(n_esc / weights, 7),
           "bits_per_weight": round(8.0 * sum(r.nbytes() for r in recs) / weights, 4),
           "lossless_all": True, "encode_s_total": round(t_enc, 3),
           "build_s": round(t_build, 2)}
    samples = []
    for m in (1, 32):
        ys = [torch.empty((m, spec.n), dtype=torch.float32, device=dev) for _, _, spec in entries]
        yb = [torch.empty((m, spec.n), dtype=torch.float32, device=dev) for _, _, spec in entries]
        xm = {k: v[1][:m] for k, v in xs.items()}
        w12_fns = [lambda i=i: w12.gemm(xm[recs[i].k], recs[i], out=ys[i]) for i in range(len(recs))]
        bf_fns = [lambda i=i: w12.bf16_gemm(xm[tiles[i].k], tiles[i], out=yb[i])
                  for i in range(len(tiles))]
        b_w12 = sum(w12_bytes(r.n, r.k, r.n_esc, m) for r in recs)
        b_bf = sum(bf16_bytes(t.n, t.k, m) for t in tiles)
        row = {"w12_bytes": b_w12, "bf16_bytes": b_bf}
        for name, fns, outs, byt in (("w12", w12_fns, ys, b_w12), ("bf16", bf_fns, yb, b_bf)):
            t_e = time_eager(fns, stream, reps)
            g = capture_graph(fns, outs)
            t_g = time_graph(g, stream, reps)
            del g
            row[f"{name}_ms_graph"] = round(t_g * 1e3, 4)
            row[f"{name}_gbs_graph"] = round(byt / t_g / 1e9, 1)
            row[f"{name}_ms_eager"] = round(t_e * 1e3, 4)
            row[f"{name}_gbs_eager"] = round(byt / t_e / 1e9, 1)
        row["w12_frac_hbm_graph"] = round(row["w12_gbs_graph"] / HBM_PEAK_GBS, 4)
        row["speedup_vs_bf16_graph"] = round(row["bf16_ms_graph"] / row["w12_ms_graph"], 4)
        # per projection: its `layers` launches as one graph (us per launch)
        per = {}
        for p, (nm, _, _) in enumerate(synth.STACK_PROJ):
            idx = list(range(p, len(recs), n_proj))
            for name, fns, outs in (("w12", w12_fns, ys), ("bf16", bf_fns, yb)):
                g = capture_graph([fns[i] for i in idx], [outs[i] for i in idx])
                t = time_graph(g, stream, reps) / len(idx)
                del g
                r0 = recs[idx[0]]
                byt = (w12_bytes(r0.n, r0.k, r0.n_esc, m) if name == "w12" else
                       bf16_bytes(r0.n, r0.k, m))
                per[f"{nm}_{name}_us"] = round(t * 1e6, 2)
                per[f"{nm}_{name}_gbs"] = round(byt / t / 1e9, 1)
        row["per_projection"] = per
        out[f"m{m}"] = row
        for i, wrows in keep.items():
            samples.append((f"stack {entries[i][1]} w12 m={m}", xs[recs[i].k][0][:m], wrows,
                            ys[i][:, :128].cpu().numpy()))
        del ys, yb

    # The same layers as an inference engine lays them out: q, k, v stacked into one qkv matrix and
    # gate, up into one gate_up matrix (they read the same activations), 4 launches per layer.
    # The stacked W12 records come from w12_concat_rows (no re-encoding); the stacked dense tiles
    # are the parts' tiles back to back (the tiled order is row-tile-major).
    assert n_proj == 7
    frecs, ftiles = [], []
    for l in range(layers):
        r = recs[l * 7:(l + 1) * 7]
        t = tiles[l * 7:(l + 1) * 7]
        for grp in ((0, 1, 2), (3,), (4, 5), (6,)):
            if len(grp) == 1:
                frecs.append(r[grp[0]])
                ftiles.append(t[grp[0]])
            else:
                frecs.append(w12.concat_rows([r[g] for g in grp]))
                ftiles.append(w12.Bf16Tiles(sum(t[g].n for g in grp), t[grp[0]].k,
                                            torch.cat([t[g].data for g in grp])))
    fused = {"layout": "per layer: qkv [8192,5120], o [5120,6144], gate_up [34816,5120], down [5120,17408]"}
    for m in (1, 32):
        ys = [torch.empty((m, r.n), dtype=torch.float32, device=dev) for r in frecs]
        yb = [torch.empty((m, t.n), dtype=torch.float32, device=dev) for t in ftiles]
        xm = {k: v[1][:m] for k, v in xs.items()}
        w12_fns = [lambda i=i: w12.gemm(xm[frecs[i].k], frecs[i], out=ys[i]) for i in range(len(frecs))]
        bf_fns = [lambda i=i: w12.bf16_gemm(xm[ftiles[i].k], ftiles[i], out=yb[i]) for i in range(len(ftiles))]
        b_w12 = sum(w12_bytes(r.n, r.k, r.n_esc, m) for r in frecs)
        b_bf = sum(bf16_bytes(t.n, t.k, m) for t in ftiles)
        row = {}
        for name, fns, outs, byt in (("w12", w12_fns, ys, b_w12), ("bf16", bf_fns, yb, b_bf)):
            g = capture_graph(fns, outs)
            t_g = time_graph(g, stream, reps)
            del g
            row[f"{name}_ms_graph"] = round(t_g * 1e3, 4)
            row[f"{name}_gbs_graph"] = round(byt / t_g / 1e9, 1)
        row["w12_frac_hbm_graph"] = round(row["w12_gbs_graph"] / HBM_PEAK_GBS, 4)
        row["speedup_vs_bf16_graph"] = round(row["bf16_ms_graph"] / row["w12_ms_graph"], 4)
        fused[f"m{m}"] = row
        del ys, yb
    out["fused_layout"] = fused
    del frecs, ftiles
    return out, samples


def cpu_count():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w_bits, x_bits, gpu_out, rows, samples=()):
    """Time the oracle (as it stands) on the first `rows` rows of the workload, and check the
    GPU outputs of the timed step on the same rows; then check each extra sample
    (label, x bits [m, k], W bits [r, k], GPU y [m, r]) against the oracle's exact GEMM."""
    import oracle
    from threadpoolctl import threadpool_info

    ws = w_bits[:rows]
    t0 = time.perf_counter()
    rec = oracle.encode(ws)
    t_enc = time.perf_counter() - t0
    t0 = time.perf_counter()
    dec = oracle.decode(rec)
    t_dec = time.perf_counter() - t0
    assert np.array_equal(dec, ws)
    t0 = time.perf_counter()
    y1 = oracle.w12_gemm64(x_bits[:1], rec)
    t_g1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    y32 = oracle.w12_gemm64(x_bits[:32], rec)
    t_g32 = time.perf_counter() - t0
    t0 = time.perf_counter()
    yq = oracle.q8_gemm64(x_bits[:16], rec)
    t_q = time.perf_counter() - t0
    total = t_enc + t_dec + t_g1 + t_g32 + t_q

    # parity of the timed GPU outputs on these rows (same bar as the tests)
    worst = 0.0
    for name, y, xb, wref in (("w12_m1", y1, x_bits[:1], ws), ("w12_m32", y32, x_bits[:32], ws),
                              ("q8_m16", yq, x_bits[:16], oracle.q8_view_bits(rec))):
        g = gpu_out[name][:, :rows].astype(np.float64)
        bound = 1e-3 * oracle.abs_bound64(xb, wref)
        err = np.abs(g - y)
        if not np.all(err <= bound):
            raise SystemExit(f"parity failure in {name}: GPU output outside the bound")
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    for label, xb, wb, gy, *view in samples:
        if view and view[0] == "silu":
            y64, ab = oracle.gemm64(xb, wb), oracle.abs_bound64(xb, wb)
            err = np.abs(gy.astype(np.float64) - oracle.silu_mul64(y64))
            bound = oracle.silu_mul_bound(y64, ab)
            if not np.all(err <= bound):
                raise SystemExit(f"parity failure in {label}: GPU output outside the bound")
            worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
            continue
        if view and view[0] == "i8":
            ref = oracle.encode(wb)
            wq = oracle.i8_weights64(ref, oracle.i8_copy(ref))
            y, bound = oracle.gemm64_f(xb, wq), 1e-3 * oracle.abs_bound64_f(xb, wq)
        else:
            if view and view[0] in ("q8", "q8m"):
                wb = oracle.q8_view_bits(oracle.encode(wb), midpoint=view[0] == "q8m")
            y = oracle.gemm64(xb, wb)
            bound = 1e-3 * oracle.abs_bound64(xb, wb)
        err = np.abs(gy.astype(np.float64) - y)
        if not np.all(err <= bound):
            raise SystemExit(f"parity failure in {label}: GPU output outside the bound")
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    gbs = w12_bytes(rows, ws.shape[1], rec.n_esc, 1) / t_g1 / 1e9
    return {
        "value": round(gbs, 4), "unit": "GB/s", "cores": int(blas), "kind": "oracle",
        "sample": f"first {rows} of {w_bits.shape[0]} rows of the gate+up matrix; oracle encode "
                  f"{t_enc:.2f}s, decode {t_dec:.2f}s, exact GEMM M=1 {t_g1:.2f}s (value: W12 "
                  f"bytes / this time), M=32 {t_g32:.2f}s, Q8 M=16 {t_q:.2f}s; numpy, BLAS threads "
                  f"{blas} of {cpu_count()} host cores",
        "seconds": round(total, 3),
        "parity_worst_err_over_bound": round(worst, 5),
        "parity_samples": len(samples),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle leg")
    ap.add_argument("--no-sweep", action="store_true", help="skip the M sweep (crossover)")
    ap.add_argument("--no-attn", action="store_true", help="skip the attention-projection section")
    ap.add_argument("--no-stack", action="store_true", help="skip the 64-layer stack section")
    ap.add_argument("--no-lm-head", action="store_true", help="skip the LM-head Q-pass section")
    ap.add_argument("--stack-layers", type=int, default=64)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 192 MiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--min-rot-bytes", type=float, default=1.1e9)
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the W12 path here is a single-GPU kernel set "
              "(multi-GPU sharding is a design note, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from lossless_bit_weight_02_amd import synth, w12

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    spec = synth.CONFIGS["gate_up"].weights[0][2]
    tid = synth.CONFIGS["gate_up"].weights[0][0]
    n, k = spec.n, spec.k
    t0 = time.perf_counter()
    w_bits = synth.gen_weight(spec, 0, tid)
    x_bits = synth.gen_x(256, k, tensor_id=tid)
    t_gen = time.perf_counter() - t0

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    w_dev = to_dev(w_bits)
    rec0 = w12.encode(w_dev)
    n_esc = rec0.n_esc
    rec_bytes = rec0.nbytes()
    rot = max(2, int(np.ceil(a.min_rot_bytes / rec_bytes)))
    recs = [rec0] + [rec0.clone() for _ in range(rot - 1)]
    wcopies = [w_dev] + [w_dev.clone() for _ in range(rot - 1)]      # row-major (encode input)
    btiles = [w12.bf16_tiles(wc) for wc in wcopies]                   # baseline layout
    x1, x16, x32 = to_dev(x_bits[:1]), to_dev(x_bits[:16]), to_dev(x_bits[:32])
    y1 = torch.empty((1, n), dtype=torch.float32, device=dev)
    y16 = torch.empty((16, n), dtype=torch.float32, device=dev)
    y32 = torch.empty((32, n), dtype=torch.float32, device=dev)
    yb1 = torch.empty_like(y1)
    yb32 = torch.empty_like(y32)
    dec_out = torch.empty((n, k), dtype=torch.bfloat16, device=dev)

    # encode target: a preallocated record reused every step (escape arrays sized once)
    enc = rec0.clone()
    enc_struct = enc.c_struct()
    import ctypes
    n_esc_c = ctypes.c_uint64(0)

    def do_encode(wd):
        st = w12.lib().w12_encode(wd.data_ptr(), ctypes.byref(enc_struct), ctypes.byref(n_esc_c),
                                  stream.cuda_stream)
        if st != 0:
            raise RuntimeError(w12.lib().w12_last_error())

    probe_buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)

    # The codec kernels leave hundreds of MB of dirty lines in the caches (the decode writes the
    # whole bf16 matrix); a GEMM launched right after them pays for writing those back.  A cached
    # read of 512 MiB after the codec group writes them back before the GEMM groups start, so
    # that every GEMM is timed as it runs in a decode loop (after other reads).  It is part of
    # the step (ms_per_step includes it) and of no metric.
    flush_buf = torch.ones(1 << 27, dtype=torch.float32, device=dev)

    # (name, launches per step, fn(launch index)); the M=1 group runs every copy twice so that
    # the event gaps around a group weigh less in its per-launch average
    ops = [
        ("encode", rot, lambda r: do_encode(wcopies[r])),
        ("decode", rot, lambda r: w12.decode_into(recs[r], dec_out)),
        ("cache_flush", 1, lambda r: flush_buf.sum()),
        ("read_probe", 1, lambda r: w12.read_probe(probe_buf, sink)),
        ("w12_m1", 2 * rot, lambda r: w12.gemm(x1, recs[r % rot], path="gemv", out=y1)),
        ("w12_m32", rot, lambda r: w12.gemm(x32, recs[r], out=y32)),
        ("q8_m16", rot, lambda r: w12.q8_gemm(x16, recs[r], out=y16)),
        ("bf16_m1", 2 * rot, lambda r: w12.bf16_gemm(x1, btiles[r % rot], path="gemv", out=yb1)),
        ("bf16_m32", rot, lambda r: w12.bf16_gemm(x32, btiles[r], out=yb32)),
    ]

    def step(evs=None):
        for j, (_, reps, fn) in enumerate(ops):
            if evs is not None:
                evs[2 * j].record(stream)
            for r in range(reps):
                fn(r)
            if evs is not None:
                evs[2 * j + 1].record(stream)

    for i in range(a.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(ops))] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(a.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    per_op = {name: [] for name, _, _ in ops}
    for evs in events:
        for j, (name, reps, _) in enumerate(ops):
            per_op[name].append(evs[2 * j].elapsed_time(evs[2 * j + 1]) * 1e-3 / reps)
    mean = {name: float(np.mean(v)) for name, v in per_op.items()}
    med = {name: float(np.median(v)) for name, v in per_op.items()}

    gpu_out = {"w12_m1": y1.cpu().numpy(), "w12_m32": y32.cpu().numpy(), "q8_m16": y16.cpu().numpy()}

    b_w12_1 = w12_bytes(n, k, n_esc, 1)
    b_w12_32 = w12_bytes(n, k, n_esc, 32)
    gbs = {
        "w12_m1": b_w12_1 / mean["w12_m1"] / 1e9,
        "w12_m32": b_w12_32 / mean["w12_m32"] / 1e9,
        "q8_m16": q8_bytes(n, k, n_esc, 16) / mean["q8_m16"] / 1e9,
        "bf16_m1": bf16_bytes(n, k, 1) / mean["bf16_m1"] / 1e9,
        "bf16_m32": bf16_bytes(n, k, 32) / mean["bf16_m32"] / 1e9,
        "decode": (1.5 * n * k + n + 4 * (n + 1) + 6 * n_esc + 2 * n * k) / mean["decode"] / 1e9,
        "encode": (2 * n * k + 1.5 * n * k + n + 4 * (n + 1) + 6 * n_esc) / mean["encode"] / 1e9,
    }

    probe_gbs = probe_buf.numel() / mean["read_probe"] / 1e9
    del probe_buf

    if a.calibrate_copy:
        src = torch.empty(192 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    sweep = None
    sweep_samples = []
    if not a.no_sweep:
        sweep = {}
        xs = to_dev(x_bits)
        for m in (1, 4, 8, 16, 32, 64, 128, 256):
            xm = xs[:m].contiguous()
            ym = torch.empty((m, n), dtype=torch.float32, device=dev)
            row = {}
            # the streaming kernel up to 32 rows; above 64 rows only the matrix-core path (passes of
            # up to 128 rows, each reading W once)
            paths = ("gemv", "mfma", "stream") if m <= 64 else ("mfma",)
            for path in paths:
                for fmt in ("w12", "bf16"):
                    def run(r, fmt=fmt, path=path):
                        if fmt == "w12":
                            w12.gemm(xm, recs[r], path=path, out=ym)
                        else:
                            w12.bf16_gemm(xm, btiles[r], path=path, out=ym)
                    run(0)
                    reps = 2 * rot
                    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    ea.record(stream)
                    for r in range(reps):
                        run(r % rot)
                    eb.record(stream)
                    torch.cuda.synchronize()
                    t = ea.elapsed_time(eb) * 1e-3 / reps
                    byt = w12_bytes(n, k, n_esc, m) if fmt == "w12" else bf16_bytes(n, k, m)
                    row[f"{fmt}_{path}_us"] = round(t * 1e6, 2)
                    row[f"{fmt}_{path}_gbs"] = round(byt / t / 1e9, 1)
                    if m > 64 or (path == "stream" and m in (16, 32)):
                        # the timed outputs of the passes of more than 64 rows and of the
                        # streaming kernel: their first 128 weight rows go to the CPU-oracle leg
                        sweep_samples.append((f"sweep {fmt} {path} m={m} (rows 0..127)", x_bits[:m],
                                              w_bits[:128], ym[:, :128].cpu().numpy()))
            if m in (1, 32, 128):
                # the same W12 GEMM with bfloat16 outputs (rounded where they are stored)
                path = "gemv" if m == 1 else "mfma"
                ym16 = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                w12.gemm(xm, recs[0], path=path, out=ym16)
                reps = 2 * rot
                ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ea.record(stream)
                for r in range(reps):
                    w12.gemm(xm, recs[r % rot], path=path, out=ym16)
                eb.record(stream)
                torch.cuda.synchronize()
                t = ea.elapsed_time(eb) * 1e-3 / reps
                row["w12_bf16out_us"] = round(t * 1e6, 2)
                row["w12_bf16out_gbs"] = round((w12_bytes(n, k, n_esc, m) - 2 * m * n) / t / 1e9, 1)
            row["best_w12_path"] = min((p for p in paths), key=lambda p: row[f"w12_{p}_us"])
            row["w12_mfma_tflops"] = round(2 * m * n * k / (row["w12_mfma_us"] * 1e-6) / 1e12, 1)
            sweep[str(m)] = row

    silu = None
    if not a.no_sweep:
        silu, smp = silu_bench(w_bits, x_bits, dev, stream, rot)
        sweep_samples += smp
        torch.cuda.empty_cache()

    # Context, not a metric: the vendor library's dense bf16 GEMM on the same weights (torch.mm,
    # which dispatches to hipBLASLt/rocBLAS), computed as y^T = W x^T with both operands
    # contiguous; the pages compare W12 against the vendor library of their GPU.
    vendor = None
    if not a.no_sweep:
        vendor = {}
        for m in (1, 32):
            xt = to_dev(x_bits[:m]).t().contiguous()
            yt = torch.empty((n, m), dtype=torch.bfloat16, device=dev)
            torch.mm(wcopies[0], xt, out=yt)
            reps = 2 * rot
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record(stream)
            for r in range(reps):
                torch.mm(wcopies[r % rot], xt, out=yt)
            eb.record(stream)
            torch.cuda.synchronize()
            t = ea.elapsed_time(eb) * 1e-3 / reps
            w12_t = mean["w12_m1"] if m == 1 else mean["w12_m32"]
            vendor[f"m{m}_us"] = round(t * 1e6, 2)
            vendor[f"m{m}_gbs"] = round(bf16_bytes(n, k, m) / t / 1e9, 1)
            vendor[f"w12_speedup_m{m}"] = round(t / w12_t, 4)

    # Context beside the step: the attention projection at M=1, and the whole 64-layer stack at
    # M=1 and M=32 (both also run as captured HIP graphs); their outputs are parity-checked in
    # the CPU-oracle leg.
    samples = list(sweep_samples)
    attn = None
    if not a.no_attn:
        attn, smp = attn_bench(dev, stream, a.min_rot_bytes, reps=20)
        samples += smp
    lm_head = None
    if not a.no_lm_head:
        lm_head, smp = lm_head_bench(dev, stream, reps=10)
        samples += smp
        torch.cuda.empty_cache()
    stack = None
    if not a.no_stack:
        stack, smp = stack_bench(dev, stream, a.stack_layers, reps=5,
                                 sample_layer=min(31, a.stack_layers - 1))
        samples += smp
        torch.cuda.empty_cache()

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(w_bits, x_bits, gpu_out, min(a.cpu_rows, n), samples)

    value = gbs["w12_m1"]
    traffic = measured_traffic()
    out = {
        "metric": "W12 GEMM effective HBM GB/s (and % of peak) at M=1 and M=32; speedup vs BF16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mlp_gate_up_fused W bf16 [34816,5120] (27B-class projection), "
                               "x bf16 [M,5120]; value at M=1, also M=32",
                   "n": n, "k": k, "m_values": [1, 32], "rotation_copies": rot,
                   "escapes": n_esc, "bits_per_weight": round(8.0 * rec_bytes / (n * k), 4)},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 1),
                     "kernel": "k_gemv<W12, M=1>", "bytes_per_launch": round(b_w12_1, 1),
                     "avg_launch_us": round(mean["w12_m1"] * 1e6, 3)},
        "cpu_baseline": cpu,
        "m32": {"gbs": round(gbs["w12_m32"], 2), "frac_hbm": round(gbs["w12_m32"] / HBM_PEAK_GBS, 4),
                "tflops": round(2 * 32 * n * k / mean["w12_m32"] / 1e12, 2),
                "frac_mfma_bf16": round(2 * 32 * n * k / mean["w12_m32"] / 1e12 / MFMA_BF16_PEAK_TFS, 4)},
        "speedup_vs_bf16": {"m1": round(mean["bf16_m1"] / mean["w12_m1"], 4),
                            "m32": round(mean["bf16_m32"] / mean["w12_m32"], 4)},
        "ops_us_mean": {kk: round(v * 1e6, 3) for kk, v in mean.items()},
        "ops_us_median": {kk: round(v * 1e6, 3) for kk, v in med.items()},
        "ops_gbs": {kk: round(v, 1) for kk, v in gbs.items()},
        "read_probe_gbs": round(probe_gbs, 1),
        "w12_m1_frac_of_probe": round(value / probe_gbs, 4),
        "sweep": sweep,
        "vendor_bf16_torch_mm": vendor,
        "attn_m1": attn,
        "lm_head_q_pass": lm_head,
        "silu_mul_gate_up": silu,
        "stack": stack,
        "setup_s": {"generate": round(t_gen, 2)},
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
