"""Python binding of libw12.so (ctypes): argument marshalling over torch device tensors.

Every step runs in the HIP library; this module only allocates the output tensors with torch,
passes raw device pointers and the current stream, and turns non-zero statuses into W12Error.
If the library is missing, loading fails loudly: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw12.so")

W12_OK = 0
W12_ERR_ARG = -1
W12_ERR_SHAPE = -2
W12_ERR_ALIGN = -3
W12_ERR_CAPACITY = -4
W12_ERR_RANGE = -5
W12_ERR_HIP = -6

PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_STREAM = 0, 1, 2, 3
Q8_MIDPOINT = 0x10
OUT_BF16 = 0x20
_PATHS = {None: PATH_AUTO, "auto": PATH_AUTO, "gemv": PATH_GEMV, "mfma": PATH_MFMA, "stream": PATH_STREAM}


class W12Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"w12 status {status}: {msg}")
        self.status = status


class _W12Weight(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("base", ctypes.c_void_p), ("ae", ctypes.c_void_p), ("lo", ctypes.c_void_p),
                ("esc_ptr", ctypes.c_void_p), ("esc_col", ctypes.c_void_p),
                ("esc_val", ctypes.c_void_p), ("esc_cap", ctypes.c_uint64)]


class _W12I8(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


_lib = None
_lock = threading.Lock()

# name -> (restype, argtypes)
EXPORTS = {
    "w12_abi_version": (ctypes.c_int, []),
    "w12_release_workspace": (ctypes.c_int, [ctypes.c_void_p]),
    "w12_last_error": (ctypes.c_char_p, []),
    "w12_encode": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(_W12Weight),
                                  ctypes.POINTER(ctypes.c_uint64), ctypes.c_void_p]),
    "w12_decode": (ctypes.c_int, [ctypes.POINTER(_W12Weight), ctypes.c_void_p, ctypes.c_void_p]),
    "w12_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12Weight),
                                ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "w12_gemm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12Weight),
                                        ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "w12_q8_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12Weight),
                                   ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "w12_q8_top1": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12Weight),
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "w12_gemm_top1": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12Weight),
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "w12_gemm_silu_mul": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12Weight),
                                         ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "w12_interleave_rows": (ctypes.c_int, [ctypes.POINTER(_W12Weight), ctypes.POINTER(_W12Weight),
                                           ctypes.POINTER(_W12Weight), ctypes.POINTER(ctypes.c_uint64),
                                           ctypes.c_void_p]),
    "w12_i8_build": (ctypes.c_int, [ctypes.POINTER(_W12Weight), ctypes.POINTER(_W12I8), ctypes.c_void_p]),
    "w12_i8_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12I8),
                                   ctypes.POINTER(_W12Weight), ctypes.c_void_p, ctypes.c_uint32,
                                   ctypes.c_void_p]),
    "w12_i8_top1": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_W12I8),
                                   ctypes.POINTER(_W12Weight), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_uint32, ctypes.c_void_p]),
    "w12_concat_rows": (ctypes.c_int, [ctypes.POINTER(_W12Weight), ctypes.c_int,
                                       ctypes.POINTER(_W12Weight), ctypes.POINTER(ctypes.c_uint64),
                                       ctypes.c_void_p]),
    "w12_bf16_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_uint32, ctypes.c_void_p]),
    "w12_bf16_to_tiles": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p]),
    "w12_read_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_void_p]),
}


def padded_rows(n: int) -> int:
    """Rows of the tiled plane storage (16-row tiles)."""
    return 16 * ((int(n) + 15) // 16)


def lib():
    """The loaded library (raises if it was never built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m lossless_bit_weight_02_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in EXPORTS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            if L.w12_abi_version() != 1:
                raise RuntimeError("libw12.so ABI version mismatch")
            _lib = L
    return _lib


def _check(status: int):
    if status != W12_OK:
        raise W12Error(status, lib().w12_last_error().decode(errors="replace"))


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bfloat16 (or 16-bit raw bits), got {t.dtype}")


class W12Weight:
    """A W12 record held as torch device tensors (layout of include/w12.h; ``ae`` and ``lo`` are
    in the tiled storage order, padded_rows(n) rows)."""

    def __init__(self, n, k, base, ae, lo, esc_ptr, esc_col, esc_val):
        self.n, self.k = int(n), int(k)
        self.base, self.ae, self.lo = base, ae, lo
        self.esc_ptr, self.esc_col, self.esc_val = esc_ptr, esc_col, esc_val

    @property
    def n_esc(self) -> int:
        return int(self.esc_col.numel())

    @property
    def device(self):
        return self.ae.device

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.base, self.ae, self.lo, self.esc_ptr, self.esc_col, self.esc_val))

    def bits_per_weight(self) -> float:
        return 8.0 * self.nbytes() / (self.n * self.k)

    def c_struct(self) -> _W12Weight:
        return _W12Weight(self.n, self.k, _ptr(self.base), _ptr(self.ae), _ptr(self.lo),
                          _ptr(self.esc_ptr), _ptr(self.esc_col), _ptr(self.esc_val),
                          self.esc_col.numel())

    def clone(self) -> "W12Weight":
        return W12Weight(self.n, self.k, *(t.clone() for t in
                                           (self.base, self.ae, self.lo, self.esc_ptr,
                                            self.esc_col, self.esc_val)))

    def to_numpy(self) -> dict:
        """Host copies of every array as stored (uint8/uint32/uint16 numpy arrays; ``ae_s`` and
        ``lo_s`` flat, in the tiled storage order)."""
        def host(t, dt):
            return t.cpu().numpy().view(dt)
        import numpy as np
        return dict(n=self.n, k=self.k, base=host(self.base, np.uint8),
                    ae_s=host(self.ae, np.uint8), lo_s=host(self.lo, np.uint8),
                    esc_ptr=host(self.esc_ptr, np.uint32), esc_col=host(self.esc_col, np.uint32),
                    esc_val=host(self.esc_val, np.uint16))


def encode(w: torch.Tensor, esc_guess: int | None = None) -> W12Weight:
    """bfloat16 W [n, k] on the GPU -> W12Weight (one host synchronisation for the escape total)."""
    w = _bits16(w)
    if w.dim() != 2 or not w.is_cuda:
        raise ValueError("w must be a 2-D CUDA tensor")
    w = w.contiguous()
    n, k = w.shape
    dev = w.device
    u8, i32, i16 = torch.uint8, torch.int32, torch.int16
    base = torch.empty(n, dtype=u8, device=dev)
    npad = padded_rows(n)
    ae = torch.empty(npad * k, dtype=u8, device=dev)
    lo = torch.empty(npad * k // 2, dtype=u8, device=dev)
    esc_ptr = torch.empty(n + 1, dtype=i32, device=dev)
    cap = max(1024, (n * k) // 256) if esc_guess is None else max(1, int(esc_guess))
    esc_col = torch.empty(cap, dtype=i32, device=dev)
    esc_val = torch.empty(cap, dtype=i16, device=dev)
    n_esc = ctypes.c_uint64(0)
    L = lib()
    def run():
        s = _W12Weight(n, k, base.data_ptr(), ae.data_ptr(), lo.data_ptr(),
                       esc_ptr.data_ptr(), esc_col.data_ptr(), esc_val.data_ptr(), esc_col.numel())
        return L.w12_encode(w.data_ptr(), ctypes.byref(s), ctypes.byref(n_esc), _stream_handle(dev))

    st = run()
    if st == W12_ERR_CAPACITY:  # the first guess was too small: size exactly and encode again
        esc_col = torch.empty(max(1, n_esc.value), dtype=i32, device=dev)
        esc_val = torch.empty(max(1, n_esc.value), dtype=i16, device=dev)
        st = run()
    _check(st)
    ne = n_esc.value
    return W12Weight(n, k, base, ae, lo, esc_ptr, esc_col[:ne], esc_val[:ne])


def concat_rows(parts) -> W12Weight:
    """Record of the row-stacked matrix [W_0; W_1; ...] from the parts' records (same k; every part
    but the last with n % 16 == 0), built on the device without re-encoding."""
    parts = list(parts)
    if not parts:
        raise ValueError("no parts")
    dev = parts[0].device
    k = parts[0].k
    n = sum(p.n for p in parts)
    ne = sum(p.n_esc for p in parts)
    npad = padded_rows(n)
    u8 = torch.uint8
    out = W12Weight(n, k, torch.empty(n, dtype=u8, device=dev), torch.empty(npad * k, dtype=u8, device=dev),
                    torch.empty(npad * k // 2, dtype=u8, device=dev),
                    torch.empty(n + 1, dtype=torch.int32, device=dev),
                    torch.empty(max(1, ne), dtype=torch.int32, device=dev)[:ne],
                    torch.empty(max(1, ne), dtype=torch.int16, device=dev)[:ne])
    arr = (_W12Weight * len(parts))(*[p.c_struct() for p in parts])
    s = out.c_struct()
    s.esc_cap = ne
    n_esc = ctypes.c_uint64(0)
    _check(lib().w12_concat_rows(arr, len(parts), ctypes.byref(s), ctypes.byref(n_esc), _stream_handle(dev)))
    return out


def interleave_rows(gate: W12Weight, up: W12Weight) -> W12Weight:
    """Record of the gate and up projections with rows interleaved in groups of 8 (rows 16t..16t+7
    gate rows 8t..8t+7, rows 16t+8..16t+15 up rows 8t..8t+7), built on the device without
    re-encoding; the input of gemm_silu_mul."""
    dev, k, n = gate.device, gate.k, 2 * gate.n
    ne = gate.n_esc + up.n_esc
    npad = padded_rows(n)
    u8 = torch.uint8
    out = W12Weight(n, k, torch.empty(n, dtype=u8, device=dev), torch.empty(npad * k, dtype=u8, device=dev),
                    torch.empty(npad * k // 2, dtype=u8, device=dev),
                    torch.empty(n + 1, dtype=torch.int32, device=dev),
                    torch.empty(max(1, ne), dtype=torch.int32, device=dev)[:ne],
                    torch.empty(max(1, ne), dtype=torch.int16, device=dev)[:ne])
    g, u, o = gate.c_struct(), up.c_struct(), out.c_struct()
    o.esc_cap = ne
    n_esc = ctypes.c_uint64(0)
    _check(lib().w12_interleave_rows(ctypes.byref(g), ctypes.byref(u), ctypes.byref(o), ctypes.byref(n_esc),
                                     _stream_handle(dev)))
    return out


def decode_into(wt: W12Weight, out: torch.Tensor) -> torch.Tensor:
    """Decode into a preallocated contiguous bfloat16 [n, k] tensor."""
    if out.numel() != wt.n * wt.k or not out.is_contiguous() or out.element_size() != 2:
        raise ValueError("out must be a contiguous 16-bit tensor with n*k elements")
    s = wt.c_struct()
    _check(lib().w12_decode(ctypes.byref(s), out.data_ptr(), _stream_handle(wt.device)))
    return out


def decode(wt: W12Weight) -> torch.Tensor:
    """W12Weight -> bfloat16 W [n, k] (bit-exact)."""
    return decode_into(wt, torch.empty((wt.n, wt.k), dtype=torch.bfloat16, device=wt.device))


def _prep_x(x: torch.Tensor, k: int, device) -> torch.Tensor:
    """x as the kernels read it: 2-D, 16-bit (bfloat16 bits), contiguous, on the weights' device,
    with k columns.  A wrong x raises here, before anything is launched."""
    x = _bits16(x)
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D CUDA tensor")
    if x.device != device:
        raise ValueError(f"x is on {x.device}, the weights on {device}")
    if x.shape[1] != k:
        raise ValueError(f"x has {x.shape[1]} columns, the weights have k={k}")
    return x.contiguous()


def _check_out(out: torch.Tensor, shape, dtypes, device, what="out"):
    """A caller-provided output: contiguous, on the weights' device, of the given shape, and of
    one of the given dtypes (a wrong one would be written past its end or misread)."""
    if not isinstance(out, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if out.device != device:
        raise ValueError(f"{what} is on {out.device}, the weights on {device}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.dtype not in dtypes:
        raise ValueError(f"{what} has dtype {out.dtype}, expected one of {dtypes}")
    if not out.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _gemm_io(x, n, k, device, out, out_bf16):
    """Checked (x, out) of a GEMM call: out [m, n] float32, or bfloat16 (OUT_BF16: the float
    result rounded to nearest even), allocated when not given."""
    x = _prep_x(x, k, device)
    if out is None:
        dt = torch.bfloat16 if out_bf16 else torch.float32
        out = torch.empty((x.shape[0], n), dtype=dt, device=device)
    else:
        _check_out(out, (x.shape[0], n), (torch.float32, torch.bfloat16), device)
    return x, out


def _out_flag(out):
    """float32 outputs, or bfloat16 ones (OUT_BF16: the float result rounded to nearest even)."""
    return OUT_BF16 if out.dtype == torch.bfloat16 else 0


def gemm(x: torch.Tensor, wt: W12Weight, path: str | None = None, out: torch.Tensor | None = None,
         out_bf16: bool = False):
    """Exact pass: y = x W^T (fp32, or bfloat16 with ``out_bf16`` / a bfloat16 ``out``) with W
    read from its W12 record."""
    x, out = _gemm_io(x, wt.n, wt.k, wt.device, out, out_bf16)
    if x.shape[0] == 0:
        return out
    s = wt.c_struct()
    _check(lib().w12_gemm(x.data_ptr(), x.shape[0], ctypes.byref(s), out.data_ptr(),
                          _PATHS[path] | _out_flag(out), _stream_handle(x.device)))
    return out


def gemm_silu_mul(x: torch.Tensor, wt: W12Weight, path: str | None = None, out: torch.Tensor | None = None,
                  out_bf16: bool = False):
    """Exact pass on row-interleaved gate+up weights (interleave_rows) with SiLU(gate) * up
    applied where the outputs are stored: h [m, n / 2] float32 (or bfloat16)."""
    x, out = _gemm_io(x, wt.n // 2, wt.k, wt.device, out, out_bf16)
    if x.shape[0] == 0:
        return out
    s = wt.c_struct()
    _check(lib().w12_gemm_silu_mul(x.data_ptr(), x.shape[0], ctypes.byref(s), out.data_ptr(),
                                   _PATHS[path] | _out_flag(out), _stream_handle(x.device)))
    return out


def gemm_noalloc(x: torch.Tensor, wt: W12Weight, out: torch.Tensor, path: str | None = None):
    """gemm into a caller-provided ``out`` (float32 or bfloat16 [m, n]) through the allocation-free
    entry point: the library allocates nothing; its scratch is a fixed per-GPU array shared by
    every call on that GPU (calls overlapping in time on one GPU race)."""
    x, out = _gemm_io(x, wt.n, wt.k, wt.device, out, False)
    if x.shape[0] == 0:
        return out
    s = wt.c_struct()
    _check(lib().w12_gemm_noalloc(x.data_ptr(), x.shape[0], ctypes.byref(s), out.data_ptr(),
                                  _PATHS[path] | _out_flag(out), _stream_handle(x.device)))
    return out


def q8_gemm(x: torch.Tensor, wt: W12Weight, path: str | None = None, out: torch.Tensor | None = None,
            midpoint: bool = False, out_bf16: bool = False):
    """Q pass: y = x W_q^T with W_q the 8-bit view (B plane taken as 0, or as 8 with
    ``midpoint``), escapes exact; outputs as in gemm."""
    x, out = _gemm_io(x, wt.n, wt.k, wt.device, out, out_bf16)
    if x.shape[0] == 0:
        return out
    s = wt.c_struct()
    s.lo = None
    flags = _PATHS[path] | (Q8_MIDPOINT if midpoint else 0) | _out_flag(out)
    _check(lib().w12_q8_gemm(x.data_ptr(), x.shape[0], ctypes.byref(s), out.data_ptr(),
                             flags, _stream_handle(x.device)))
    return out


def _top1(fn, x, wt, lo, out, flags=0):
    x = _prep_x(x, wt.k, wt.device)
    m = x.shape[0]
    if out is None:
        out = (torch.empty(m, dtype=torch.int32, device=x.device),
               torch.empty(m, dtype=torch.float32, device=x.device))
    else:
        if len(out) != 2:
            raise ValueError("out must be a pair (index int32 [m], value float32 [m])")
        _check_out(out[0], (m,), (torch.int32,), wt.device, "out[0]")
        _check_out(out[1], (m,), (torch.float32,), wt.device, "out[1]")
    if m == 0:
        return out
    s = wt.c_struct()
    if not lo:
        s.lo = None
    _check(fn(x.data_ptr(), m, ctypes.byref(s), out[0].data_ptr(), out[1].data_ptr(), flags,
              _stream_handle(x.device)))
    return out


def q8_top1(x: torch.Tensor, wt: W12Weight, out=None, midpoint: bool = False):
    """Top-1 of the Q pass per row of x: (index int32 [m], value float32 [m]), no logits written;
    ``midpoint`` reads the dropped nibble as 8 as in q8_gemm."""
    return _top1(lib().w12_q8_top1, x, wt, False, out, Q8_MIDPOINT if midpoint else 0)


def gemm_top1(x: torch.Tensor, wt: W12Weight, out=None):
    """Top-1 of the exact pass per row of x: (index int32 [m], value float32 [m])."""
    return _top1(lib().w12_gemm_top1, x, wt, True, out)


class I8Copy:
    """The separate 8-bit Q-pass copy of a W12 record: int8 codes in the AE plane's storage order
    (padded_rows(n) * k) and a float32 scale per row; it shares ``rec``'s escape list."""

    def __init__(self, rec: W12Weight, q, scale):
        self.rec, self.q, self.scale = rec, q, scale
        self.n, self.k = rec.n, rec.k

    @property
    def device(self):
        return self.q.device

    def nbytes(self) -> int:
        return self.q.numel() + self.scale.numel() * 4

    def c_struct(self) -> _W12I8:
        return _W12I8(self.n, self.k, self.q.data_ptr(), self.scale.data_ptr())

    def to_numpy(self) -> dict:
        import numpy as np
        return dict(q_s=self.q.cpu().numpy().view(np.int8), scale=self.scale.cpu().numpy())


def i8_build(rec: W12Weight) -> I8Copy:
    """The 8-bit Q-pass copy of ``rec`` (per-row scale from the largest in-window magnitude / 127,
    codes rounded to nearest even, escaped slots 0), built on the device."""
    q = torch.empty(padded_rows(rec.n) * rec.k, dtype=torch.int8, device=rec.device)
    scale = torch.empty(rec.n, dtype=torch.float32, device=rec.device)
    cp = I8Copy(rec, q, scale)
    s, c = rec.c_struct(), cp.c_struct()
    _check(lib().w12_i8_build(ctypes.byref(s), ctypes.byref(c), _stream_handle(rec.device)))
    return cp


def i8_gemm(x: torch.Tensor, cp: I8Copy, path: str | None = None, out: torch.Tensor | None = None,
            out_bf16: bool = False):
    """Q pass on the 8-bit copy: y = x (s q)^T with the record's escapes exact; outputs as in gemm."""
    x, out = _gemm_io(x, cp.n, cp.k, cp.device, out, out_bf16)
    if x.shape[0] == 0:
        return out
    c, s = cp.c_struct(), cp.rec.c_struct()
    s.ae = None
    s.lo = None
    _check(lib().w12_i8_gemm(x.data_ptr(), x.shape[0], ctypes.byref(c), ctypes.byref(s), out.data_ptr(),
                             _PATHS[path] | _out_flag(out), _stream_handle(x.device)))
    return out


def i8_top1(x: torch.Tensor, cp: I8Copy, out=None):
    """Top-1 of the Q pass on the 8-bit copy per row of x: (index int32 [m], value float32 [m])."""
    c = cp.c_struct()
    return _top1(lambda xp, m, s, ip, vp, fl, st: lib().w12_i8_top1(xp, m, ctypes.byref(c), s, ip, vp, fl, st),
                 x, cp.rec, False, out)


class Bf16Tiles:
    """Dense bfloat16 W in the tiled storage order of the baseline kernels."""

    def __init__(self, n, k, data):
        self.n, self.k, self.data = int(n), int(k), data

    def nbytes(self) -> int:
        return self.data.numel() * 2


def bf16_tiles(w: torch.Tensor) -> Bf16Tiles:
    """bfloat16 W [n, k] (row-major, on the GPU) -> the baseline's tiled storage."""
    w = _bits16(w).contiguous()
    n, k = w.shape
    out = torch.empty(padded_rows(n) * k, dtype=torch.bfloat16, device=w.device)
    _check(lib().w12_bf16_to_tiles(w.data_ptr(), n, k, out.data_ptr(), _stream_handle(w.device)))
    return Bf16Tiles(n, k, out)


def bf16_gemm(x: torch.Tensor, wt: Bf16Tiles, path: str | None = None, out: torch.Tensor | None = None,
              out_bf16: bool = False):
    """Same-build dense baseline: y = x W^T with W plain bfloat16 (tiled storage); outputs as in
    gemm."""
    x, out = _gemm_io(x, wt.n, wt.k, wt.data.device, out, out_bf16)
    if x.shape[0] == 0:
        return out
    _check(lib().w12_bf16_gemm(x.data_ptr(), x.shape[0], wt.data.data_ptr(), wt.n, wt.k,
                               out.data_ptr(), _PATHS[path] | _out_flag(out), _stream_handle(x.device)))
    return out


def read_probe(buf: torch.Tensor, sink: torch.Tensor | None = None):
    """Stream every byte of ``buf`` through the read-bandwidth probe kernel."""
    if sink is None:
        sink = torch.zeros(4096, dtype=torch.int32, device=buf.device)
    _check(lib().w12_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                _stream_handle(buf.device)))
    return sink


def release_workspace(stream: "torch.cuda.Stream | None" = None, device=None):
    """Free the library's GEMM workspace of ``stream`` (default: the current stream of
    ``device``) on its device; waits for the stream's work first.  A later GEMM call on the
    stream allocates a new one."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    with torch.cuda.device(stream.device):
        _check(lib().w12_release_workspace(stream.cuda_stream))
