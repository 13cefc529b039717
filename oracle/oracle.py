"""ctypes front end of the fp64 CPU oracle (``m3_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``. The product path (the HIP library
and its binding) never imports, links or calls anything here, and this module
imports nothing from the product package.

All arrays use the flat token axis (padded batches are flattened to
``batch*seqlen`` tokens, sequence ``s`` starting at ``s*seqlen``):
``x [T,H,R,P]``, ``dt, lam [T,H]``, ``theta [T,H,N/2]`` (or ``[T,Gth,N/2]``, one angle row shared by each group of H/Gth heads), ``B, C [T,G,R,N]``,
``A, D [H]``, ``h_in [S,H,N,P]``, ``Bprev [S,G,R,N]``, ``xprev [S,H,R,P]``
(rank-major: the R columns of B_t, X_t are stored one after another), and the
optional block prologue/epilogue: ``B_bias, C_bias [H,N]``, ``z`` (like x),
``bc_norm`` (bool) and ``bc_eps``; and the variants: ``A_tok`` (like dt: a
per-token decay rate replacing A) and ``lam`` = None with ``lam_fixed``.
Token inputs may be float64, float32 or uint16 (bf16 bit patterns); they are
converted exactly to double inside the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB = os.path.join(_HERE, "libm3oracle.so")

F64, F32, BF16 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Wextra", "-Wno-unused-parameter",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Args(ctypes.Structure):
    _fields_ = [
        ("nseq", ctypes.c_int32),
        ("seq_start", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
        ("H", ctypes.c_int32), ("G", ctypes.c_int32), ("P", ctypes.c_int32),
        ("N", ctypes.c_int32), ("R", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("lam", ctypes.c_void_p),
        ("theta", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("h_in", ctypes.c_void_p),
        ("Bprev", ctypes.c_void_p), ("xprev", ctypes.c_void_p),
        ("B_bias", ctypes.c_void_p), ("C_bias", ctypes.c_void_p), ("z", ctypes.c_void_p),
        ("bc_norm", ctypes.c_int32), ("bc_eps", ctypes.c_double),
        ("A_tok", ctypes.c_void_p), ("lam_fixed", ctypes.c_double), ("th_groups", ctypes.c_int32),
    ]


class _Grads(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in (
        "dy", "dh_out", "dx", "ddt", "dlam", "dtheta", "dB", "dC", "dA", "dD", "dh_in", "dBprev", "dxprev",
        "dB_bias", "dC_bias", "dz", "dA_tok")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        l = ctypes.CDLL(_LIB)
        l.m3o_scan.argtypes = [ctypes.POINTER(_Args), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        l.m3o_scan_slab.argtypes = [ctypes.POINTER(_Args), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
        l.m3o_decode.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        l.m3o_max_threads.restype = ctypes.c_int
        l.m3o_scan_chunked.argtypes = [ctypes.POINTER(_Args), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        l.m3o_scan_bwd.argtypes = [ctypes.POINTER(_Args), ctypes.POINTER(_Grads), ctypes.c_int]
        _lib = l
    return _lib


def max_threads() -> int:
    return lib().m3o_max_threads()


def _tag(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


class _Pack:
    """Holds contiguous copies alive for the duration of a call."""

    def __init__(self, inp: dict, seq_start, seq_len):
        keep = {}
        tag = _tag(inp["x"])
        for k in ("x", "dt", "lam", "theta", "B", "C", "Bprev", "xprev", "z", "A_tok"):
            v = inp.get(k)
            if v is not None:
                v = np.ascontiguousarray(v)
                if _tag(v) != tag:
                    raise TypeError(f"{k}: all token inputs must share one dtype")
            keep[k] = v
        for k in ("A", "D", "h_in", "B_bias", "C_bias"):
            v = inp.get(k)
            keep[k] = None if v is None else np.ascontiguousarray(v, dtype=np.float64)
        x = keep["x"]
        B = keep["B"]
        H, R, P = x.shape[-3], x.shape[-2], x.shape[-1]
        G, N = B.shape[-3], B.shape[-1]
        self.Gth = keep["theta"].shape[-2]   # angle rows per token: H, or fewer shared by groups of heads
        keep["seq_start"] = np.ascontiguousarray(seq_start, dtype=np.int64)
        keep["seq_len"] = np.ascontiguousarray(seq_len, dtype=np.int64)
        self.keep = keep
        self.H, self.G, self.P, self.N, self.R = H, G, P, N, R
        self.nseq = len(keep["seq_len"])
        self.args = _Args(self.nseq, _ptr(keep["seq_start"]), _ptr(keep["seq_len"]),
                          H, G, P, N, R, tag,
                          _ptr(keep["x"]), _ptr(keep["dt"]), _ptr(keep["lam"]), _ptr(keep["theta"]),
                          _ptr(keep["B"]), _ptr(keep["C"]), _ptr(keep["A"]), _ptr(keep["D"]),
                          _ptr(keep["h_in"]), _ptr(keep["Bprev"]), _ptr(keep["xprev"]),
                          _ptr(keep["B_bias"]), _ptr(keep["C_bias"]), _ptr(keep["z"]),
                          1 if inp.get("bc_norm") else 0, float(inp.get("bc_eps", 0.0)),
                          _ptr(keep["A_tok"]), float(inp.get("lam_fixed", 0.0)), self.Gth)


def flatten(inp: dict) -> tuple[dict, np.ndarray, np.ndarray]:
    """[batch, L, ...] inputs -> flat token axis + sequence table. Packed
    inputs (key ``cu_seqlens``, batch 1) take their table from cu_seqlens."""
    out = dict(inp)
    b, L = inp["x"].shape[0], inp["x"].shape[1]
    for k in ("x", "dt", "lam", "theta", "B", "C", "z", "A_tok"):
        if inp.get(k) is not None:
            out[k] = inp[k].reshape((b * L,) + inp[k].shape[2:])
    if inp.get("cu_seqlens") is not None:
        if b != 1:
            raise ValueError("packed inputs have batch 1")
        cu = np.asarray(inp["cu_seqlens"], dtype=np.int64)
        return out, cu[:-1].copy(), np.diff(cu)
    return out, np.arange(b, dtype=np.int64) * L, np.full(b, L, dtype=np.int64)


def scan(inp: dict, form: int = 1, nthreads: int = 0, want_state: bool = True):
    """Whole scan. Returns (y [same leading shape as x], h_out [S,H,N,P])."""
    flat, st, ln = flatten(inp)
    pk = _Pack(flat, st, ln)
    T = flat["x"].shape[0]
    y = np.zeros((T, pk.H, pk.R, pk.P), dtype=np.float64)
    h = np.zeros((pk.nseq, pk.H, pk.N, pk.P), dtype=np.float64) if want_state else None
    rc = lib().m3o_scan(ctypes.byref(pk.args), form, y.ctypes.data, _ptr(h), nthreads)
    if rc:
        raise ValueError("oracle rejected its arguments")
    return y.reshape(inp["x"].shape), h


def scan_chunked(inp: dict, chunk: int, nthreads: int = 0, want_state: bool = True):
    """Whole scan in the chunked SSD form (O3C) with chunks of `chunk` tokens.
    Returns (y [same leading shape as x], h_out [S,H,N,P])."""
    flat, st, ln = flatten(inp)
    pk = _Pack(flat, st, ln)
    T = flat["x"].shape[0]
    y = np.zeros((T, pk.H, pk.R, pk.P), dtype=np.float64)
    h = np.zeros((pk.nseq, pk.H, pk.N, pk.P), dtype=np.float64) if want_state else None
    rc = lib().m3o_scan_chunked(ctypes.byref(pk.args), int(chunk), y.ctypes.data, _ptr(h), nthreads)
    if rc:
        raise ValueError("oracle rejected its arguments")
    return y.reshape(inp["x"].shape), h


def scan_slab(inp: dict, s: int, h: int, form: int = 1, want_state: bool = True):
    """One (sequence, head) slab. Returns (y [len,R,P], h_out [N,P] or None)."""
    flat, st, ln = flatten(inp)
    pk = _Pack(flat, st, ln)
    y = np.zeros((int(ln[s]), pk.R, pk.P), dtype=np.float64)
    hs = np.zeros((pk.N, pk.P), dtype=np.float64) if want_state else None
    rc = lib().m3o_scan_slab(ctypes.byref(pk.args), form, s, h, y.ctypes.data, _ptr(hs))
    if rc:
        raise ValueError("oracle rejected its arguments")
    return y, hs


def decode(inp: dict, h: np.ndarray, nthreads: int = 0):
    """One decode step. inp token arrays have a leading batch axis (no L).
    Returns (y [batch,H,R,P], h_new [batch,H,N,P]) in float64."""
    b = inp["x"].shape[0]
    pk = _Pack(inp, np.arange(b, dtype=np.int64), np.ones(b, dtype=np.int64))
    hio = np.array(h, dtype=np.float64, copy=True, order="C")
    y = np.zeros((b, pk.H, pk.R, pk.P), dtype=np.float64)
    rc = lib().m3o_decode(ctypes.byref(pk.args), hio.ctypes.data, y.ctypes.data, nthreads)
    if rc:
        raise ValueError("oracle rejected its arguments")
    return y, hio


def scan_bwd(inp: dict, dy: np.ndarray, dh_out: np.ndarray | None = None, nthreads: int = 0) -> dict:
    """Gradient of the whole scan (OB, reverse mode in fp64): given dL/dy
    (shaped like x) and dL/dh_out ([S,H,N,P] or None), returns float64 arrays
    dx, ddt, dlam, dtheta, dB, dC (shaped like the inputs), dA, dD [H], dh_in
    [S,H,N,P], and, where the inputs have them, dBprev, dxprev, dB_bias,
    dC_bias, dz."""
    flat, st, ln = flatten(inp)
    pk = _Pack(flat, st, ln)
    T = flat["x"].shape[0]
    H, G, P, N, R, S = pk.H, pk.G, pk.P, pk.N, pk.R, pk.nseq
    dyf = np.ascontiguousarray(np.asarray(dy, dtype=np.float64).reshape(T, H, R, P))
    dho = None if dh_out is None else np.ascontiguousarray(dh_out, dtype=np.float64)
    out = dict(dx=np.zeros((T, H, R, P)), ddt=np.zeros((T, H)), dtheta=np.zeros((T, pk.Gth, N // 2)),
               dB=np.zeros((T, G, R, N)), dC=np.zeros((T, G, R, N)), dD=np.zeros(H), dh_in=np.zeros((S, H, N, P)))
    if inp.get("lam") is not None:
        out["dlam"] = np.zeros((T, H))
    if inp.get("A_tok") is not None:
        out["dA_tok"] = np.zeros((T, H))
    else:
        out["dA"] = np.zeros(H)
    if inp.get("Bprev") is not None:
        out["dBprev"], out["dxprev"] = np.zeros((S, G, R, N)), np.zeros((S, H, R, P))
    if inp.get("B_bias") is not None:
        out["dB_bias"] = np.zeros((H, N))
    if inp.get("C_bias") is not None:
        out["dC_bias"] = np.zeros((H, N))
    if inp.get("z") is not None:
        out["dz"] = np.zeros((T, H, R, P))
    g = _Grads(dyf.ctypes.data, _ptr(dho), *[_ptr(out.get(k)) for k in (
        "dx", "ddt", "dlam", "dtheta", "dB", "dC", "dA", "dD", "dh_in", "dBprev", "dxprev", "dB_bias", "dC_bias", "dz",
        "dA_tok")])
    if lib().m3o_scan_bwd(ctypes.byref(pk.args), ctypes.byref(g), nthreads):
        raise ValueError("oracle rejected its arguments")
    for k, src in (("dx", "x"), ("ddt", "dt"), ("dlam", "dt"), ("dtheta", "theta"), ("dB", "B"), ("dC", "C"),
                   ("dA_tok", "dt")):
        if k in out:
            out[k] = out[k].reshape(inp[src].shape)
    if "dz" in out:
        out["dz"] = out["dz"].reshape(inp["z"].shape)
    return out

