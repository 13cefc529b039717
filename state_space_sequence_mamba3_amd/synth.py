"""Seeded synthetic inputs for the Mamba-3 SSM recurrence.

This module draws random numbers and lays them out; it performs none of the
recurrence's arithmetic. Both the tests' CPU oracle and the GPU path consume
exactly the arrays made here (bf16 values travel as their uint16 bit patterns),
and the bench uses the device-side twin ``torch_scan_inputs``.

Distributions (one head dim P, state dim N, rank R, B/C groups G):
  x ~ N(0, 1)                       [b, L, H, R, P]
  dt = softplus(N(-2, 0.5))         [b, L, H]        (step, post-activation)
  lam = sigmoid(N(0, 1))            [b, L, H]        (trapezoid weight)
  theta ~ U(-pi, pi)                [b, L, H, N/2]   (frequency; angle = dt*theta)
  B, C ~ N(0, 1/N)                  [b, L, G, R, N]
  A = -exp(N(0, 0.5))               [H]  fp32
  D ~ N(0, 1)                       [H]  fp32
N(m, s) names mean and standard deviation. Layouts are rank-major: the R
columns of B_t, C_t (length N) and X_t (length P) are stored one after another. Arrays are drawn whole, in the
order A, D, x, dt, lam, theta, B, C, then (decode only) state, Bprev, xprev,
from numpy's PCG64 seeded with 1000 + config index unless a seed is given.
Token inputs are rounded to bf16 (round to nearest even, via fp32) for the bf16
configurations; A, D and states are fp32.

The block prologue / epilogue inputs (``block_inputs``) come from a generator
of their own: B and C biases ~ U(0.5, 1.5) [H, N] fp32 (positive, around the
all-ones initialisation of the biases), then a gate z ~ N(0, 1) shaped like x.
"""
from __future__ import annotations

import math

import numpy as np

# The five workloads. "chunk" is tokens per chunk (the rank-expanded tile of a
# chunk has chunk*R rows).
CONFIGS = {
    0: dict(name="tiny SISO scan fp32", kind="scan", batch=1, seqlen=256, nheads=4, headdim=16,
            dstate=16, rank=1, chunk=64, dtype="f32"),
    1: dict(name="SISO scan bf16 8x4096 H64 P64 N128", kind="scan", batch=8, seqlen=4096, nheads=64,
            headdim=64, dstate=128, rank=1, chunk=64, dtype="bf16"),
    2: dict(name="MIMO scan bf16 8x4096 H64 P64 N64 R4", kind="scan", batch=8, seqlen=4096, nheads=64,
            headdim=64, dstate=64, rank=4, chunk=64, dtype="bf16"),
    3: dict(name="MIMO decode bf16 batch256 H64 P64 N64 R4", kind="decode", batch=256, seqlen=1,
            nheads=64, headdim=64, dstate=64, rank=4, chunk=0, dtype="bf16", steps=1000, ring=64),
    4: dict(name="packed MIMO scan bf16 65536 tok H64 P64 N128 R4", kind="scan", batch=1, seqlen=65536,
            nheads=64, headdim=64, dstate=128, rank=4, chunk=128, dtype="bf16", packed=True, nseq=8,
            len_lo=1024, len_hi=16384),
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float array -> bf16 bit patterns (uint16), round to nearest even via fp32."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def packed_lengths(rng: np.random.Generator, nseq: int, total: int, lo: int, hi: int) -> np.ndarray:
    """Lengths drawn from U(lo, hi), scaled to sum to ``total``: floor for all
    but the last, which takes the remainder."""
    u = rng.uniform(lo, hi, size=nseq)
    ln = np.floor(u * total / u.sum()).astype(np.int64)
    ln[-1] = total - ln[:-1].sum()
    return ln


def _normal(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std) + np.float32(mean))


def _softplus(v):
    v = v.astype(np.float64)
    return np.where(v > 20, v, np.log1p(np.exp(np.minimum(v, 20))))


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v.astype(np.float64)))


def _tok(a, dtype):
    return bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def scan_inputs(cfg: int | dict, seed: int | None = None, **over) -> dict:
    """Inputs of a scan workload as numpy arrays in the library's layouts.

    ``cfg`` is a config index or dict; keyword overrides replace sizes (e.g.
    ``batch=2, seqlen=300``). Returns keys x, dt, lam, theta, B, C (uint16 bf16
    bits or float32), A, D (float32), cu_seqlens (int32, packed only), meta.
    """
    c = dict(CONFIGS[cfg]) if isinstance(cfg, int) else dict(cfg)
    c.update(over)
    if seed is None:
        seed = 1000 + (cfg if isinstance(cfg, int) else 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    b, L, H, P, N, R = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    dt_ = c["dtype"]
    A = (-np.exp(_normal(rng, (H,), 0.0, 0.5).astype(np.float64))).astype(np.float32)
    D = _normal(rng, (H,)).astype(np.float32)
    out = dict(A=A, D=D)
    out["x"] = _tok(_normal(rng, (b, L, H, R, P)), dt_)
    out["dt"] = _tok(_softplus(_normal(rng, (b, L, H), -2.0, 0.5)), dt_)
    out["lam"] = _tok(_sigmoid(_normal(rng, (b, L, H))), dt_)
    out["theta"] = _tok(rng.uniform(-math.pi, math.pi, size=(b, L, H, N // 2)).astype(np.float32), dt_)
    out["B"] = _tok(_normal(rng, (b, L, G, R, N), 0.0, 1.0 / math.sqrt(N)), dt_)
    out["C"] = _tok(_normal(rng, (b, L, G, R, N), 0.0, 1.0 / math.sqrt(N)), dt_)
    if c.get("packed"):
        if b != 1:
            raise ValueError("packed workloads have batch 1")
        ln = packed_lengths(rng, c["nseq"], L, c["len_lo"], c["len_hi"])
        out["cu_seqlens"] = np.concatenate([[0], np.cumsum(ln)]).astype(np.int32)
    out["meta"] = dict(c, ngroups=G, seed=seed)
    return out


def resume_inputs(inp: dict, seed: int) -> dict:
    """Adds a state h_in [S,H,N,P] ~ N(0,1) fp32 and a previous token
    (Bprev [S,G,R,N], xprev [S,H,R,P]) drawn like a token, for resume tests."""
    m = inp["meta"]
    rng = np.random.Generator(np.random.PCG64(seed))
    S = len(inp["cu_seqlens"]) - 1 if inp.get("cu_seqlens") is not None else m["batch"]
    H, P, N, R, G = m["nheads"], m["headdim"], m["dstate"], m["rank"], m["ngroups"]
    out = dict(inp)
    out["h_in"] = _normal(rng, (S, H, N, P)).astype(np.float32)
    out["Bprev"] = _tok(_normal(rng, (S, G, R, N), 0.0, 1.0 / math.sqrt(N)), m["dtype"])
    out["xprev"] = _tok(_normal(rng, (S, H, R, P)), m["dtype"])
    return out


def block_inputs(inp: dict, seed: int, norm: bool = True, B_bias: bool = True, C_bias: bool = True,
                 gate: bool = True, eps: float = 1e-5) -> dict:
    """Adds the inputs of the fused block prologue / epilogue to a scan or
    decode input set: the B/C RMS-norm switch and its eps, per-head B and C
    biases [H, N] fp32 ~ U[0.5, 1.5] (positive, around the all-ones
    initialisation), and a gate z shaped like x (~N(0, 1), token dtype)."""
    m = inp["meta"]
    rng = np.random.Generator(np.random.PCG64(seed))
    H, N = m["nheads"], m["dstate"]
    out = dict(inp)
    out["bc_norm"], out["bc_eps"] = bool(norm), float(eps)
    if B_bias:
        out["B_bias"] = rng.uniform(0.5, 1.5, size=(H, N)).astype(np.float32)
    if C_bias:
        out["C_bias"] = rng.uniform(0.5, 1.5, size=(H, N)).astype(np.float32)
    if gate:
        out["z"] = _tok(_normal(rng, inp["x"].shape), m["dtype"])
    return out


def variant_inputs(inp: dict, seed: int, A_tok: bool = True, lam_fixed: float | None = None,
                   theta_groups: int | None = None) -> dict:
    """The variants: a per-token decay rate A_t ~ -exp(N(0, 0.5)) shaped like
    dt (token dtype), replacing A; with lam_fixed, no lam array; with
    theta_groups, Gth angle rows per token (the rows of heads 0, H/Gth, ...),
    each shared by H/Gth consecutive heads."""
    m = inp["meta"]
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(inp)
    if theta_groups is not None:
        H = inp["theta"].shape[-2]
        out["theta"] = np.ascontiguousarray(inp["theta"][..., ::H // theta_groups, :])
    if A_tok:
        out["A_tok"] = _tok(-np.exp(_normal(rng, inp["dt"].shape, 0.0, 0.5)), m["dtype"])
    if lam_fixed is not None:
        out["lam"], out["lam_fixed"] = None, float(lam_fixed)
    return out


def grad_inputs(inp: dict, seed: int, dh_out: bool = True) -> dict:
    """Output gradients for a backward test: dy ~ N(0, 1) shaped like x (token
    dtype) and, if asked, dh_out ~ N(0, 1) [S, H, N, P] fp32."""
    m = inp["meta"]
    rng = np.random.Generator(np.random.PCG64(seed))
    S = len(inp["cu_seqlens"]) - 1 if inp.get("cu_seqlens") is not None else m["batch"]
    out = dict(dy=_tok(_normal(rng, inp["x"].shape), m["dtype"]))
    if dh_out:
        out["dh_out"] = _normal(rng, (S, m["nheads"], m["dstate"], m["headdim"])).astype(np.float32)
    return out


def decode_inputs(cfg: int | dict = 3, seed: int | None = None, ring: int = 1, **over) -> dict:
    """Decode workload: ``ring`` token-input sets (each like one token of a
    scan, leading axis ring), a previous token, and an fp32 state ~ N(0,1).
    Returns x [ring,b,H,R,P], dt/lam [ring,b,H], theta [ring,b,H,N/2],
    B/C [ring,b,G,R,N], A, D, h [b,H,N,P], Bprev [b,G,R,N], xprev [b,H,R,P]."""
    c = dict(CONFIGS[cfg]) if isinstance(cfg, int) else dict(cfg)
    c.update(over)
    if seed is None:
        seed = 1000 + (cfg if isinstance(cfg, int) else 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    b, H, P, N, R = c["batch"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    dt_ = c["dtype"]
    A = (-np.exp(_normal(rng, (H,), 0.0, 0.5).astype(np.float64))).astype(np.float32)
    D = _normal(rng, (H,)).astype(np.float32)
    out = dict(A=A, D=D)
    out["x"] = _tok(_normal(rng, (ring, b, H, R, P)), dt_)
    out["dt"] = _tok(_softplus(_normal(rng, (ring, b, H), -2.0, 0.5)), dt_)
    out["lam"] = _tok(_sigmoid(_normal(rng, (ring, b, H))), dt_)
    out["theta"] = _tok(rng.uniform(-math.pi, math.pi, size=(ring, b, H, N // 2)).astype(np.float32), dt_)
    out["B"] = _tok(_normal(rng, (ring, b, G, R, N), 0.0, 1.0 / math.sqrt(N)), dt_)
    out["C"] = _tok(_normal(rng, (ring, b, G, R, N), 0.0, 1.0 / math.sqrt(N)), dt_)
    out["h"] = _normal(rng, (b, H, N, P)).astype(np.float32)
    out["Bprev"] = _tok(_normal(rng, (b, G, R, N), 0.0, 1.0 / math.sqrt(N)), dt_)
    out["xprev"] = _tok(_normal(rng, (b, H, R, P)), dt_)
    out["meta"] = dict(c, ngroups=G, seed=seed)
    return out


def torch_scan_inputs(cfg: int | dict, device, seed: int = 0, **over) -> dict:
    """Device-side twin of ``scan_inputs`` for the bench (same shapes and
    distributions, torch's generator, so not bit-identical to numpy's)."""
    import torch

    c = dict(CONFIGS[cfg]) if isinstance(cfg, int) else dict(cfg)
    c.update(over)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    b, L, H, P, N, R = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    td = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32

    def nrm(shape, mean=0.0, std=1.0):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std + mean

    out = dict(A=-torch.exp(nrm((H,), 0.0, 0.5)), D=nrm((H,)))
    out["x"] = nrm((b, L, H, R, P)).to(td)
    out["dt"] = torch.nn.functional.softplus(nrm((b, L, H), -2.0, 0.5)).to(td)
    out["lam"] = torch.sigmoid(nrm((b, L, H))).to(td)
    out["theta"] = ((torch.rand((b, L, H, N // 2), generator=g, device=device) * 2 - 1) * math.pi).to(td)
    out["B"] = nrm((b, L, G, R, N), 0.0, 1.0 / math.sqrt(N)).to(td)
    out["C"] = nrm((b, L, G, R, N), 0.0, 1.0 / math.sqrt(N)).to(td)
    if c.get("packed"):
        rng = np.random.Generator(np.random.PCG64(1000 + seed))
        ln = packed_lengths(rng, c["nseq"], L, c["len_lo"], c["len_hi"])
        out["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(ln)]), dtype=torch.int32, device=device)
    out["meta"] = dict(c, ngroups=G, seed=seed)
    return out


def torch_block_inputs(d: dict, device, seed: int = 0) -> dict:
    """Device-side twin of ``block_inputs`` (norm on, both biases, gate)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    H, N = d["A"].shape[0], d["B"].shape[-1]
    out = dict(d)
    out["bc_norm"], out["bc_eps"] = True, 1e-5
    out["B_bias"] = torch.rand((H, N), generator=g, device=device) + 0.5
    out["C_bias"] = torch.rand((H, N), generator=g, device=device) + 0.5
    out["z"] = torch.randn(d["x"].shape, generator=g, device=device, dtype=torch.float32).to(d["x"].dtype)
    return out
