"""Helpers of the GPU parity tests: device upload of the seeded inputs and the
tolerance metric (per (sequence, head) slab: max |gpu - oracle| / max |oracle|,
the maximum over slabs must stay within the tolerance)."""
import sys

import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2

TOKEN_KEYS = ("x", "dt", "lam", "theta", "B", "C", "Bprev", "xprev")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a, dev):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def from_dev(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def upload(inp, dev):
    out = {}
    for k, v in inp.items():
        if k == "meta":
            continue
        out[k] = to_dev(v, dev) if isinstance(v, np.ndarray) else v
    return out


def slab_relerr(g, o, axis_token=1):
    """g, o: [S, L, H, ...] or [L, ...] arrays; returns max over (s, h) slabs of
    max|g-o| / max|o| (slab = all tokens and trailing dims of one (s, h))."""
    d = np.abs(g - o)
    if g.ndim >= 4:
        # [b, L, H, P, R] -> reduce over L and trailing dims
        red = tuple(i for i in range(g.ndim) if i not in (0, 2))
        num = d.max(axis=red)
        den = np.abs(o).max(axis=red)
    else:
        num, den = d.max(), np.abs(o).max()
    return float(np.max(num / np.maximum(den, 1e-30)))


def state_relerr(g, o):
    """States [S, H, N, P]: per (s, h) slab."""
    num = np.abs(g - o).max(axis=(2, 3))
    den = np.abs(o).max(axis=(2, 3))
    return float(np.max(num / np.maximum(den, 1e-30)))
