"""GPU parity of the scan's backward (mamba3_scan_bwd) against the fp64
gradient oracle OB, itself pinned by finite differences of the forward.

Metric: per gradient array and per slab, as for the forward: a slab is one
(sequence, head) of a token-indexed gradient (one (sequence, group) for dB, dC
and a shared angle row's dtheta; packed sequences are split at cu_seqlens) and
one (sequence, head) or (sequence, group) of dh_in, dBprev, dxprev. Per slab
max |gpu - oracle| / max |oracle|; the maximum over slabs is held to 1e-4 for
fp32 token inputs and 2e-2 for bf16 ones (gradients returned in bf16). The
per-head parameter gradients (dA, dD, the bias gradients) are each one sum over
every sequence and token of a head, whose relative error is set by cancellation
in that sum rather than by any slab of the kernel's work; they are held to the
same bounds over the whole array (all heads). A slab whose oracle gradient
vanishes (max below 1e-9) is held to max |gpu| < 1e-6. All calls go through the
C ABI."""
import numpy as np
import pytest

import state_space_sequence_mamba3_amd as m3
from state_space_sequence_mamba3_amd import synth
from tests.gpu_util import TOL_BF16, TOL_F32, device, from_dev, note, upload

pytestmark = pytest.mark.gpu

KEYS = ("dx", "ddt", "dlam", "dtheta", "dB", "dC", "dA", "dD", "dh_in", "dBprev", "dxprev", "dB_bias", "dC_bias", "dz",
        "dA_tok")


def run_bwd(inp, gr):
    import torch
    d = upload(inp, device())
    dy = upload(gr, device())
    g = m3.mamba3_scan_bwd(d["x"], d["dt"], d.get("lam"), d["theta"], d["B"], d["C"], d.get("A"), d.get("D"),
                           dy=dy["dy"], dh_out=dy.get("dh_out"), h_in=d.get("h_in"), Bprev=d.get("Bprev"),
                           xprev=d.get("xprev"), cu_seqlens=d.get("cu_seqlens"), B_bias=d.get("B_bias"),
                           C_bias=d.get("C_bias"), z=d.get("z"), bc_norm=d.get("bc_norm", False),
                           bc_eps=d.get("bc_eps", 1e-5), A_tok=d.get("A_tok"), lam_fixed=d.get("lam_fixed", 0.5))
    torch.cuda.synchronize()
    return {k: from_dev(v) for k, v in g.items()}


TOKEN_KEYS = ("dx", "ddt", "dlam", "dtheta", "dB", "dC", "dz", "dA_tok")   # [batch, L, head or group, ...]
STATE_KEYS = ("dh_in", "dBprev", "dxprev")                                    # [sequence, head or group, ...]


def slabs(k, a, cu):
    """The slabs of gradient k (array a in the oracle's shape), as a list of arrays."""
    if k in TOKEN_KEYS:
        seqs = ([a[0, int(cu[i]):int(cu[i + 1])] for i in range(len(cu) - 1)] if cu is not None
                else [a[i] for i in range(a.shape[0])])
        return [q[:, j] for q in seqs for j in range(a.shape[2]) if q.shape[0] > 0]
    if k in STATE_KEYS:
        return [a[i, j] for i in range(a.shape[0]) for j in range(a.shape[1])]
    return [a]                                                                  # dA, dD, biases: whole array


def slab_err(k, a, b, cu):
    worst = 0.0
    for ga, ob in zip(slabs(k, a, cu), slabs(k, b, cu)):
        den = np.abs(ob).max()
        if den < 1e-9:
            # an exactly vanishing gradient (e.g. the angle's with a zero state): the kernel's
            # value is rounding residue of terms that cancel, held to an absolute bound
            e = 0.0 if np.abs(ga).max() < 1e-6 else float("inf")
        else:
            e = float(np.abs(ga - ob).max() / den)
        worst = max(worst, e)
    return worst


def compare(oracle, inp, gr, tol, label):
    gg = run_bwd(inp, gr)
    go = oracle.scan_bwd({k: v for k, v in inp.items() if k != "meta"}, gr["dy"].astype(np.float64)
                         if gr["dy"].dtype != np.uint16 else synth.bits_to_f32(gr["dy"]).astype(np.float64),
                         gr.get("dh_out"))
    worst = {}
    cu = inp.get("cu_seqlens")
    for k in KEYS:
        if k not in go:
            continue
        worst[k] = slab_err(k, gg[k].reshape(go[k].shape), go[k], cu)
    note(f"{label}: " + " ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    bad = {k: v for k, v in worst.items() if not v < tol}
    assert not bad, bad
    return gg


F32_SHAPES = [
    dict(batch=2, seqlen=70, nheads=2, headdim=16, dstate=16, rank=1),
    dict(batch=1, seqlen=45, nheads=2, headdim=16, dstate=32, rank=4),
    dict(batch=2, seqlen=33, nheads=4, headdim=8, dstate=8, rank=2, ngroups=2),
    dict(batch=1, seqlen=20, nheads=2, headdim=64, dstate=64, rank=4, ngroups=1),
    dict(batch=3, seqlen=1, nheads=2, headdim=16, dstate=16, rank=2),
]


@pytest.mark.parametrize("shape", F32_SHAPES)
@pytest.mark.parametrize("extras", ["plain", "resume", "block"])
def test_bwd_fp32(oracle, shape, extras):
    cfg = dict(synth.CONFIGS[0], **shape)
    inp = synth.scan_inputs(cfg, seed=91)
    if extras in ("resume", "block"):
        inp = synth.resume_inputs(inp, seed=92)
    if extras == "block":
        inp = synth.block_inputs(inp, seed=93)
    gr = synth.grad_inputs(inp, seed=94, dh_out=extras != "plain")
    compare(oracle, inp, gr, TOL_F32, f"bwd f32 {shape} {extras}")


def test_bwd_fp32_packed(oracle):
    cfg = dict(synth.CONFIGS[0], batch=1, seqlen=150, nheads=2, headdim=16, dstate=16, rank=2)
    inp = synth.scan_inputs(cfg, seed=95)
    inp["cu_seqlens"] = np.array([0, 40, 40, 41, 100, 150, 150], dtype=np.int32)
    inp = synth.block_inputs(synth.resume_inputs(inp, seed=96), seed=97)
    gr = synth.grad_inputs(inp, seed=98)
    gg = compare(oracle, inp, gr, TOL_F32, "bwd f32 packed")
    # an empty sequence passes dh_out through to dh_in and gets no dBprev, dxprev
    assert np.array_equal(gg["dh_in"][1], gr["dh_out"][1].astype(np.float64))
    assert not gg["dBprev"][1].any() and not gg["dxprev"][1].any()


@pytest.mark.parametrize("name,spec", [
    ("siso_n128", dict(cfg=1, batch=1, seqlen=90, nheads=2)),
    ("mimo_n64_r4", dict(cfg=2, batch=1, seqlen=70, nheads=2)),
    ("mimo_n128_r4_g1", dict(cfg=4, batch=1, seqlen=50, nheads=2, packed=False, ngroups=1)),
    ("siso_n64", dict(cfg=1, batch=1, seqlen=75, nheads=2, dstate=64)),
    ("r2_n128", dict(cfg=2, batch=1, seqlen=75, nheads=2, dstate=128, rank=2)),
    ("r2_n64", dict(cfg=2, batch=2, seqlen=70, nheads=2, rank=2)),
])
@pytest.mark.parametrize("block", [False, True])
def test_bwd_bf16(oracle, name, spec, block):
    spec = dict(spec)
    cfg = spec.pop("cfg")
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=101, **spec), seed=102)
    if block:
        inp = synth.block_inputs(inp, seed=103)
    gr = synth.grad_inputs(inp, seed=104)
    compare(oracle, inp, gr, TOL_BF16, f"bwd bf16 {name} block={block}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [dict(A_tok=True), dict(A_tok=True, lam_fixed=0.5), dict(A_tok=False, lam_fixed=1.0),
                                     dict(A_tok=False, theta_groups=1)])
def test_bwd_variants(oracle, dtype, variant):
    """Per-token decay rate (per-token dA), fixed trapezoid weights (no dlam) and one angle row
    shared by the heads (dtheta sums their shares)."""
    cfg = dict(synth.CONFIGS[1], dtype=dtype, batch=1, seqlen=70, nheads=2)
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=111), seed=112)
    inp = synth.variant_inputs(inp, seed=113, **variant)
    if variant["A_tok"]:
        inp["A"] = None
    gr = synth.grad_inputs(inp, seed=114)
    compare(oracle, inp, gr, TOL_F32 if dtype == "f32" else TOL_BF16, f"bwd {dtype} variant {variant}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_shared_angles_grouped(oracle, dtype):
    """Two angle rows shared by pairs of heads, with B/C groups and a resumed state."""
    cfg = dict(synth.CONFIGS[1], dtype=dtype, batch=2, seqlen=45, nheads=4, ngroups=2)
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=115), seed=116)
    inp = synth.variant_inputs(inp, seed=117, A_tok=False, theta_groups=2)
    gr = synth.grad_inputs(inp, seed=118)
    compare(oracle, inp, gr, TOL_F32 if dtype == "f32" else TOL_BF16, f"bwd {dtype} shared angles, G=2")


def test_bwd_deterministic():
    cfg = dict(synth.CONFIGS[0], batch=2, seqlen=100, nheads=4, headdim=16, dstate=16, rank=2, ngroups=2)
    inp = synth.block_inputs(synth.resume_inputs(synth.scan_inputs(cfg, seed=105), seed=106), seed=107)
    gr = synth.grad_inputs(inp, seed=108)
    note("bwd determinism")
    a, b = run_bwd(inp, gr), run_bwd(inp, gr)
    for k in a:
        assert a[k].tobytes() == b[k].tobytes(), k


def test_bwd_deterministic_bf16_state_pass():
    """The bf16 MFMA backward of a padded SISO batch, whose chunk states come from the state-only
    forward scan: bitwise equal gradients on two runs."""
    cfg = dict(synth.CONFIGS[1], batch=2, seqlen=150, nheads=4)
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=121), seed=122)
    gr = synth.grad_inputs(inp, seed=123)
    note("bwd determinism, bf16 with the state pass")
    a, b = run_bwd(inp, gr), run_bwd(inp, gr)
    for k in a:
        assert a[k].tobytes() == b[k].tobytes(), k


@pytest.mark.parametrize("cfg", [1, 2])
def test_bwd_state_sources_agree(cfg):
    """Chunk states from the state-only forward scan (a padded batch) and from the backward
    kernel's own forward walk (the same two sequences as a packed batch) give the same gradients
    up to rounding: within 2^-6 of the other path's largest magnitude, two bf16 steps (the paths
    round the chunk states' bf16 operands differently, and most gradients are stored in bf16).
    A misplaced or missing chunk state moves them by far more."""
    c = dict(synth.CONFIGS[cfg], batch=2, seqlen=150, nheads=4)
    inp = synth.scan_inputs(c, seed=126 + cfg)
    gr = synth.grad_inputs(inp, seed=128 + cfg)
    tok = ("x", "dt", "lam", "theta", "B", "C")
    pk = {k: (v.reshape((1, 300) + v.shape[2:]) if k in tok else v) for k, v in inp.items()}
    pk["cu_seqlens"] = np.array([0, 150, 300], dtype=np.int32)
    gpk = dict(gr, dy=gr["dy"].reshape((1, 300) + gr["dy"].shape[2:]))
    note(f"bwd state sources, config {cfg}: padded (state pass) against packed (forward walk)")
    a, b = run_bwd(inp, gr), run_bwd(pk, gpk)
    for k in a:
        x, y = a[k].reshape(-1).astype(np.float64), b[k].reshape(-1).astype(np.float64)
        scale = max(np.abs(y).max(), 1e-30)
        assert np.abs(x - y).max() / scale < 2.0 ** -6, k


@pytest.mark.parametrize("cfg", [1, 2])
def test_bwd_full_size_sampled_heads(oracle, cfg):
    """The bf16 backward at the full layer workload (8 x 4096 tokens, 64 heads) in the bench's launch
    configuration; for two sampled heads, every gradient of all 8 sequences (dA, dD of the head
    included) against the oracle run on that head's inputs alone (G = H: a head reads only its own
    B, C and angle rows)."""
    import torch
    c = synth.CONFIGS[cfg]
    note(f"full-size bf16 backward config {cfg}: {c['name']}")
    dev = device()
    d = synth.torch_scan_inputs(cfg, dev, seed=cfg)
    gen = torch.Generator(device=dev)
    gen.manual_seed(100 + cfg)
    dy = torch.randn(d["x"].shape, generator=gen, device=dev, dtype=torch.float32).to(d["x"].dtype)
    g = m3.mamba3_scan_bwd(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"], dy=dy)
    torch.cuda.synchronize()

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    rng = np.random.default_rng(cfg)
    for hh in (0, int(rng.integers(1, c["nheads"]))):
        one = {k: bits(d[k][:, :, hh:hh + 1]) for k in ("x", "dt", "lam", "theta", "B", "C")}
        one.update(A=d["A"][hh:hh + 1].cpu().numpy(), D=d["D"][hh:hh + 1].cpu().numpy())
        dy1 = synth.bits_to_f32(bits(dy[:, :, hh:hh + 1])).astype(np.float64)
        go = oracle.scan_bwd(one, dy1, None)
        worst = {}
        for k in ("dx", "ddt", "dlam", "dtheta", "dB", "dC"):   # per (sequence, head) slab
            a = from_dev(g[k][:, :, hh:hh + 1]).reshape(go[k].shape)
            worst[k] = slab_err(k, a, go[k], None)
        for k in ("dA", "dD"):
            worst[k] = float(abs(from_dev(g[k][hh:hh + 1])[0] - go[k][0]) / abs(go[k][0]))
        note(f"  head {hh}: " + " ".join(f"{k} {v:.1e}" for k, v in worst.items()))
        bad = {k: v for k, v in worst.items() if not v < TOL_BF16}
        assert not bad, bad
    del d, dy, g
    torch.cuda.empty_cache()
