"""GPU parity of the bf16 MFMA chunked scan against the fp64 oracle (max
relative error 2e-2 per (sequence, head) slab, for y and the final state),
without and with the fused block prologue / epilogue (B/C RMS norm, per-head
B/C biases, SiLU(z) output gate).

Small cases run the whole oracle; the full-size workloads (8 x 4096 tokens,
64 heads; the packed 65536-token workload) run the kernel at full size in the
bench's launch configuration and check sampled (sequence, head) slabs, each
recomputed by the oracle from that slab's inputs."""
import numpy as np
import pytest

import state_space_sequence_mamba3_amd as m3
from state_space_sequence_mamba3_amd import synth
from tests.gpu_util import TOL_BF16, device, from_dev, note, slab_relerr, state_relerr, upload

pytestmark = pytest.mark.gpu


def run(d, chunk, want_state=True):
    import torch
    y, h = m3.mamba3_scan_fwd(d["x"], d["dt"], d.get("lam"), d["theta"], d["B"], d["C"], d.get("A"), d.get("D"),
                              h_in=d.get("h_in"), Bprev=d.get("Bprev"), xprev=d.get("xprev"),
                              cu_seqlens=d.get("cu_seqlens"), chunk=chunk, want_state=want_state,
                              B_bias=d.get("B_bias"), C_bias=d.get("C_bias"), z=d.get("z"),
                              bc_norm=d.get("bc_norm", False), bc_eps=d.get("bc_eps", 1e-5),
                              A_tok=d.get("A_tok"), lam_fixed=d.get("lam_fixed", 0.5))
    torch.cuda.synchronize()
    return y, h


def packed_relerr(g, o, cu):
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            worst = max(worst, slab_relerr(g[:, a:b], o[:, a:b]))
    return worst


SMALL = {
    "cfg1_siso_n128": dict(cfg=1, batch=2, seqlen=300, nheads=3),
    "cfg2_mimo_n64": dict(cfg=2, batch=2, seqlen=200, nheads=3),
    "cfg4_mimo_n128_q128": dict(cfg=4, batch=1, seqlen=333, nheads=2, packed=False),
    "n64_r1": dict(cfg=1, batch=1, seqlen=150, nheads=2, dstate=64),
    "n64_r4_q32": dict(cfg=2, batch=1, seqlen=150, nheads=2, chunk=32),
    "n128_r2": dict(cfg=1, batch=1, seqlen=190, nheads=2, rank=2),
    "n128_r4_q64": dict(cfg=4, batch=1, seqlen=250, nheads=2, chunk=64, packed=False),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("resume", [False, True])
def test_small_vs_full_oracle(oracle, name, resume):
    spec = dict(SMALL[name])
    cfg = spec.pop("cfg")
    inp = synth.scan_inputs(cfg, seed=100 + len(name), **spec)
    if resume:
        inp = synth.resume_inputs(inp, seed=5)
    chunk = inp["meta"]["chunk"]
    note(f"bf16 scan {name} resume={resume} x{inp['x'].shape} chunk={chunk}")
    y, h = run(upload(inp, device()), chunk)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("name", sorted(SMALL))
def test_block_prologue_epilogue(oracle, name):
    """Fused B/C RMS norm, per-head B/C biases and SiLU(z) gate, with a resumed state and a
    previous token (whose B column goes through the prologue too)."""
    spec = dict(SMALL[name])
    cfg = spec.pop("cfg")
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=200 + len(name), **spec), seed=6)
    inp = synth.block_inputs(inp, seed=7)
    chunk = inp["meta"]["chunk"]
    note(f"bf16 scan block prologue/epilogue {name} x{inp['x'].shape} chunk={chunk}")
    y, h = run(upload(inp, device()), chunk)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("cfg", [1, 2])
@pytest.mark.parametrize("features", [
    dict(norm=True, B_bias=False, C_bias=False, gate=False),
    dict(norm=False, B_bias=True, C_bias=False, gate=False),
    dict(norm=False, B_bias=False, C_bias=True, gate=False),
    dict(norm=False, B_bias=False, C_bias=False, gate=True),
    dict(norm=True, B_bias=True, C_bias=True, gate=True, eps=0.0),
])
def test_block_feature_subsets(oracle, cfg, features):
    """Each prologue / epilogue feature alone (each switches the fused kernel on), and all of
    them with eps = 0."""
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=51, batch=2, seqlen=150, nheads=2), seed=52)
    inp = synth.block_inputs(inp, seed=53, **features)
    note(f"bf16 scan block features cfg{cfg} {features}")
    y, h = run(upload(inp, device()), inp["meta"]["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


def test_block_packed_grouped(oracle):
    """Prologue / epilogue on a packed ragged batch with G = 1 (every head adds its own bias to
    the shared B and C) and empty sequences."""
    inp = synth.scan_inputs(dict(synth.CONFIGS[4], ngroups=1), seed=61, seqlen=600, nheads=2)
    inp["cu_seqlens"] = np.array([0, 1, 1, 200, 333, 600, 600], dtype=np.int32)
    inp = synth.block_inputs(synth.resume_inputs(inp, seed=62), seed=63)
    note("bf16 packed block prologue/epilogue, G=1")
    y, h = run(upload(inp, device()), 128)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    assert packed_relerr(from_dev(y), yo, inp["cu_seqlens"]) < TOL_BF16
    assert state_relerr(from_dev(h), ho) < TOL_BF16


@pytest.mark.parametrize("cfg", [1, 2, 4])
@pytest.mark.parametrize("variant", [
    dict(A_tok=True),
    dict(A_tok=False, lam_fixed=0.5),
    dict(A_tok=True, lam_fixed=1.0),
    dict(A_tok=False, theta_groups=1),
])
def test_variants(oracle, cfg, variant):
    """Per-token decay rate A_t (A absent), fixed trapezoid weights and one angle row shared by
    all heads, with a resumed state."""
    spec = dict(batch=2, seqlen=150, nheads=2) if cfg != 4 else dict(seqlen=300, nheads=2, packed=False)
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=71, **spec), seed=72)
    inp = synth.variant_inputs(inp, seed=73, **variant)
    if variant["A_tok"]:
        inp["A"] = None
    note(f"bf16 scan variant cfg{cfg} {variant}")
    y, h = run(upload(inp, device()), inp["meta"]["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_strong_decay(oracle, cfg):
    """Heads whose decay over a chunk spans from a few to hundreds of binary orders of
    magnitude: chunks beyond the factored mask's range take the per-element form, chunks
    near the threshold switch between the two."""
    inp = synth.scan_inputs(cfg, seed=41, batch=2, seqlen=400, nheads=4, packed=False)
    inp["A"] = np.array([-0.5, -9.0, -10.0, -40.0], dtype=np.float32)
    inp = synth.resume_inputs(inp, seed=42)
    note(f"bf16 strong decay cfg{cfg}")
    y, h = run(upload(inp, device()), inp["meta"]["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_large_angles(oracle, cfg):
    """Angles 64 times the generator's (exact in bf16): a chunk's cumulative angles reach
    hundreds to thousands of radians, so the state rotation by the chunk's total angle depends on
    the kernels' 2 pi reduction before the hardware sine and cosine, and the per-token tables are
    built far from the origin."""
    inp = synth.scan_inputs(cfg, seed=43, batch=2, seqlen=300, nheads=4, packed=False)
    th = inp["theta"]
    f = (th.astype(np.uint32) << 16).view(np.float32) if th.dtype == np.uint16 else th
    inp["theta"] = synth.bf16_bits(f * 64.0) if th.dtype == np.uint16 else f * 64.0
    inp = synth.resume_inputs(inp, seed=44)
    note(f"bf16 large angles cfg{cfg}")
    y, h = run(upload(inp, device()), inp["meta"]["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


def test_grouped_bc_and_no_skip(oracle):
    inp = synth.scan_inputs(dict(synth.CONFIGS[2], ngroups=1), seed=3, batch=1, seqlen=130, nheads=4)
    inp["D"] = None
    note("bf16 scan G=1, D=NULL")
    y, h = run(upload(inp, device()), 64)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k not in ("meta", "D")})
    assert slab_relerr(from_dev(y), yo) < TOL_BF16 and state_relerr(from_dev(h), ho) < TOL_BF16


# The panel kernel: a chunk is two panels (64 tokens at the packed workload's shape, N = 128,
# R = 4, chunk 128; 32 tokens at the MIMO layer's, N = 64, R = 4, chunk 64); a last chunk may end
# inside panel 0 or panel 1, or on a panel boundary.
@pytest.mark.parametrize("cfg,seqlen", [(4, 300), (4, 333), (4, 64), (4, 1), (2, 31), (2, 32), (2, 33),
                                        (2, 95), (2, 128), (2, 161)])
def test_panel_partial_chunks(oracle, cfg, seqlen):
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=70 + seqlen, batch=2, seqlen=seqlen, nheads=2,
                                                packed=False), seed=71)
    Q = inp["meta"]["chunk"]
    note(f"bf16 panel scan cfg{cfg}, last chunk of {seqlen % Q or Q} tokens")
    y, h = run(upload(inp, device()), Q)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("cfg", [2, 4])
def test_panel_grouped_no_skip(oracle, cfg):
    inp = synth.scan_inputs(dict(synth.CONFIGS[cfg], ngroups=1), seed=72, batch=1, seqlen=390, nheads=4, packed=False)
    inp["D"] = None
    note(f"bf16 panel scan cfg{cfg} G=1, D=NULL")
    y, h = run(upload(inp, device()), inp["meta"]["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k not in ("meta", "D")})
    assert slab_relerr(from_dev(y), yo) < TOL_BF16 and state_relerr(from_dev(h), ho) < TOL_BF16


@pytest.mark.parametrize("cfg", [2, 4])
def test_panel_weight_guard(oracle, cfg):
    """A trapezoid weight lam > 1 can make gamma_s + delta_{s+1} vanish while gamma_s does not (dt
    and lam chosen exactly representable: gamma_10 = 0.5 * 0.125, delta_11 = (1 - 2) * 0.0625); the
    chunk holding that token takes the unscaled per-element form, whose panels reach each other
    through the state referenced to each panel's start. Both panel-kernel shapes (MIMO layer:
    chunk 64 in 32-token panels; packed: chunk 128 in 64-token panels)."""
    inp = synth.scan_inputs(cfg, seed=73, batch=1, seqlen=256, nheads=2, packed=False)
    dt = np.full(inp["dt"].shape, 0.125, dtype=np.float32)
    lam = np.full(inp["lam"].shape, 0.5, dtype=np.float32)
    dt[:, 11], lam[:, 11] = 0.0625, 2.0
    dt[:, 45], lam[:, 45] = 0.0625, 2.0            # in panel 1 of the first chunk (either shape)
    dt[:, 75], lam[:, 75] = 0.0625, 2.0
    dt[:, 140], lam[:, 140] = 0.0625, 2.0          # the same in a later chunk
    inp["dt"], inp["lam"] = synth.bf16_bits(dt), synth.bf16_bits(lam)
    note(f"bf16 panel scan cfg{cfg}, vanishing trapezoid weight")
    y, h = run(upload(inp, device()), inp["meta"]["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(from_dev(y), yo), state_relerr(from_dev(h), ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("cfg,qp,qg", [(4, 128, 64), (2, 64, 32)])
def test_panel_chunk_invariance_and_determinism(cfg, qp, qg):
    """The panel kernel's chunk (qp) against a general-kernel chunk (qg) on the same inputs, and
    two runs of the panel kernel bitwise equal."""
    inp = synth.scan_inputs(cfg, seed=74, batch=1, seqlen=512, nheads=2, packed=False)
    note(f"bf16 panel scan cfg{cfg}: chunk {qp} vs {qg}, determinism")
    d = upload(inp, device())
    yp, hp = run(d, qp)
    yg, hg = run(d, qg)
    assert slab_relerr(from_dev(yp), from_dev(yg)) < TOL_BF16
    assert state_relerr(from_dev(hp), from_dev(hg)) < 1e-2
    y2, h2 = run(d, qp)
    assert from_dev(yp).tobytes() == from_dev(y2).tobytes() and np.array_equal(from_dev(hp), from_dev(h2))


def test_packed_ragged_with_empty(oracle):
    inp = synth.scan_inputs(4, seed=11, seqlen=700, nheads=2)
    inp["cu_seqlens"] = np.array([0, 1, 1, 129, 130, 400, 700, 700], dtype=np.int32)
    inp = synth.resume_inputs(inp, seed=12)
    note("bf16 packed ragged with empty sequences")
    y, h = run(upload(inp, device()), 128)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    assert packed_relerr(from_dev(y), yo, inp["cu_seqlens"]) < TOL_BF16
    assert state_relerr(from_dev(h), ho) < TOL_BF16
    assert np.array_equal(from_dev(h)[1], inp["h_in"][1].astype(np.float64))


@pytest.mark.parametrize("lengths", [
    [100, 300, 100, 300, 0, 300],                     # ties in length: ranked by index
    list(np.random.default_rng(31).integers(0, 41, size=70)),   # more than 64 sequences: launch order
])
def test_packed_sequence_order(oracle, lengths):
    """Packed batches run their sequences in an order of the kernel's choosing (longest
    first for up to 64 sequences); every sequence still gets its own state and outputs."""
    total = int(sum(lengths))
    inp = synth.scan_inputs(2, seed=33, seqlen=total, nheads=2, batch=1)
    inp["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    inp = synth.resume_inputs(inp, seed=34)
    note(f"bf16 packed order, {len(lengths)} sequences")
    y, h = run(upload(inp, device()), 64)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    assert packed_relerr(from_dev(y), yo, inp["cu_seqlens"]) < TOL_BF16
    assert state_relerr(from_dev(h), ho) < TOL_BF16


def test_chunk_size_invariance():
    inp = synth.scan_inputs(2, seed=21, batch=1, seqlen=256, nheads=2)
    note("bf16 chunk invariance 32 vs 64")
    d = upload(inp, device())
    y32, h32 = run(d, 32)
    y64, h64 = run(d, 64)
    assert slab_relerr(from_dev(y32), from_dev(y64)) < TOL_BF16
    assert state_relerr(from_dev(h32), from_dev(h64)) < 1e-2


def test_deterministic():
    inp = synth.scan_inputs(1, seed=22, batch=2, seqlen=200, nheads=2)
    note("bf16 determinism")
    d = upload(inp, device())
    y1, h1 = run(d, 64)
    y2, h2 = run(d, 64)
    assert from_dev(y1).tobytes() == from_dev(y2).tobytes() and np.array_equal(from_dev(h1), from_dev(h2))


def test_split_resume_matches_whole():
    """scan(0:T) == scan(0:k) -> (h, B_{k-1}, x_{k-1}) -> scan(k:T) on the GPU."""
    import torch
    inp = synth.scan_inputs(2, seed=23, batch=2, seqlen=200, nheads=2)
    note("bf16 split/resume")
    d = upload(inp, device())
    yw, hw = run(d, 64)
    k = 77
    tok = ("x", "dt", "lam", "theta", "B", "C")
    a = {kk: (v[:, :k].contiguous() if kk in tok else v) for kk, v in d.items()}
    b = {kk: (v[:, k:].contiguous() if kk in tok else v) for kk, v in d.items()}
    y1, h1 = run(a, 64)
    b["h_in"], b["Bprev"], b["xprev"] = h1, d["B"][:, k - 1].contiguous(), d["x"][:, k - 1].contiguous()
    y2, h2 = run(b, 64)
    assert slab_relerr(from_dev(torch.cat([y1, y2], 1)), from_dev(yw)) < TOL_BF16
    assert state_relerr(from_dev(h2), from_dev(hw)) < TOL_BF16


# ---------------------------------------------------------------- full size
def _slab_inputs(d, s, h, cu=None):
    """Host copy (bf16 bits) of one (sequence, head) slab of device inputs."""
    import torch
    G = d["B"].shape[2]
    H = d["x"].shape[2]
    g = h // (H // G)
    if cu is not None:
        a, b = int(cu[s]), int(cu[s + 1])
        sl = (0, slice(a, b))
    else:
        sl = (s, slice(None))

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[None]

    out = dict(x=bits(d["x"][sl][:, h:h + 1]), dt=bits(d["dt"][sl][:, h:h + 1]), lam=bits(d["lam"][sl][:, h:h + 1]),
               theta=bits(d["theta"][sl][:, h:h + 1]), B=bits(d["B"][sl][:, g:g + 1]), C=bits(d["C"][sl][:, g:g + 1]),
               A=d["A"][h:h + 1].cpu().numpy(), D=d["D"][h:h + 1].cpu().numpy())
    if d.get("z") is not None:
        out["z"] = bits(d["z"][sl][:, h:h + 1])
    for k in ("B_bias", "C_bias"):
        if d.get(k) is not None:
            out[k] = d[k][h:h + 1].cpu().numpy()
    if "bc_norm" in d:
        out["bc_norm"], out["bc_eps"] = d["bc_norm"], d["bc_eps"]
    return out


@pytest.mark.parametrize("cfg,block", [(1, False), (2, False), (4, False), (1, True), (2, True), (4, True)])
def test_full_size_sampled_slabs(oracle, cfg, block):
    import torch
    c = synth.CONFIGS[cfg]
    note(f"full-size bf16 scan config {cfg}: {c['name']} block prologue/epilogue={block}")
    d = synth.torch_scan_inputs(cfg, device(), seed=cfg)
    if block:
        d = synth.torch_block_inputs(d, device(), seed=cfg)
    y, h = run(d, c["chunk"])
    cu = d["cu_seqlens"].cpu().numpy() if "cu_seqlens" in d else None
    S = (len(cu) - 1) if cu is not None else c["batch"]
    rng = np.random.default_rng(cfg)
    H = c["nheads"]
    picks = [(0, 0), (S - 1, H - 1)] + [(int(rng.integers(S)), int(rng.integers(H))) for _ in range(3)]
    if cu is not None:
        # packed: the longest sequence (the kernel's first workgroups, and its longest chain of
        # chunks) and the last workgroup in the kernel's longest-first order (the shortest
        # sequence, ties by index, last head)
        ln = np.diff(cu)
        order = sorted(range(S), key=lambda i: (-int(ln[i]), i))
        picks += [(order[0], int(rng.integers(H))), (order[-1], H - 1)]
    for s, hh in picks:
        one = _slab_inputs(d, s, hh, cu)
        yo, ho = oracle.scan_slab(one, 0, 0)
        if cu is not None:
            yg = y[0, int(cu[s]):int(cu[s + 1]), hh]
        else:
            yg = y[s, :, hh]
        ey = float(np.abs(from_dev(yg) - yo).max() / np.abs(yo).max())
        eh = float(np.abs(from_dev(h[s, hh]) - ho).max() / np.abs(ho).max())
        note(f"  slab (s={s}, h={hh}) len={yo.shape[0]}: y relerr {ey:.2e}  h relerr {eh:.2e}")
        assert ey < TOL_BF16 and eh < TOL_BF16
    del d, y, h
    torch.cuda.empty_cache()
