"""GPU parity of the fp32 chunked scan and of the decode step against the fp64
oracle (tolerance: max relative error 1e-4 for fp32, 2e-2 for bf16 token
inputs, per (sequence, head) slab). All calls go through the C ABI."""
import numpy as np
import pytest

from state_space_sequence_mamba3_amd import synth
import state_space_sequence_mamba3_amd as m3
from tests.gpu_util import TOL_BF16, TOL_F32, from_dev, note, device, slab_relerr, state_relerr, upload

pytestmark = pytest.mark.gpu


def run_scan(inp, chunk, want_state=True):
    import torch
    dev = device()
    d = upload(inp, dev)
    y, h = m3.mamba3_scan_fwd(d["x"], d["dt"], d.get("lam"), d["theta"], d["B"], d["C"], d.get("A"), d.get("D"),
                              h_in=d.get("h_in"), Bprev=d.get("Bprev"), xprev=d.get("xprev"),
                              cu_seqlens=d.get("cu_seqlens"), chunk=chunk, want_state=want_state,
                              B_bias=d.get("B_bias"), C_bias=d.get("C_bias"), z=d.get("z"),
                              bc_norm=d.get("bc_norm", False), bc_eps=d.get("bc_eps", 1e-5),
                              A_tok=d.get("A_tok"), lam_fixed=d.get("lam_fixed", 0.5))
    torch.cuda.synchronize()
    return from_dev(y), (from_dev(h) if h is not None else None)


def packed_relerr(g, o, cu):
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            worst = max(worst, slab_relerr(g[:, a:b], o[:, a:b]))
    return worst


def test_config0_tiny_siso_fp32(oracle):
    inp = synth.scan_inputs(0)
    note("scan f32 config0 " + str(inp["x"].shape))
    y, h = run_scan(inp, chunk=64)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(y, yo), state_relerr(h, ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_F32 and eh < TOL_F32


@pytest.mark.parametrize("shape", [
    dict(batch=2, seqlen=200, nheads=4, headdim=16, dstate=16, rank=1, chunk=64),
    dict(batch=2, seqlen=77, nheads=4, headdim=16, dstate=16, rank=1, chunk=16),
    dict(batch=1, seqlen=130, nheads=2, headdim=16, dstate=32, rank=4, chunk=16),
    dict(batch=2, seqlen=65, nheads=4, headdim=8, dstate=8, rank=2, chunk=32, ngroups=2),
    dict(batch=1, seqlen=33, nheads=2, headdim=64, dstate=64, rank=4, chunk=8, ngroups=1),
    dict(batch=3, seqlen=1, nheads=2, headdim=16, dstate=16, rank=2, chunk=64),
])
@pytest.mark.parametrize("resume", [False, True])
def test_scan_fp32_shapes(oracle, shape, resume):
    cfg = dict(synth.CONFIGS[0], **shape)
    inp = synth.scan_inputs(cfg, seed=7)
    if resume:
        inp = synth.resume_inputs(inp, seed=8)
    note(f"scan f32 {shape} resume={resume}")
    y, h = run_scan(inp, chunk=shape["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(y, yo), state_relerr(h, ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_F32 and eh < TOL_F32


def test_scan_fp32_packed_with_empty_sequences(oracle):
    cfg = dict(synth.CONFIGS[0], batch=1, seqlen=300, nheads=2, headdim=16, dstate=16, rank=2, chunk=32)
    inp = synth.scan_inputs(cfg, seed=9)
    inp["cu_seqlens"] = np.array([0, 50, 50, 51, 180, 300, 300], dtype=np.int32)
    inp = synth.resume_inputs(inp, seed=10)
    note("scan f32 packed with empty sequences")
    y, h = run_scan(inp, chunk=32)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    assert packed_relerr(y, yo, inp["cu_seqlens"]) < TOL_F32
    assert state_relerr(h, ho) < TOL_F32
    # an empty sequence passes its state through unchanged
    assert np.array_equal(h[1], inp["h_in"][1].astype(np.float64))


@pytest.mark.parametrize("shape", [
    dict(batch=2, seqlen=200, nheads=4, headdim=16, dstate=16, rank=1, chunk=64),
    dict(batch=1, seqlen=130, nheads=2, headdim=16, dstate=32, rank=4, chunk=16),
    dict(batch=2, seqlen=65, nheads=4, headdim=8, dstate=8, rank=2, chunk=32, ngroups=2),
])
@pytest.mark.parametrize("features", [
    dict(),
    dict(norm=False),
    dict(gate=False, B_bias=False),
    dict(norm=True, B_bias=False, C_bias=False, gate=False, eps=0.0),
])
def test_scan_fp32_block_prologue_epilogue(oracle, shape, features):
    cfg = dict(synth.CONFIGS[0], **shape)
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=17), seed=18)
    inp = synth.block_inputs(inp, seed=19, **features)
    note(f"scan f32 block {shape} {features}")
    y, h = run_scan(inp, chunk=shape["chunk"])
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    ey, eh = slab_relerr(y, yo), state_relerr(h, ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < TOL_F32 and eh < TOL_F32


def test_scan_fp32_block_packed(oracle):
    cfg = dict(synth.CONFIGS[0], batch=1, seqlen=300, nheads=2, headdim=16, dstate=16, rank=2, chunk=32)
    inp = synth.scan_inputs(cfg, seed=29)
    inp["cu_seqlens"] = np.array([0, 50, 50, 51, 180, 300, 300], dtype=np.int32)
    inp = synth.block_inputs(synth.resume_inputs(inp, seed=30), seed=31)
    note("scan f32 packed block prologue/epilogue")
    y, h = run_scan(inp, chunk=32)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    assert packed_relerr(y, yo, inp["cu_seqlens"]) < TOL_F32
    assert state_relerr(h, ho) < TOL_F32


@pytest.mark.parametrize("variant", [dict(A_tok=True), dict(A_tok=False, lam_fixed=0.5),
                                     dict(A_tok=True, lam_fixed=1.0), dict(A_tok=False, theta_groups=1),
                                     dict(A_tok=True, theta_groups=2)])
def test_scan_fp32_variants(oracle, variant):
    cfg = dict(synth.CONFIGS[0], batch=2, seqlen=90, nheads=4, headdim=16, dstate=16, rank=2, chunk=32, ngroups=2)
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=75), seed=76)
    inp = synth.variant_inputs(inp, seed=77, **variant)
    if variant["A_tok"]:
        inp["A"] = None
    note(f"scan f32 variant {variant}")
    y, h = run_scan(inp, chunk=32)
    yo, ho = oracle.scan({k: v for k, v in inp.items() if k != "meta"})
    assert slab_relerr(y, yo) < TOL_F32 and state_relerr(h, ho) < TOL_F32


def test_scan_fp32_chunk_size_invariance():
    cfg = dict(synth.CONFIGS[0], batch=1, seqlen=192, nheads=2, rank=2)
    inp = synth.scan_inputs(cfg, seed=12)
    note("scan f32 chunk invariance")
    ys = [run_scan(inp, chunk=q)[0] for q in (8, 32, 64, 40)]
    for y in ys[1:]:
        assert slab_relerr(y, ys[0]) < 1e-5


def test_scan_fp32_deterministic():
    inp = synth.scan_inputs(0, seed=13)
    note("scan f32 determinism")
    y1, h1 = run_scan(inp, chunk=64)
    y2, h2 = run_scan(inp, chunk=64)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


# ------------------------------------------------------------------ decode
def run_decode(inp, steps, ring_index=None):
    import torch
    dev = device()
    d = upload(inp, dev)
    h = d["h"].clone()
    ys = []
    Bprev, xprev = d["Bprev"], d["xprev"]
    for k in range(steps):
        i = k % d["x"].shape[0]
        lam = d["lam"][i] if d.get("lam") is not None else None
        atok = d["A_tok"][i] if d.get("A_tok") is not None else None
        y = m3.mamba3_decode_step(d["x"][i], d["dt"][i], lam, d["theta"][i], d["B"][i], d["C"][i],
                                  d.get("A"), d["D"], h=h, Bprev=Bprev, xprev=xprev, B_bias=d.get("B_bias"),
                                  C_bias=d.get("C_bias"), z=d["z"][i] if d.get("z") is not None else None,
                                  bc_norm=d.get("bc_norm", False), bc_eps=d.get("bc_eps", 1e-5), A_tok=atok,
                                  lam_fixed=d.get("lam_fixed", 0.5))
        ys.append(y)
        Bprev, xprev = d["B"][i], d["x"][i]
    torch.cuda.synchronize()
    return [from_dev(y) for y in ys], from_dev(h)


def oracle_decode(oracle, inp, steps):
    h = inp["h"].astype(np.float64)
    Bprev, xprev = inp["Bprev"], inp["xprev"]
    ys = []
    for k in range(steps):
        i = k % inp["x"].shape[0]
        tok = {kk: inp[kk][i] for kk in ("x", "dt", "theta", "B", "C")}
        tok["lam"] = inp["lam"][i] if inp.get("lam") is not None else None
        if inp.get("A_tok") is not None:
            tok["A_tok"] = inp["A_tok"][i]
        tok.update(A=inp.get("A"), D=inp["D"], Bprev=Bprev, xprev=xprev)
        for kk in ("B_bias", "C_bias", "bc_norm", "bc_eps", "lam_fixed"):
            if kk in inp:
                tok[kk] = inp[kk]
        if inp.get("z") is not None:
            tok["z"] = inp["z"][i]
        y, h = oracle.decode(tok, h)
        ys.append(y)
        Bprev, xprev = inp["B"][i], inp["x"][i]
    return ys, h


@pytest.mark.parametrize("dtype,tol", [("bf16", TOL_BF16), ("f32", TOL_F32)])
@pytest.mark.parametrize("shape", [
    dict(batch=8, nheads=4, headdim=64, dstate=64, rank=4),
    dict(batch=4, nheads=4, headdim=64, dstate=128, rank=4),
    dict(batch=4, nheads=2, headdim=64, dstate=128, rank=1),
    dict(batch=5, nheads=4, headdim=16, dstate=16, rank=1, ngroups=2),
])
def test_decode_steps(oracle, dtype, tol, shape):
    cfg = dict(synth.CONFIGS[3], dtype=dtype, **shape)
    inp = synth.decode_inputs(cfg, seed=21, ring=3)
    note(f"decode {dtype} {shape}")
    yg, hg = run_decode(inp, steps=4)
    yo, ho = oracle_decode(oracle, inp, steps=4)
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        den = np.abs(b).max(axis=(2, 3))
        assert float(np.max(num / den)) < tol
    assert state_relerr(hg, ho) < (tol if dtype == "f32" else 1e-5)


@pytest.mark.parametrize("dtype,tol", [("bf16", TOL_BF16), ("f32", TOL_F32)])
@pytest.mark.parametrize("shape", [
    dict(batch=8, nheads=4, headdim=64, dstate=64, rank=4),
    dict(batch=4, nheads=4, headdim=64, dstate=128, rank=4),
    dict(batch=4, nheads=2, headdim=64, dstate=128, rank=1),
    dict(batch=4, nheads=4, headdim=64, dstate=64, rank=2, ngroups=1),
    dict(batch=5, nheads=4, headdim=16, dstate=16, rank=4, ngroups=2),
    dict(batch=3, nheads=2, headdim=32, dstate=32, rank=2),
])
def test_decode_block_prologue_epilogue(oracle, dtype, tol, shape):
    """Fused B/C RMS norm (Bprev's columns included), per-head biases and SiLU(z) gate over
    several steps; the state is fp32 whatever the token dtype."""
    cfg = dict(synth.CONFIGS[3], dtype=dtype, **shape)
    inp = synth.block_inputs(synth.decode_inputs(cfg, seed=22, ring=3), seed=23)
    note(f"decode block prologue/epilogue {dtype} {shape}")
    yg, hg = run_decode(inp, steps=4)
    yo, ho = oracle_decode(oracle, inp, steps=4)
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        den = np.abs(b).max(axis=(2, 3))
        assert float(np.max(num / den)) < tol
    assert state_relerr(hg, ho) < (tol if dtype == "f32" else 1e-5)


@pytest.mark.parametrize("features", [
    dict(norm=True, B_bias=False, C_bias=False, gate=False),
    dict(norm=False, B_bias=True, C_bias=False, gate=False),
    dict(norm=False, B_bias=False, C_bias=True, gate=False),
    dict(norm=False, B_bias=False, C_bias=False, gate=True),
])
def test_decode_block_feature_subsets(oracle, features):
    cfg = dict(synth.CONFIGS[3], batch=6, nheads=4)
    inp = synth.block_inputs(synth.decode_inputs(cfg, seed=24, ring=2), seed=25, **features)
    note(f"decode block features {features}")
    yg, hg = run_decode(inp, steps=3)
    yo, ho = oracle_decode(oracle, inp, steps=3)
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        assert float(np.max(num / np.abs(b).max(axis=(2, 3)))) < TOL_BF16
    assert state_relerr(hg, ho) < 1e-5


@pytest.mark.parametrize("dtype,tol", [("bf16", TOL_BF16), ("f32", TOL_F32)])
@pytest.mark.parametrize("shape", [
    dict(batch=4, nheads=4, headdim=64, dstate=64, rank=4),
    dict(batch=4, nheads=2, headdim=64, dstate=128, rank=1),
    dict(batch=5, nheads=4, headdim=16, dstate=16, rank=1, ngroups=2),
])
@pytest.mark.parametrize("variant", [dict(A_tok=True), dict(A_tok=True, lam_fixed=0.5),
                                     dict(A_tok=False, theta_groups=1)])
def test_decode_variants(oracle, dtype, tol, shape, variant):
    cfg = dict(synth.CONFIGS[3], dtype=dtype, **shape)
    inp = synth.variant_inputs(synth.decode_inputs(cfg, seed=26, ring=3), seed=27, **variant)
    if variant["A_tok"]:
        inp["A"] = None
    note(f"decode variant {dtype} {shape} {variant}")
    yg, hg = run_decode(inp, steps=4)
    yo, ho = oracle_decode(oracle, inp, steps=4)
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        assert float(np.max(num / np.abs(b).max(axis=(2, 3)))) < tol
    assert state_relerr(hg, ho) < (tol if dtype == "f32" else 1e-5)


def test_decode_config3_full_batch(oracle):
    inp = synth.decode_inputs(3, ring=2)
    note("decode config3 full batch, 3 steps")
    yg, hg = run_decode(inp, steps=3)
    yo, ho = oracle_decode(oracle, inp, steps=3)
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        den = np.abs(b).max(axis=(2, 3))
        assert float(np.max(num / den)) < TOL_BF16
    assert state_relerr(hg, ho) < 1e-5


def test_decode_config3_full_batch_64_steps(oracle):
    """The decode workload at full batch (256 rows x 64 heads) for 64 consecutive steps on the
    hardware exp / sincos of the bf16 path, over a ring of 16 token-input sets (the state evolves,
    so no step repeats another). Rows are independent: every step's y and the final state of
    sampled rows (the first, the last and two inside) are checked against the oracle stepping
    those rows alone, per (row, head) slab."""
    import torch
    steps, rows = 64, [0, 37, 170, 255]
    inp = synth.decode_inputs(3, seed=8, ring=16)
    note(f"decode config3 full batch, {steps} steps, sampled rows {rows}")
    dev = device()
    d = upload(inp, dev)
    h = d["h"].clone()
    Bprev, xprev = d["Bprev"], d["xprev"]
    yg = []
    for k in range(steps):
        i = k % d["x"].shape[0]
        y = m3.mamba3_decode_step(d["x"][i], d["dt"][i], d["lam"][i], d["theta"][i], d["B"][i], d["C"][i],
                                  d["A"], d["D"], h=h, Bprev=Bprev, xprev=xprev)
        yg.append(from_dev(y[rows]))
        Bprev, xprev = d["B"][i], d["x"][i]
    torch.cuda.synchronize()
    hg = from_dev(h[rows])
    sub = {kk: inp[kk][:, rows] for kk in ("x", "dt", "lam", "theta", "B", "C")}
    sub.update(A=inp["A"], D=inp["D"], h=inp["h"][rows], Bprev=inp["Bprev"][rows], xprev=inp["xprev"][rows])
    yo, ho = oracle_decode(oracle, sub, steps=steps)
    worst = 0.0
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        worst = max(worst, float(np.max(num / np.abs(b).max(axis=(2, 3)))))
    note(f"  y relerr (max over steps and slabs) {worst:.2e}  h relerr {state_relerr(hg, ho):.2e}")
    assert worst < TOL_BF16
    assert state_relerr(hg, ho) < 1e-4


def test_decode_siso_full_batch(oracle):
    """The SISO decode shape of the bench (batch 256, 64 heads, N = 128, R = 1), whole batch, 2 steps."""
    inp = synth.decode_inputs(dict(synth.CONFIGS[3], dstate=128, rank=1), ring=2)
    note("SISO decode full batch, 2 steps")
    yg, hg = run_decode(inp, steps=2)
    yo, ho = oracle_decode(oracle, inp, steps=2)
    for a, b in zip(yg, yo):
        num = np.abs(a - b).max(axis=(2, 3))
        den = np.abs(b).max(axis=(2, 3))
        assert float(np.max(num / den)) < TOL_BF16
    assert state_relerr(hg, ho) < 1e-5


def test_decode_without_previous_token(oracle):
    cfg = dict(synth.CONFIGS[3], batch=4, nheads=2)
    inp = synth.decode_inputs(cfg, seed=5, ring=1)
    note("decode without previous token")
    import torch
    dev = device()
    d = upload(inp, dev)
    h = d["h"].clone()
    y = m3.mamba3_decode_step(d["x"][0], d["dt"][0], d["lam"][0], d["theta"][0], d["B"][0], d["C"][0],
                              d["A"], d["D"], h=h)
    torch.cuda.synchronize()
    tok = {kk: inp[kk][0] for kk in ("x", "dt", "lam", "theta", "B", "C")}
    tok.update(A=inp["A"], D=inp["D"])
    yo, ho = oracle.decode(tok, inp["h"].astype(np.float64))
    assert state_relerr(from_dev(h), ho) < 1e-5
    num = np.abs(from_dev(y) - yo).max(axis=(2, 3))
    assert float(np.max(num / np.abs(yo).max(axis=(2, 3)))) < TOL_BF16


@pytest.mark.parametrize("shape,block", [
    (dict(), False),                                          # column kernel (P = 64)
    (dict(), True),                                           # column kernel, fused prologue / gate
    (dict(headdim=16, dstate=16, rank=1, dtype="f32"), True),   # tile kernel (P = 16), fp32
])
def test_decode_slots(oracle, shape, block):
    """Slot-indexed states: batch rows update pool slots [3, -, 0, 6, -] (one row with a negative
    slot, one past the pool); inactive rows leave their y rows and every other slot untouched,
    bit for bit; active rows match the oracle from the gathered states and match, bit for bit,
    the same step run on the gathered states without slots."""
    import torch
    dev = device()
    cfg = dict(synth.CONFIGS[3], batch=5, nheads=4, **shape)
    inp = synth.decode_inputs(cfg, seed=28, ring=1)
    if block:
        inp = synth.block_inputs(inp, seed=30)
    d = upload(inp, dev)
    H, N, P = 4, cfg["dstate"], cfg["headdim"]
    tol = TOL_F32 if cfg.get("dtype") == "f32" else TOL_BF16
    blk = {}
    if block:
        blk = dict(B_bias=d["B_bias"], C_bias=d["C_bias"], z=d["z"][0], bc_norm=True, bc_eps=d["bc_eps"])
    rng = np.random.default_rng(29)
    pool0 = rng.standard_normal((7, H, N, P)).astype(np.float32)
    slots = np.array([3, -1, 0, 6, 7], dtype=np.int32)
    active = [i for i, s in enumerate(slots) if 0 <= s < 7]
    pool = torch.from_numpy(pool0).to(dev)
    sl = torch.from_numpy(slots).to(dev)
    sentinel = torch.full_like(d["x"][0], 7.0)
    note("decode with slots")
    args = [d[k][0] for k in ("x", "dt", "lam", "theta", "B", "C")] + [d["A"], d["D"]]
    m3.mamba3_decode_step(*args, h=pool, y=sentinel, Bprev=d["Bprev"], xprev=d["xprev"], slots=sl, **blk)
    hg = torch.from_numpy(pool0[slots[active]]).to(dev).contiguous()
    hfull = torch.zeros((5, H, N, P), dtype=torch.float32, device=dev)
    hfull[active] = hg
    y_ref = m3.mamba3_decode_step(*args, h=hfull, Bprev=d["Bprev"], xprev=d["xprev"], **blk)
    torch.cuda.synchronize()
    pool_g, y_g, y_r, h_r = from_dev(pool), from_dev(sentinel), from_dev(y_ref), from_dev(hfull)
    untouched = [s for s in range(7) if s not in slots[active]]
    assert np.array_equal(pool_g[untouched], pool0[untouched])
    assert np.all(y_g[[1, 4]] == 7.0)
    assert np.array_equal(y_g[active], y_r[active]) and np.array_equal(pool_g[slots[active]], h_r[active])
    tok = {k: inp[k][0][active] for k in ("x", "dt", "lam", "theta", "B", "C")}
    tok.update(A=inp["A"], D=inp["D"], Bprev=inp["Bprev"][active], xprev=inp["xprev"][active])
    if block:
        tok.update(B_bias=inp["B_bias"], C_bias=inp["C_bias"], z=inp["z"][0][active], bc_norm=True,
                   bc_eps=inp["bc_eps"])
    yo, ho = oracle.decode(tok, pool0[slots[active]].astype(np.float64))
    num = np.abs(y_g[active] - yo).max(axis=(2, 3))
    assert float(np.max(num / np.abs(yo).max(axis=(2, 3)))) < tol
    assert state_relerr(pool_g[slots[active]], ho) < (tol if cfg.get("dtype") == "f32" else 1e-5)


def test_decode_graph_replay():
    """Three decode steps captured in a HIP graph and replayed several times, with the program's
    own eager work and synchronisations between the replays: every replay equals the same three
    steps run eagerly from the same starting state, bit for bit."""
    import torch
    dev = device()
    cfg = dict(synth.CONFIGS[3], batch=8, nheads=4)
    inp = synth.decode_inputs(cfg, seed=33, ring=3)
    d = upload(inp, dev)
    h0 = d["h"].clone()
    h = h0.clone()
    ys = [torch.empty_like(d["x"][0]) for _ in range(3)]

    def steps():
        Bprev, xprev = d["Bprev"], d["xprev"]
        for i in range(3):
            m3.mamba3_decode_step(d["x"][i], d["dt"][i], d["lam"][i], d["theta"][i], d["B"][i], d["C"][i], d["A"],
                                  d["D"], h=h, y=ys[i], Bprev=Bprev, xprev=xprev,
                                  stream=torch.cuda.current_stream())
            Bprev, xprev = d["B"][i], d["x"][i]

    note("decode graph replay")
    steps()
    torch.cuda.synchronize()
    y_eager = [y.clone() for y in ys]
    h_eager = h.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.copy_(h0)
        with torch.cuda.graph(g):
            steps()
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(h0)                       # eager work between the replays
        ys[0].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(ys, y_eager)), rep
        assert torch.equal(h, h_eager), rep
