"""GPU parity of state passing between segments (mamba3_state_passing) and of
the segmented scan built on it: each sequence cut into nseg segments, the
segments scanned from zero states, their entering states chained by the state
passing kernel, and the segments scanned again from those states. Checked
against the fp64 oracle's whole-sequence scan (y, final state) and, for the
entering states themselves, against the oracle's state after each segment
boundary (a scan of the prefix up to the boundary). Tolerances as for the
scans: 1e-4 for fp32, 2e-2 for bf16 token inputs."""
import numpy as np
import pytest

import state_space_sequence_mamba3_amd as m3
from state_space_sequence_mamba3_amd import synth
from tests.gpu_util import TOL_BF16, TOL_F32, device, from_dev, note, slab_relerr, state_relerr, upload

pytestmark = pytest.mark.gpu


def segmented(d, nseg, chunk):
    import torch
    y, h = m3.mamba3_scan_segmented(d["x"], d["dt"], d.get("lam"), d["theta"], d["B"], d["C"], d.get("A"),
                                    d.get("D"), nseg=nseg, h_in=d.get("h_in"), Bprev=d.get("Bprev"),
                                    xprev=d.get("xprev"), chunk=chunk, B_bias=d.get("B_bias"),
                                    C_bias=d.get("C_bias"), z=d.get("z"), bc_norm=d.get("bc_norm", False),
                                    bc_eps=d.get("bc_eps", 1e-5), A_tok=d.get("A_tok"),
                                    lam_fixed=d.get("lam_fixed", 0.5))
    torch.cuda.synchronize()
    return from_dev(y), from_dev(h)


def oracle_inputs(inp):
    return {k: v for k, v in inp.items() if k != "meta"}


def boundary_states(oracle, inp, nseg):
    """The oracle's state entering every segment: h_in (or zero) for the first,
    then the final state of the prefix that ends at each boundary."""
    m = inp["meta"]
    b, L, H, N, P = m["batch"], m["seqlen"], m["nheads"], m["dstate"], m["headdim"]
    Ls = L // nseg
    out = np.zeros((b, nseg, H, N, P))
    if inp.get("h_in") is not None:
        out[:, 0] = inp["h_in"]
    for k in range(1, nseg):
        pre = {kk: (v[:, :k * Ls] if kk in ("x", "dt", "lam", "theta", "B", "C", "z", "A_tok") and v is not None
                    else v) for kk, v in oracle_inputs(inp).items()}
        _, h = oracle.scan(pre)
        out[:, k] = h
    return out.reshape(b * nseg, H, N, P)


CASES = [
    # (label, config, overrides, nseg, chunk, extras)
    ("bf16 SISO", 1, dict(batch=2, seqlen=384, nheads=2), 4, 64, ()),
    ("bf16 SISO ragged segments", 1, dict(batch=1, seqlen=200, nheads=2), 2, 64, ("resume",)),
    ("bf16 MIMO resume", 2, dict(batch=2, seqlen=192, nheads=2), 3, 64, ("resume",)),
    ("bf16 MIMO block + variants", 2, dict(batch=1, seqlen=256, nheads=4, ngroups=2), 4, 64,
     ("resume", "block", "variants")),
    ("f32 tiny", 0, dict(batch=2, seqlen=240), 5, 32, ("resume",)),
    ("f32 grouped + variants", 0, dict(batch=1, seqlen=180, nheads=4, ngroups=2, rank=2), 3, 32,
     ("resume", "block", "variants")),
    ("bf16 one segment", 1, dict(batch=2, seqlen=130, nheads=2), 1, 64, ("resume",)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_segmented_scan(oracle, case):
    label, cfg, over, nseg, chunk, extras = case
    inp = synth.scan_inputs(cfg, seed=131, **over)
    if "resume" in extras:
        inp = synth.resume_inputs(inp, seed=132)
    if "block" in extras:
        inp = synth.block_inputs(inp, seed=133)
    if "variants" in extras:
        inp = synth.variant_inputs(inp, seed=134, A_tok=True, lam_fixed=0.5, theta_groups=1)
        inp["A"] = None
    tol = TOL_F32 if inp["meta"]["dtype"] == "f32" else TOL_BF16
    note(f"segmented scan: {label}, nseg {nseg}")
    d = upload(inp, device())
    y, h = segmented(d, nseg, chunk)
    yo, ho = oracle.scan(oracle_inputs(inp))
    ey, eh = slab_relerr(y, yo), state_relerr(h, ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < tol and eh < tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_entering_states(oracle, dtype):
    """The state passing kernel's entering states and boundary tokens, step by step."""
    import torch
    cfg = 0 if dtype == "f32" else 1
    over = dict(batch=2, seqlen=192) if dtype == "f32" else dict(batch=2, seqlen=256, nheads=2)
    nseg = 4
    inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=141, **over), seed=142)
    m = inp["meta"]
    b, L, H = m["batch"], m["seqlen"], m["nheads"]
    d = upload(inp, device())
    note(f"state passing {dtype}: entering states")
    seg = lambda t: t.reshape((b * nseg, L // nseg) + tuple(t.shape[2:]))
    _, U = m3.mamba3_scan_fwd(*(seg(d[k]) for k in ("x", "dt", "lam", "theta", "B", "C")), d["A"], None,
                              chunk=m["chunk"])
    seg_h, seg_B, seg_x, h_out = m3.mamba3_state_passing(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"],
                                                         d["A"], nseg=nseg, U=U, h_in=d["h_in"], Bprev=d["Bprev"],
                                                         xprev=d["xprev"])
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    ref = boundary_states(oracle, inp, nseg)
    assert state_relerr(from_dev(seg_h), ref) < tol
    _, ho = oracle.scan(oracle_inputs(inp))
    assert state_relerr(from_dev(h_out), ho) < tol
    # boundary tokens are copied exactly: the sequence's own for segment 0, else the last token before
    Ls = L // nseg
    xb = from_dev(seg_x).reshape(b, nseg, *seg_x.shape[1:])
    Bb = from_dev(seg_B).reshape(b, nseg, *seg_B.shape[1:])
    x_all, B_all = from_dev(d["x"]), from_dev(d["B"])
    assert np.array_equal(xb[:, 0], from_dev(d["xprev"])) and np.array_equal(Bb[:, 0], from_dev(d["Bprev"]))
    for k in range(1, nseg):
        assert np.array_equal(xb[:, k], x_all[:, k * Ls - 1]) and np.array_equal(Bb[:, k], B_all[:, k * Ls - 1])


def test_long_sequence_matches_unsplit():
    """A 16384-token bf16 SISO sequence: segmented (8 segments) against the plain scan on the GPU,
    per slab, within the bf16 tolerance (both paths round the same inputs differently)."""
    import torch
    inp = synth.scan_inputs(1, seed=151, batch=1, seqlen=16384, nheads=8)
    d = upload(inp, device())
    note("segmented vs plain, 16384 tokens")
    y1, h1 = m3.mamba3_scan_fwd(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"], chunk=64)
    y2, h2 = segmented(d, 8, 64)
    torch.cuda.synchronize()
    assert slab_relerr(y2, from_dev(y1)) < TOL_BF16 and state_relerr(h2, from_dev(h1)) < TOL_BF16


def test_long_sequence_full_size_sampled_heads(oracle):
    """The bench's long-sequence workload (one 65536-token SISO sequence, 64 heads) in its launch
    configuration (16 segments): two sampled heads' y and final state against the oracle's
    whole-sequence scan of that head alone (G = H: a head reads only its own rows)."""
    import torch
    dev = device()
    c = synth.CONFIGS[1]
    d = synth.torch_scan_inputs(1, dev, seed=11, batch=1, seqlen=65536)
    note("segmented scan, 1 x 65536 tokens, 16 segments")
    y, h = m3.mamba3_scan_segmented(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"],
                                    nseg=16, chunk=c["chunk"])
    torch.cuda.synchronize()

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    for hh in (0, 37):
        one = {k: bits(d[k][:, :, hh:hh + 1]) for k in ("x", "dt", "lam", "theta", "B", "C")}
        one.update(A=d["A"][hh:hh + 1].cpu().numpy(), D=d["D"][hh:hh + 1].cpu().numpy())
        yo, ho = oracle.scan_slab(one, 0, 0)
        ey = float(np.abs(from_dev(y[0, :, hh]) - yo).max() / np.abs(yo).max())
        eh = float(np.abs(from_dev(h[0, hh]) - ho).max() / np.abs(ho).max())
        note(f"  head {hh}: y relerr {ey:.2e}  h relerr {eh:.2e}")
        assert ey < TOL_BF16 and eh < TOL_BF16
    del d, y, h
    torch.cuda.empty_cache()


# ---- packed batches: each sequence cut into segments of seg_tokens tokens ----

def expected_segment_table(cu, seqlen, L):
    """The segment rows' first tokens, then the last sequence's end up to the row bound."""
    nseq = len(cu) - 1
    rows = nseq + -(-seqlen // L)
    out = []
    for i in range(nseq):
        a = min(max(int(cu[i]), 0), seqlen)
        b = min(max(int(cu[i + 1]), a), seqlen)
        n = max(1, -(-(b - a) // L))
        out += [a + k * L for k in range(n)]
    end = min(max(int(cu[nseq]), min(max(int(cu[nseq - 1]), 0), seqlen)), seqlen) if nseq else 0
    return np.array(out + [end] * (rows + 1 - len(out)), dtype=np.int64)


@pytest.mark.parametrize("cu,L", [
    ([0, 1, 1, 129, 130, 400, 700, 700], 64),
    ([0, 1, 1, 129, 130, 400, 700, 700], 100),
    ([0, 256, 512], 128),                     # lengths a multiple of the segment
    ([0, 0], 7),                              # one empty sequence
    ([0, 5, 9], 1000),                        # one segment per sequence
    (list(np.cumsum([0] + list(np.random.default_rng(5).integers(0, 300, size=1500)))), 97),   # > 1024 sequences
])
def test_segment_table(cu, L):
    """Index work: the table is compared exactly."""
    import torch
    cu = np.asarray(cu, dtype=np.int32)
    T = int(cu[-1])
    note(f"segment table: {len(cu) - 1} sequences, {T} tokens, segments of {L}")
    seg = m3.mamba3_segment_table(torch.from_numpy(cu).to(device()), T, L)
    torch.cuda.synchronize()
    assert np.array_equal(seg.cpu().numpy().astype(np.int64), expected_segment_table(cu, T, L))


def packed_segmented(d, seg_tokens, chunk):
    import torch
    y, h = m3.mamba3_scan_segmented(d["x"], d["dt"], d.get("lam"), d["theta"], d["B"], d["C"], d.get("A"),
                                    d.get("D"), seg_tokens=seg_tokens, cu_seqlens=d["cu_seqlens"],
                                    h_in=d.get("h_in"), Bprev=d.get("Bprev"), xprev=d.get("xprev"), chunk=chunk,
                                    B_bias=d.get("B_bias"), C_bias=d.get("C_bias"), z=d.get("z"),
                                    bc_norm=d.get("bc_norm", False), bc_eps=d.get("bc_eps", 1e-5),
                                    A_tok=d.get("A_tok"), lam_fixed=d.get("lam_fixed", 0.5))
    torch.cuda.synchronize()
    return from_dev(y), from_dev(h)


def packed_relerr(g, o, cu):
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            worst = max(worst, slab_relerr(g[:, a:b], o[:, a:b]))
    return worst


RAGGED = [0, 1, 1, 129, 130, 400, 700, 700]   # 1-token, empty, ragged and trailing empty members
PACKED_CASES = [
    # (label, config, overrides, cu_seqlens, seg_tokens, extras)
    ("bf16 panel shape", 4, dict(seqlen=700, nheads=2), RAGGED, 128, ("resume",)),
    ("bf16 panel shape, segments off the chunk grid", 4, dict(seqlen=700, nheads=2), RAGGED, 100, ("resume",)),
    ("bf16 panel shape, no resume", 4, dict(seqlen=700, nheads=2), RAGGED, 64, ()),
    ("bf16 SISO", 1, dict(batch=1, seqlen=700, nheads=2), RAGGED, 96, ("resume",)),
    ("bf16 MIMO block + variants", 2, dict(batch=1, seqlen=700, nheads=4, ngroups=2), RAGGED, 80,
     ("resume", "block", "variants")),
    ("f32 tiny", 0, dict(batch=1, seqlen=700), RAGGED, 50, ("resume",)),
    ("f32 grouped + variants", 0, dict(batch=1, seqlen=700, nheads=4, ngroups=2, rank=2), RAGGED, 64,
     ("resume", "block", "variants")),
    ("bf16 panel shape, one segment each", 4, dict(seqlen=700, nheads=2), RAGGED, 4096, ("resume",)),
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=[c[0] for c in PACKED_CASES])
def test_packed_segmented_scan(oracle, case):
    """Packed batches with empty and 1-token members, segmented, against the oracle's
    whole-sequence scan: y per (sequence, head) slab and every sequence's final state."""
    label, cfg, over, cu, L, extras = case
    inp = synth.scan_inputs(cfg, seed=161, **dict(over, packed=False))
    inp["cu_seqlens"] = np.array(cu, dtype=np.int32)
    if "resume" in extras:
        inp = synth.resume_inputs(inp, seed=162)
    if "block" in extras:
        inp = synth.block_inputs(inp, seed=163)
    if "variants" in extras:
        inp = synth.variant_inputs(inp, seed=164, A_tok=True, lam_fixed=0.5, theta_groups=1)
        inp["A"] = None
    tol = TOL_F32 if inp["meta"]["dtype"] == "f32" else TOL_BF16
    note(f"packed segmented scan: {label}, segments of {L}")
    y, h = packed_segmented(upload(inp, device()), L, inp["meta"]["chunk"])
    yo, ho = oracle.scan(oracle_inputs(inp))
    ey, eh = packed_relerr(y, yo, inp["cu_seqlens"]), state_relerr(h, ho)
    note(f"  y relerr {ey:.2e}  h relerr {eh:.2e}")
    assert ey < tol and eh < tol
    if "resume" in extras:   # an empty sequence leaves its entering state as it is
        assert np.array_equal(h[1], inp["h_in"][1].astype(np.float64))


def packed_boundary_states(oracle, inp, L):
    """The oracle's state entering every segment row of a packed batch: a sequence's h_in (or zero)
    for its first segment, else the final state of the sequence's prefix up to the boundary (all
    prefixes scanned as one packed batch of their own)."""
    cu = inp["cu_seqlens"]
    idx, pcu, owner = [], [0], []
    first = {}
    rows = 0
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        n = max(1, -(-(b - a) // L))
        first[i] = rows
        for k in range(1, n):
            idx += list(range(a, a + k * L))
            pcu.append(len(idx))
            owner.append((i, rows + k))
        rows += n
    pre = {}
    for kk, v in oracle_inputs(inp).items():
        if kk in ("x", "dt", "lam", "theta", "B", "C", "z", "A_tok") and v is not None:
            pre[kk] = v[:, idx]
        elif kk in ("h_in", "Bprev", "xprev") and v is not None:
            pre[kk] = v[[i for i, _ in owner]]
        else:
            pre[kk] = v
    pre["cu_seqlens"] = np.array(pcu, dtype=np.int32)
    m = inp["meta"]
    H, N, P = m["nheads"], m["dstate"], m["headdim"]
    out = np.zeros((rows, H, N, P))
    for i, r in first.items():
        if inp.get("h_in") is not None:
            out[r] = inp["h_in"][i]
    if owner:
        _, hp = oracle.scan(pre)
        for j, (_, r) in enumerate(owner):
            out[r] = hp[j]
    return out, rows


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_entering_states(oracle, dtype):
    """The public packed path step by step: the segment table, the segment rows scanned from zero
    states as a packed batch, state passing (which reduces each segment's sums itself), and its
    entering states, boundary tokens and final states against the oracle."""
    import torch
    cfg, L = (0, 48) if dtype == "f32" else (2, 64)
    over = dict(batch=1, seqlen=700) if dtype == "f32" else dict(batch=1, seqlen=700, nheads=2)
    inp = synth.scan_inputs(cfg, seed=171, **over)
    inp["cu_seqlens"] = np.array(RAGGED, dtype=np.int32)
    inp = synth.resume_inputs(inp, seed=172)
    m = inp["meta"]
    d = upload(inp, device())
    note(f"packed state passing {dtype}: entering states, segments of {L}")
    T = m["seqlen"]
    seg_cu = m3.mamba3_segment_table(d["cu_seqlens"], T, L)
    _, U = m3.mamba3_scan_fwd(*(d[k] for k in ("x", "dt", "lam", "theta", "B", "C")), d["A"], None,
                              cu_seqlens=seg_cu, chunk=m["chunk"])
    seg_h, seg_B, seg_x, h_out = m3.mamba3_state_passing(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"],
                                                         d["A"], U=U, h_in=d["h_in"], Bprev=d["Bprev"],
                                                         xprev=d["xprev"], cu_seqlens=d["cu_seqlens"],
                                                         seg_tokens=L)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    ref, rows = packed_boundary_states(oracle, inp, L)
    assert state_relerr(from_dev(seg_h)[:rows], ref) < tol
    _, ho = oracle.scan(oracle_inputs(inp))
    assert state_relerr(from_dev(h_out), ho) < tol
    # boundary tokens exactly: the sequence's own before its first segment, else the token before
    cu = inp["cu_seqlens"]
    xb, Bb = from_dev(seg_x), from_dev(seg_B)
    x_all, B_all = from_dev(d["x"])[0], from_dev(d["B"])[0]
    r = 0
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        n = max(1, -(-(b - a) // L))
        assert np.array_equal(xb[r], from_dev(d["xprev"])[i])
        assert np.array_equal(Bb[r], from_dev(d["Bprev"])[i])
        for k in range(1, n):
            assert np.array_equal(xb[r + k], x_all[a + k * L - 1]) and np.array_equal(Bb[r + k], B_all[a + k * L - 1])
        r += n


def test_packed_segmented_full_size_sampled(oracle):
    """The packed workload (8 sequences, 65536 tokens, 64 heads, N = 128, R = 4, chunk 128) in the
    bench's segmented launch configuration (segments of 4096 tokens): sampled (sequence, head)
    slabs, including the longest sequence (five segments) and the shortest, against the oracle's
    whole-sequence scan of each slab (G = H: a head reads only its own rows)."""
    import torch
    from tests.test_gpu_bf16_scan import _slab_inputs
    c = synth.CONFIGS[4]
    d = synth.torch_scan_inputs(4, device(), seed=4)
    note("packed segmented scan, 65536 tokens, segments of 4096")
    y, h = m3.mamba3_scan_segmented(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"],
                                    seg_tokens=4096, cu_seqlens=d["cu_seqlens"], chunk=c["chunk"])
    torch.cuda.synchronize()
    cu = d["cu_seqlens"].cpu().numpy()
    ln = np.diff(cu)
    S, H = len(cu) - 1, c["nheads"]
    picks = [(int(np.argmax(ln)), 5), (int(np.argmin(ln)), H - 1), (3, 40)]
    for s, hh in picks:
        yo, ho = oracle.scan_slab(_slab_inputs(d, s, hh, cu), 0, 0)
        yg = y[0, int(cu[s]):int(cu[s + 1]), hh]
        ey = float(np.abs(from_dev(yg) - yo).max() / np.abs(yo).max())
        eh = float(np.abs(from_dev(h[s, hh]) - ho).max() / np.abs(ho).max())
        note(f"  slab (s={s}, h={hh}) len={yo.shape[0]}: y relerr {ey:.2e}  h relerr {eh:.2e}")
        assert ey < TOL_BF16 and eh < TOL_BF16
    del d, y, h
    torch.cuda.empty_cache()
