#!/usr/bin/env python3
"""Bench of the Mamba-3 SSM recurrence on one MI355X.

Headline: prefill throughput (tokens/s) of the bf16 chunked MIMO scan on the
packed long-context workload: 8 variable-length sequences totalling 65536
tokens (state reset at each start), 64 heads, head dim 64, state 128, rank 4,
chunk 128. One step = one whole scan of that batch (every step of the hot
path: chunk-local prefixes and rotations, score and output MFMAs, the rank-4
state update, the state pass across chunks, outputs). Inputs are synthetic
(seeded, device-generated) and resident in HBM before timing starts. Its
cpu_baseline is the fp64 oracle on whole slabs drawn like that workload.

The same JSON line carries, under ``secondary``, each with its roofline and
(where it is a forward scan or decode) the oracle timed on the host beside
it: the SISO and MIMO layer scans (8 x 4096 tokens), the tiny fp32 scan, the
MIMO and packed scans with B, C shared by all heads, the fused block
prologue / epilogue (B/C RMS norm, per-head B/C biases, SiLU(z) gate), the
backward of the SISO and MIMO scans, the decode step (batch 256, 64 heads,
N=64, R=4, fp32 state updated in place, 1000 consecutive steps over a ring
of 64 token-input sets), the SISO decode shape (N=128, R=1), decode with
slot-indexed states (continuous batching) and one long sequence scanned
plain and in segments.

Timing: HIP events recorded on the stream the kernels are launched on (torch's
current stream, which the binding passes to the library), W untimed warmup
steps, then exactly K timed steps between device synchronisations.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Mamba-3 SSM prefill tokens/s + decode step \u00b5s at 1 GPU; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
VALU_F32_PEAK_TFS = 157.3      # MI355X fp32 vector, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published


def scan_bytes(c, block=False):
    """Algorithmic HBM bytes of one scan: every input read once, y and the
    final state written once (token inputs bf16, A/D/state fp32); with the
    block prologue / epilogue also the gate z and the two [H, N] fp32 bias
    tables."""
    b, L, H, P, N, R = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    T = b * L
    S = c.get("nseq", b) if c.get("packed") else b
    es = 2 if c.get("dtype", "bf16") == "bf16" else 4
    tok = T * (H * P * R * es * (3 if block else 2)   # x, y (, z)
               + H * es * 2                          # dt, lam
               + H * (N // 2) * es                   # theta
               + 2 * G * N * R * es)                 # B, C
    return tok + S * H * N * P * 4 + 2 * H * 4 + (2 * H * N * 4 if block else 0)


# plain bf16 shapes (N, P, R, Q) the panel kernel runs -> tokens per panel; mirrors the library
PANEL_SHAPES = {(128, 64, 4, 128): 64, (64, 64, 4, 64): 32}


def score_span(c):
    """Tokens over which the score and output contractions run causally: the chunk, except in
    the panel kernel (plain or with the fused block prologue / epilogue), whose two panels of a
    chunk reach each other through the state."""
    N, P, R, Q = c["dstate"], c["headdim"], c["rank"], c["chunk"]
    if c.get("dtype") == "bf16" and (N, P, R, Q) in PANEL_SHAPES:
        return PANEL_SHAPES[(N, P, R, Q)]
    return Q


def scan_flops(c):
    """Algorithmic FLOPs of the chunked form the kernel runs, per token-head (causal half of
    the score and output contractions over the span Qs, inter-chunk output and chunk-state
    update): R^2 (N + P)(Qs + 1) + 4 R N P."""
    L, H, P, N, R = c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    Qs = score_span(c)
    return c["batch"] * L * H * (R * R * (N + P) * (Qs + 1) + 4 * R * N * P)


# (N, P, R) -> chunk length of the MFMA backward (bf16 token inputs); mirrors the library's table
BWD_MFMA_CHUNK = {(128, 64, 1): 32, (64, 64, 1): 32, (64, 64, 4): 16, (128, 64, 2): 16, (128, 64, 4): 8, (64, 64, 2): 32}


def bwd_chunk(c):
    """Chunk length of the backward that runs: the MFMA kernel's for bf16 inputs
    of its shapes, else the VALU kernel's (largest power of two <= 64 whose LDS
    layout fits 160 KB). Mirrors the library's choice."""
    N, P, R = c["dstate"], c["headdim"], c["rank"]
    if c.get("dtype") == "bf16" and (N, P, R) in BWD_MFMA_CHUNK:
        return BWD_MFMA_CHUNK[(N, P, R)]
    for q in (64, 32, 16, 8, 4, 2, 1):
        QR, K = q * R, N // 2
        wk = max(max(QR, K) * (P + 1), 512)
        o = 3 * q * K + 12 * q + q * q + 7 * QR
        o = (o + 3) & ~3
        o += 4 * QR * (N + 1) + 2 * QR * (P + 1) + 2 * N * (P + 1) + 2 * QR * (QR + 1) + 2 * wk
        o += 4 * R * N + 3 * R * P + R + 2 * N + 16
        if o * 4 <= 160 * 1024:
            return q
    return 0


def bwd_bytes(c):
    """Algorithmic HBM bytes of the backward: the forward's token inputs and dy
    read once, their gradients written once (bf16), A read and dA, dD written."""
    b, L, H, P, N, R = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    T = b * L
    es = 2
    return T * (H * P * R * es * 3 + H * es * 4 + H * (N // 2) * es * 2 + 4 * G * N * R * es) + 3 * H * 4


def bwd_flops(c, q):
    """Flops of the chunked backward at chunk q per token-head: the six causal
    chunk contractions (scores, intra outputs, dP, dX, dC, dB: R^2 q/2 (3N + 3P)
    multiply-adds) and seven N x P x R ones (state update, inter output, dX and
    dB state terms, dC inter term, the rotated state, dH)."""
    L, H, P, N, R = c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    return 2 * c["batch"] * L * H * (R * R * q / 2 * (3 * N + 3 * P) + 7 * R * N * P)


def decode_bytes(c, block=False):
    b, H, P, N, R = c["batch"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    es = 2
    return (b * H * N * P * 4 * 2                       # state read + write
            + b * H * P * R * es * (4 if block else 3)  # x, xprev, y (, z)
            + b * G * N * R * es * 3                    # B, C, Bprev
            + b * H * (N // 2) * es + b * H * es * 2    # theta, dt, lam
            + (2 * H * N * 4 if block else 0))          # bias tables


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return t0.elapsed_time(t1) / steps, wall


def m3_config(cfg, **over):
    from state_space_sequence_mamba3_amd import synth
    return dict(synth.CONFIGS[cfg], **over)


def scan_kernel_name(c):
    """The forward kernel that runs a scan of these shapes (mirrors the library's dispatch)."""
    N, P, R, Q = c["dstate"], c["headdim"], c["rank"], c["chunk"]
    if c.get("dtype") != "bf16":
        return f"k_scan_f32<N={N},P={P},R={R},Q={Q}>"
    if (N, P, R, Q) in PANEL_SHAPES:
        return f"k_scan_mimo<N={N},P={P},R={R},Q={Q}" + (",EPI>" if c.get("block") else ">")
    return f"k_scan_bf16<N={N},P={P},R={R},Q={Q}>"


def bench_scan(cfg, steps, warmup, dev, block=False, **over):
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    c = dict(synth.CONFIGS[cfg], **over)
    d = synth.torch_scan_inputs(cfg, dev, seed=cfg, **over)
    if block:
        d = synth.torch_block_inputs(d, dev, seed=cfg)
    y = torch.empty_like(d["x"])
    S = int(d["cu_seqlens"].numel()) - 1 if "cu_seqlens" in d else c["batch"]
    h = torch.empty((S, c["nheads"], c["dstate"], c["headdim"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        m3.mamba3_scan_fwd(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"], y=y, h_out=h,
                           cu_seqlens=d.get("cu_seqlens"), chunk=c["chunk"], stream=stream,
                           B_bias=d.get("B_bias"), C_bias=d.get("C_bias"), z=d.get("z"),
                           bc_norm=d.get("bc_norm", False), bc_eps=d.get("bc_eps", 1e-5))

    ms, wall = timed(step, steps, warmup, stream)
    tokens = c["batch"] * c["seqlen"]
    nbytes, flops = scan_bytes(c, block), scan_flops(dict(c, block=block))
    name = c["name"] + (f" (B, C shared: G={c['ngroups']})" if "ngroups" in over else "")
    name += " + BC norm, BC biases, SiLU gate" if block else ""
    out = dict(workload=name, kernel=scan_kernel_name(dict(c, block=block)), ms=ms, tokens_per_s=tokens / (ms * 1e-3), bytes=nbytes,
               flops=flops,
               hbm_gbs=nbytes / (ms * 1e-3) / 1e9, mfma_tfs=flops / (ms * 1e-3) / 1e12, wall_s=wall)
    del d, y, h
    torch.cuda.empty_cache()
    return out


def measured_peaks(dev):
    """What this GPU reaches outside the library, as context for the published peaks: a plain
    device copy of 1 GiB (bytes read + written per second) and a bf16 GEMM of 8192^3 through
    torch (hipBLASLt)."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    ms, _ = timed(lambda: dst.copy_(src), 20, 3, stream)
    copy_gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    ms, _ = timed(lambda: torch.matmul(a, b, out=c), 20, 3, stream)
    gemm_tfs = 2 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"device_copy_GBps": copy_gbs, "bf16_gemm_8192_TFLOPs": gemm_tfs}


def bench_long(steps, warmup, dev, seqlen=65536, nseg=16):
    """One long SISO sequence (batch 1): the plain scan (one workgroup per head walks every
    token) against the segmented scan (nseg segments per sequence scanned as independent rows,
    their entering states chained by mamba3_state_passing, then scanned again)."""
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    over = dict(batch=1, seqlen=seqlen)
    c = dict(synth.CONFIGS[1], **over)
    d = synth.torch_scan_inputs(1, dev, seed=11, **over)
    y = torch.empty_like(d["x"])
    h = torch.empty((1, c["nheads"], c["dstate"], c["headdim"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    args = [d[k] for k in ("x", "dt", "lam", "theta", "B", "C", "A", "D")]

    def plain():
        m3.mamba3_scan_fwd(*args, y=y, h_out=h, chunk=c["chunk"], stream=stream)

    def segmented():
        m3.mamba3_scan_segmented(*args, nseg=nseg, chunk=c["chunk"], stream=stream)

    out = {}
    for name, fn in (("plain", plain), ("segmented", segmented)):
        ms, _ = timed(fn, steps, warmup, stream)
        out[name] = dict(ms=ms, tokens_per_s=seqlen / (ms * 1e-3))
    out["workload"] = f"SISO scan bf16 1x{seqlen} H64 P64 N128, plain vs {nseg} segments"
    del d, y, h, args
    torch.cuda.empty_cache()
    return out


def bench_packed_segmented(steps, warmup, dev, seg_tokens=(2048, 4096, 8192)):
    """The packed workload (8 sequences, 65536 tokens, N = 128, R = 4) scanned in segments of
    seg_tokens tokens (segment table, state-only scan, state passing, scan), beside the plain scan."""
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    c = dict(synth.CONFIGS[4])
    d = synth.torch_scan_inputs(4, dev, seed=4)
    y = torch.empty_like(d["x"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    args = [d[k] for k in ("x", "dt", "lam", "theta", "B", "C", "A", "D")]
    out = {}
    fns = [("plain", lambda: m3.mamba3_scan_fwd(*args, y=y, cu_seqlens=d["cu_seqlens"], chunk=c["chunk"],
                                                stream=stream))]
    for L in seg_tokens:
        nws = m3.lib().mamba3_scan_segmented_workspace_size(ctypes.byref(m3.ScanSegmentedArgs(
            m3.scan_args(*args, y=y, cu_seqlens=d["cu_seqlens"], chunk=c["chunk"]), 0, None, 0, L)))
        ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
        fns.append((f"segments_{L}", lambda L=L, ws=ws: m3.mamba3_scan_segmented(
            *args, y=y, seg_tokens=L, cu_seqlens=d["cu_seqlens"], chunk=c["chunk"], workspace=ws, stream=stream)))
    for name, fn in fns:
        ms, _ = timed(fn, steps, warmup, stream)
        out[name] = dict(ms=ms, tokens_per_s=c["seqlen"] / (ms * 1e-3))
    out["workload"] = "packed MIMO scan bf16 65536 tok (8 sequences) H64 P64 N128 R4, plain vs segments"
    del d, y, args, fns
    torch.cuda.empty_cache()
    return out


def bench_bwd(cfg, steps, warmup, dev):
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    c = dict(synth.CONFIGS[cfg])
    d = synth.torch_scan_inputs(cfg, dev, seed=cfg)
    g = torch.Generator(device=dev)
    g.manual_seed(100 + cfg)
    dy = torch.randn(d["x"].shape, generator=g, device=dev, dtype=torch.float32).to(d["x"].dtype)
    ws = None
    stream = torch.cuda.current_stream()

    def step():
        nonlocal ws
        out = m3.mamba3_scan_bwd(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"], dy=dy,
                                 cu_seqlens=d.get("cu_seqlens"), workspace=ws, stream=stream)
        return out

    # the workspace is allocated once (chunk states and partial sums), outside the timed region
    import ctypes
    fwd = m3.scan_args(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"], y=None)
    a = m3.ScanBwdArgs(fwd=fwd)   # the size depends on the forward's shapes only
    need = m3.lib().mamba3_scan_bwd_workspace_size(ctypes.byref(a))
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    ms, wall = timed(step, steps, warmup, stream)
    q = bwd_chunk(c)
    mfma = c.get("dtype") == "bf16" and (c["dstate"], c["headdim"], c["rank"]) in BWD_MFMA_CHUNK
    nbytes, flops = bwd_bytes(c), bwd_flops(c, q)
    tokens = c["batch"] * c["seqlen"]
    out = dict(workload=c["name"] + " backward", ms=ms, tokens_per_s=tokens / (ms * 1e-3), bytes=nbytes, flops=flops,
               chunk=q, workspace_bytes=need, hbm_gbs=nbytes / (ms * 1e-3) / 1e9,
               alu_tfs=flops / (ms * 1e-3) / 1e12, wall_s=wall, mfma=mfma)
    del d, dy, ws
    torch.cuda.empty_cache()
    return out


def bench_decode(steps_per_rep, reps, dev, block=False, siso=False, slots=False):
    """The decode step over 1000 consecutive steps. siso: the SISO shape (N=128, R=1) instead of
    MIMO; slots: the states live in a pool twice the batch, each row updating a scattered slot,
    plus one inactive row (slot -1), which also gives this launch a grid of its own in profiles."""
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    c = synth.CONFIGS[3]
    if siso:
        c = dict(c, dstate=128, rank=1, name="SISO decode bf16 batch256 H64 P64 N128")
    ring = c["ring"]
    b, H, P, N, R = c["batch"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    act = b          # active rows
    if slots:
        b += 1       # the inactive row
    g = torch.Generator(device=dev)
    g.manual_seed(3)

    def nrm(shape, mean=0.0, std=1.0):
        return torch.randn(shape, generator=g, device=dev) * std + mean

    import math
    x = nrm((ring, b, H, R, P)).bfloat16()
    dt = torch.nn.functional.softplus(nrm((ring, b, H), -2.0, 0.5)).bfloat16()
    lam = torch.sigmoid(nrm((ring, b, H))).bfloat16()
    th = ((torch.rand((ring, b, H, N // 2), generator=g, device=dev) * 2 - 1) * math.pi).bfloat16()
    B = nrm((ring, b, H, R, N), 0, 1 / math.sqrt(N)).bfloat16()
    C = nrm((ring, b, H, R, N), 0, 1 / math.sqrt(N)).bfloat16()
    A = -torch.exp(nrm((H,), 0, 0.5))
    D = nrm((H,))
    h = nrm((2 * act if slots else b, H, N, P))
    sl = {}
    if slots:   # active rows take half the slots of the pool, in a shuffled order; the last row is inactive
        perm = torch.randperm(2 * act, generator=torch.Generator().manual_seed(5))[:act]
        sl = dict(slots=torch.cat([perm, torch.tensor([-1])]).to(torch.int32).to(dev))
    ys = torch.empty((ring, b, H, R, P), dtype=torch.bfloat16, device=dev)
    blk = {}
    if block:   # fused prologue / epilogue: BC norm, per-head biases ~ U(0.5, 1.5), gate z ~ N(0, 1)
        z = nrm((ring, b, H, R, P)).bfloat16()
        blk = dict(B_bias=torch.rand((H, N), generator=g, device=dev) + 0.5,
                   C_bias=torch.rand((H, N), generator=g, device=dev) + 0.5, bc_norm=True, bc_eps=1e-5)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    state = {"k": 0}

    def zarg(i):
        return dict(blk, z=z[i], **sl) if block else dict(sl)

    def step():
        k = state["k"]
        i, j = k % ring, (k - 1) % ring
        m3.mamba3_decode_step(x[i], dt[i], lam[i], th[i], B[i], C[i], A, D, h=h, y=ys[i], Bprev=B[j], xprev=x[j],
                              stream=stream, **zarg(i))
        state["k"] = k + 1

    ms, wall = timed(step, steps_per_rep, 10, stream)
    nbytes = decode_bytes(c, block) + (b * 4 if slots else 0)   # active rows (+ the slot table)
    us = ms * 1e3
    # per-step event pairs (outside the timed region) for the median
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps_per_rep)]
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    median = per[len(per) // 2]
    # the same steps replayed from a HIP graph (one ring period captured), wall time per step
    graph_us = None
    try:
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            state["k"] = 0
            gstream = torch.cuda.current_stream()
            with torch.cuda.graph(gr, stream=gstream):
                for _ in range(ring):
                    k = state["k"]
                    i, j = k % ring, (k - 1) % ring
                    m3.mamba3_decode_step(x[i], dt[i], lam[i], th[i], B[i], C[i], A, D, h=h, y=ys[i], Bprev=B[j],
                                          xprev=x[j], stream=torch.cuda.current_stream(), **zarg(i))
                    state["k"] = k + 1
        torch.cuda.synchronize()
        reps = max(1, steps_per_rep // ring)
        gr.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for _ in range(reps):
            gr.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - w0) / (reps * ring) * 1e6
    except Exception as exc:  # graph capture unavailable: report the eager figures only
        print(f"# decode graph replay skipped: {exc}", file=sys.stderr)
    name = c["name"] + (" + BC norm, BC biases, SiLU gate" if block else "") + (
        f", slot-indexed states (pool of {2 * act}, one more row inactive)" if slots else "")
    return dict(workload=name, us_per_step=us, median_us=median, graph_wall_us=graph_us, steps=steps_per_rep,
                bytes_per_step=nbytes, hbm_gbs=nbytes / (us * 1e-6) / 1e9, wall_s=wall)


_HOST_THREADS = None


def host_threads():
    """The oracle's OpenMP thread count, read once before any one-thread run (a run on fewer
    threads changes what the OpenMP runtime reports afterwards)."""
    global _HOST_THREADS
    if _HOST_THREADS is None:
        from oracle import oracle as o
        _HOST_THREADS = o.max_threads()
    return _HOST_THREADS


def oracle_rate(cfg, threads, target_s, seqlen, nslab):
    """Throughput of the fp64 oracle (O1, C + OpenMP over (sequence, head) slabs) in
    token-heads/s: whole slabs drawn like config cfg (one sequence of seqlen tokens, nslab
    heads), scanned repeatedly for about target_s seconds on `threads` threads. The oracle's
    cost is linear in tokens, so the rate does not depend on the slab length."""
    from oracle import oracle as o
    from state_space_sequence_mamba3_amd import synth
    inp = synth.scan_inputs(cfg, seed=500 + cfg, batch=1, seqlen=seqlen, nheads=nslab, packed=False)
    inp = {k: v for k, v in inp.items() if k != "meta"}
    done, spent = 0, 0.0
    while spent < target_s:
        t0 = time.perf_counter()
        o.scan(inp, form=1, nthreads=threads)
        spent += time.perf_counter() - t0
        done += nslab * seqlen
    return done / spent, f"{done // seqlen} slabs of {seqlen} tokens ({nslab} distinct) in {spent:.1f} s"


def cpu_baseline(cfg, target_s=10.0, seqlen=8192):
    """The oracle on a bounded sample of config cfg's slabs, on every host thread and on one
    thread; rates in tokens/s of the whole job (token-heads/s divided by the heads)."""
    from oracle import oracle as o
    from state_space_sequence_mamba3_amd import synth
    c = synth.CONFIGS[cfg]
    threads = host_threads()
    rate, sample = oracle_rate(cfg, threads, target_s, seqlen, threads)
    rate1, sample1 = oracle_rate(cfg, 1, max(1.0, target_s / 4), min(seqlen, 1024), 1)
    H = c["nheads"]
    return dict(value=rate / H, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{sample}, drawn like '{c['name']}'; token-heads/s divided by its {H} heads",
                single_thread_value=rate1 / H, single_thread_sample=sample1)


def cpu_baseline_tiny(target_s=1.0):
    """The oracle on the whole tiny fp32 workload (1 x 256 tokens, 4 heads), repeated."""
    from oracle import oracle as o
    from state_space_sequence_mamba3_amd import synth
    c = synth.CONFIGS[0]
    threads = host_threads()
    inp = {k: v for k, v in synth.scan_inputs(0).items() if k != "meta"}
    n, spent = 0, 0.0
    while spent < target_s:
        t0 = time.perf_counter()
        o.scan(inp, form=1, nthreads=threads)
        spent += time.perf_counter() - t0
        n += 1
    return dict(value=n * c["batch"] * c["seqlen"] / spent, unit="tokens/s", ms_per_step=spent / n * 1e3,
                cores=threads, kind="oracle", sample=f"the whole workload {n} times in {spent:.1f} s")


def cpu_baseline_decode(target_s=4.0, rows=16):
    """The oracle's decode step on `rows` batch rows of the decode workload (all 64 heads),
    stepped repeatedly; the time per step is scaled to the batch of 256."""
    import numpy as np
    from oracle import oracle as o
    from state_space_sequence_mamba3_amd import synth
    c = synth.CONFIGS[3]
    threads = host_threads()
    inp = synth.decode_inputs(3, seed=503, batch=rows, ring=1)
    tok = {k: inp[k][0] for k in ("x", "dt", "lam", "theta", "B", "C")}
    tok.update(A=inp["A"], D=inp["D"], Bprev=inp["Bprev"], xprev=inp["xprev"])
    h = inp["h"].astype(np.float64)
    n, spent = 0, 0.0
    while spent < target_s:
        t0 = time.perf_counter()
        _, h = o.decode(tok, h, nthreads=threads)
        spent += time.perf_counter() - t0
        n += 1
    us = spent / n * 1e6 * c["batch"] / rows
    return dict(value=us, unit="us/step", cores=threads, kind="oracle",
                sample=f"{n} steps of {rows} batch rows x {c['nheads']} heads in {spent:.1f} s; "
                       f"time scaled to the batch of {c['batch']}")


def traffic_record(kernel):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, if they were taken on the current kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "state_space_sequence_mamba3_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    return rec.get("bytes_per_launch")


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    """Kernel name without the argument list and namespaces."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("m3::(anonymous namespace)::", "").replace("at::native::(anonymous namespace)::", "at::native::")
    depth = 0
    for i, ch in enumerate(n):   # cut the argument list: the first '(' outside template brackets
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return n[:i]
    return n


def summarize_stats(stats_dir, out_md, command):
    """Writes a short text summary of a rocprofv3 --kernel-trace --stats run: the library's
    kernels from the per-dispatch trace, one row per (kernel, workgroups), so that launches of
    one kernel on different workloads are told apart."""
    from collections import defaultdict
    groups = defaultdict(list)
    other, other_ms = set(), 0.0
    for r in _csv_rows(os.path.join(stats_dir, "run_kernel_trace.csv")):
        ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        if not any(k in r["Kernel_Name"] for k in ("k_scan", "k_decode", "k_bwd", "k_segment_sums", "k_state_passing")):
            other.add(r["Kernel_Name"])
            other_ms += ns / 1e6
            continue
        wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        groups[(r["Kernel_Name"], wg)].append((float(r["Start_Timestamp"]), ns))
    lines = ["# rocprofv3 kernel statistics", "", "Command (run from /tmp with TMPDIR=/tmp; R = repository root):", "",
             "```", command, "```", "",
             "Per (kernel, workgroups), from the run's kernel trace. The bench times the last half of each "
             "workload's launches (its warmup equals its timed steps by default): the last column averages those.", "",
             "| kernel | workgroups | calls | average us | min us | max us | total ms | average of the last half us |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, wg), tv in sorted(groups.items(), key=lambda kv: -sum(n for _, n in kv[1])):
        v = [n for _, n in sorted(tv)]
        last = v[len(v) // 2:]
        lines.append(f"| `{_short(name)}` | {wg} | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {min(v) / 1e3:.2f} | "
                     f"{max(v) / 1e3:.2f} | {sum(v) / 1e6:.3f} | {sum(last) / len(last) / 1e3:.2f} |")
    lines += ["", f"Not listed: {len(other)} other kernels (torch's input generation and copies), {other_ms:.3f} ms in total."]
    open(out_md, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


def summarize_traffic(fetch_dir, write_dir, out_dir, commands, copy_bytes=1 << 30):
    """Turns rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch; each
    may be several runs, comma-separated) of `bench.py --copy-calibration` into
    HBM bytes per launch of the scan and decode kernels, each counter scaled by
    its reading on the plain 1 GiB device copy. Writes traffic_<kernel>.json records (read by the bench
    while the kernel source is unchanged) and a text summary."""
    import hashlib
    from collections import defaultdict

    def per_dispatch(dirs, counter):
        """{(kernel, workgroups): [bytes per dispatch]} over one or more runs (comma-separated dirs)"""
        by = defaultdict(list)
        for d in dirs.split(","):
            agg, names = defaultdict(float), {}
            for r in _csv_rows(os.path.join(d, "run_counter_collection.csv")):
                if r["Counter_Name"] == counter:
                    agg[r["Dispatch_Id"]] += float(r["Counter_Value"])
                    names[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            for k, v in agg.items():
                by[names[k]].append(v * 1024.0)
        return by

    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    # the calibration copies: the device-to-device copy kernel's dispatches of about 1 GiB
    copy_f = [v for (n, _), vs in fetch.items() if "copyBuffer" in n for v in vs if v > copy_bytes / 2]
    copy_w = [v for (n, _), vs in write.items() if "copyBuffer" in n for v in vs if v > copy_bytes / 2]
    if not copy_f or not copy_w:
        raise SystemExit("no copy kernel found in the counter runs (run bench.py with --copy-calibration)")
    kf, kw = copy_bytes / (sum(copy_f) / len(copy_f)), copy_bytes / (sum(copy_w) / len(copy_w))
    # the headline SISO scan, the decode steps, the SISO backward, and the fused block prologue /
    # epilogue variants (demangled or mangled names, as rocprofv3 prints them; workgroups of the
    # bench's launch: 8 x 64 (sequence, head) slabs, 256 x 64 decode rows, 257 x 64 with slots)
    dec = ("k_decode_colIDF16bLi64ELi4ELb0E", "k_decode_col<__bf16, 64, 4, false>")
    kernels = {"scan_bf16": ("scan_bf16.hip", ("Cfg<128, 64, 1, 64, 4, 32, 64, false, true>",), 512),
               "scan_bf16_mimo": ("scan_mimo.hip", ("MCfg<64, 64, 4, 64, 4, 32, true, 2, false>",), 512),
               "scan_bf16_packed": ("scan_mimo.hip", ("MCfg<128, 64, 4, 128, 8, 64, true, 2, false>",), 512),
               "scan_bf16_block": ("scan_bf16.hip", ("Cfg<128, 64, 1, 64, 4, 32, 64, true, true>",), 512),
               "decode": ("decode.hip", dec, 16384),
               "decode_slots": ("decode.hip", dec, 16448),
               "decode_block": ("decode.hip", ("k_decode_colIDF16bLi64ELi4ELb1E", "k_decode_col<__bf16, 64, 4, true>"),
                                16384),
               "decode_siso": ("decode.hip", ("k_decode_colIDF16bLi128ELi1ELb0E", "k_decode_col<__bf16, 128, 1, false>"),
                               16384),
               "scan_bwd": ("scan_bwd.hip", ("BCfg<128, 64, 1, 32, 8>",), 512),
               # the backward's chunk states: the state-only forward scan at chunk 32
               "scan_bwd_states": ("scan_bf16.hip", ("Cfg<128, 64, 1, 32, 4, 32, 32, false, false>",), 512)}
    md = ["# HBM traffic per launch from rocprofv3 counters", "", "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):",
          "", "```", *commands, "```", "",
          f"Calibration: a plain 1 GiB device copy reads {sum(copy_f) / len(copy_f) / 2**30:.4f} GiB by FETCH_SIZE and writes "
          f"{sum(copy_w) / len(copy_w) / 2**30:.4f} GiB by WRITE_SIZE; scale factors {kf:.4f} (fetch), {kw:.4f} (write).", "",
          "| kernel | workgroups | dispatches | fetch MB | write MB | traffic MB per launch |", "|---|---|---|---|---|---|"]
    for key, (src, pats, wg) in kernels.items():
        hit = lambda nw: nw[1] == wg and any(p in nw[0] for p in pats)
        fs = [v for nw, vs in fetch.items() if hit(nw) for v in vs]
        ws = [v for nw, vs in write.items() if hit(nw) for v in vs]
        if not fs or not ws:
            continue
        fb, wb = kf * sum(fs) / len(fs), kw * sum(ws) / len(ws)
        name = next(nw[0] for nw in fetch if hit(nw))
        srcp = os.path.join(ROOT, "state_space_sequence_mamba3_amd", "csrc", src)
        rec = {"kernel": _short(name), "source": src,
               "source_sha256": hashlib.sha256(open(srcp, "rb").read()).hexdigest(),
               "fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb, "dispatches": len(fs),
               "copy_scale_fetch": kf, "copy_scale_write": kw, "workgroups": wg}
        json.dump(rec, open(os.path.join(out_dir, f"traffic_{key}.json"), "w"), indent=1)
        md.append(f"| `{_short(name)}` | {wg} | {len(fs)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} |")
    out_md = os.path.join(out_dir, "traffic_scan_bf16_and_decode_bench_workloads.md")
    open(out_md, "w").write("\n".join(md) + "\n")
    print(f"wrote {out_md}")


MFMA_KERNELS = {"scan_bf16_packed": ("scan_mimo.hip", ("MCfg<128, 64, 4, 128, 8, 64, true, 2, false>",), 512),
                "scan_bf16_mimo": ("scan_mimo.hip", ("MCfg<64, 64, 4, 64, 4, 32, true, 2, false>",), 512),
                "scan_bf16": ("scan_bf16.hip", ("Cfg<128, 64, 1, 64, 4, 32, 64, false, true>",), 512)}
CU_COUNT = 256
XCD_COUNT = 8
SIMDS_PER_CU = 4


def summarize_mfma(pmc_dir, out_dir, command):
    """Turns one rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
    GRBM_GUI_ACTIVE into per-launch MFMA records of the scan kernels: the MFMA busy share of the
    CUs' active cycles (busy cycles / (GUI-active cycles x CUs), rocprof's MFMA utilisation) and the
    bf16 MFMA work the counters saw (MOPS x 512 flops). Writes mfma_<kernel>.json records (read by
    the bench while the kernel source is unchanged) and a text summary. On MI355X GRBM_GUI_ACTIVE
    sums the 8 XCDs (a per-XCD share divided by the 2.4 GHz clock gives the kernel's duration), and
    the MFMA busy cycles sum over the 1024 SIMDs (they equal the counted flops over the 1024 bf16
    flops a SIMD retires per cycle), so the busy share is busy / (GUI / 8 x 1024)."""
    import hashlib
    from collections import defaultdict
    agg, names = defaultdict(lambda: defaultdict(float)), {}
    for r in _csv_rows(os.path.join(pmc_dir, "run_counter_collection.csv")):
        agg[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
    md = ["# MFMA counters per launch from rocprofv3", "", "Command (run from /tmp with TMPDIR=/tmp; R = repository root):",
          "", "```", command, "```", "",
          f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCD_COUNT} XCDs x {CU_COUNT * SIMDS_PER_CU} SIMDs): "
          "GRBM_GUI_ACTIVE sums the XCDs and the busy cycles sum the SIMDs. Counted bf16 work = "
          "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops (it includes the masked halves of diagonal tiles).", "",
          "| kernel | workgroups | dispatches | MFMA busy cycles | GUI active cycles | MFMA busy | counted bf16 GFLOP |",
          "|---|---|---|---|---|---|---|"]
    for key, (src, pats, wg) in MFMA_KERNELS.items():
        ds = [d for d, nw in names.items() if nw[1] == wg and any(p in nw[0] for p in pats)]
        if not ds:
            continue
        mean = lambda c: sum(agg[d][c] for d in ds) / len(ds)
        busy, gui, mops = mean("SQ_VALU_MFMA_BUSY_CYCLES"), mean("GRBM_GUI_ACTIVE"), mean("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        srcp = os.path.join(ROOT, "state_space_sequence_mamba3_amd", "csrc", src)
        rec = {"kernel": _short(names[ds[0]][0]), "source": src,
               "source_sha256": hashlib.sha256(open(srcp, "rb").read()).hexdigest(), "dispatches": len(ds),
               "workgroups": wg, "mfma_busy_cycles": busy, "gui_active_cycles": gui, "mops_bf16": mops,
               "simds": CU_COUNT * SIMDS_PER_CU, "xcds": XCD_COUNT,
               "busy_frac": busy / (gui / XCD_COUNT * CU_COUNT * SIMDS_PER_CU) if gui else None,
               "counter_flops": mops * 512}
        json.dump(rec, open(os.path.join(out_dir, f"mfma_{key}.json"), "w"), indent=1)
        md.append(f"| `{rec['kernel']}` | {wg} | {len(ds)} | {busy:.4g} | {gui:.4g} | "
                  f"{rec['busy_frac'] if rec['busy_frac'] is not None else float('nan'):.3f} | {mops * 512 / 1e9:.1f} |")
    out_md = os.path.join(out_dir, "mfma_scan_bf16_bench_workloads.md")
    open(out_md, "w").write("\n".join(md) + "\n")
    print(f"wrote {out_md}")


def summarize_counters(pmc_dir, out_md, command, kernels=("k_scan_mimo", "k_scan_bf16", "k_scan_bwd_mfma")):
    """Per-dispatch averages of every counter of one rocprofv3 --pmc run, per (kernel, workgroups),
    for the library's kernels (instruction mixes, wait and busy cycles): a text summary."""
    from collections import defaultdict
    agg, names = defaultdict(lambda: defaultdict(float)), {}
    for r in _csv_rows(os.path.join(pmc_dir, "run_counter_collection.csv")):
        agg[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
    groups = defaultdict(list)
    for d, nw in names.items():
        if any(k in nw[0] for k in kernels):
            groups[(_short(nw[0]), nw[1])].append(d)
    counters = sorted({c for d in agg for c in agg[d]})
    md = ["# rocprofv3 counters per dispatch", "", "Command (run from /tmp with TMPDIR=/tmp; R = repository root):", "",
          "```", command, "```", "",
          "Per (kernel, workgroups): the average over its dispatches of each counter summed over the GPU "
          "(SQ_*_CYCLES and SQ_WAIT_* count in units of 4 cycles).", "",
          "| kernel | workgroups | dispatches | " + " | ".join(counters) + " |",
          "|---|---|---|" + "---|" * len(counters)]
    for (k, wg), ds in sorted(groups.items()):
        md.append(f"| `{k}` | {wg} | {len(ds)} | " +
                  " | ".join(f"{sum(agg[d][c] for d in ds) / len(ds):.4g}" for c in counters) + " |")
    open(out_md, "w").write("\n".join(md) + "\n")
    print(f"wrote {out_md}")


def counter_record(key):
    """MFMA counters per launch from a committed rocprofv3 --pmc record (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE), if taken on the current kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"mfma_{key}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "state_space_sequence_mamba3_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    return rec


def scan_roofline(r, traffic_key=None, counter_key=None):
    """Roofline entry of a scan line: the binding roofline (whichever of HBM bytes and MFMA flops
    needs more time at peak), with the other figure beside it, and the counter records."""
    mfma_bound = r["flops"] / (MFMA_BF16_PEAK_TFS * 1e12) > r["bytes"] / (HBM_PEAK_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": r["mfma_tfs"], "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
             "frac": r["mfma_tfs"] / MFMA_BF16_PEAK_TFS, "hbm_gbs": r["hbm_gbs"],
             "hbm_frac": r["hbm_gbs"] / HBM_PEAK_GBS} if mfma_bound else
            {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": r["hbm_gbs"] / HBM_PEAK_GBS, "mfma_tflops": r["mfma_tfs"],
             "mfma_frac": r["mfma_tfs"] / MFMA_BF16_PEAK_TFS})
    roof["traffic"] = traffic_record(traffic_key) if traffic_key else None
    roof.update(bytes_per_launch=r["bytes"], flops_per_launch=r["flops"], launch_ms=r["ms"])
    cr = counter_record(counter_key) if counter_key else None
    if cr:
        # counter figures beside the algorithmic ones: MFMA busy share of the CUs' active cycles,
        # and the bf16 MFMA work the counters saw (it includes masked tiles and padding)
        roof["mfma_busy_counter"] = cr["busy_frac"]
        roof["mfma_counter_tflops"] = cr["counter_flops"] / (r["ms"] * 1e-3) / 1e12
        roof["mfma_counter_frac"] = roof["mfma_counter_tflops"] / MFMA_BF16_PEAK_TFS
    return roof


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-stats":
        # bench.py --summarize-stats STATS_DIR OUT_MD COMMAND
        summarize_stats(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-traffic":
        # bench.py --summarize-traffic FETCH_DIR WRITE_DIR OUT_DIR COMMAND...
        summarize_traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters PMC_DIR OUT_MD COMMAND
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-mfma":
        # bench.py --summarize-mfma PMC_DIR OUT_DIR COMMAND
        summarize_mfma(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["scan", "decode", "bwd", "long", "all"], default="all")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}); the scan and decode shard over "
              "(sequence, head) with no communication, so each GPU would run this same workload share",
              file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    import state_space_sequence_mamba3_amd as m3
    m3.lib()

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": src.numel() * 4, "launches": 3}), flush=True)
        del src, dst

    K, W = args.steps, args.warmup
    res = {}
    # the layer workloads take a fraction of a millisecond: more launches for a stable figure. They
    # run first, so the headline's timed steps do not take the fresh GPU's first launches.
    KL, WL = max(K, 50), max(W, 20)
    if args.only in ("scan", "all"):
        res["siso"] = bench_scan(1, KL, WL, dev)
        print(f"# siso scan {res['siso']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["mimo"] = bench_scan(2, KL, WL, dev)
        print(f"# mimo scan {res['mimo']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["tiny"] = bench_scan(0, KL, WL, dev)
        print(f"# tiny fp32 scan {res['tiny']['ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)
        res["packed"] = bench_scan(4, K, W, dev)
        print(f"# packed MIMO scan {res['packed']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only == "all":
        # B and C shared by all heads (one group), as the MIMO layer can be configured
        res["mimo_g1"] = bench_scan(2, KL, WL, dev, ngroups=1)
        print(f"# mimo scan G=1 {res['mimo_g1']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["packed_g1"] = bench_scan(4, K, W, dev, ngroups=1)
        print(f"# packed scan G=1 {res['packed_g1']['ms']:.3f} ms", file=sys.stderr, flush=True)
        # the fused block prologue / epilogue on
        res["siso_block"] = bench_scan(1, KL, WL, dev, block=True)
        print(f"# siso scan + block {res['siso_block']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["mimo_block"] = bench_scan(2, KL, WL, dev, block=True)
        print(f"# mimo scan + block {res['mimo_block']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["packed_block"] = bench_scan(4, K, W, dev, block=True)
        print(f"# packed scan + block {res['packed_block']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only in ("bwd", "all"):
        # the backward: a few steps, each is a whole backward of the batch
        res["siso_bwd"] = bench_bwd(1, 3, 1, dev)
        print(f"# siso backward {res['siso_bwd']['ms']:.2f} ms", file=sys.stderr, flush=True)
        res["mimo_bwd"] = bench_bwd(2, 3, 1, dev)
        print(f"# mimo backward {res['mimo_bwd']['ms']:.2f} ms", file=sys.stderr, flush=True)
    if args.only in ("decode", "all"):
        res["decode"] = bench_decode(1000, 1, dev)
        print(f"# decode {res['decode']['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    if args.only == "all":
        res["decode_block"] = bench_decode(1000, 1, dev, block=True)
        print(f"# decode + block {res['decode_block']['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    if args.only in ("decode", "all"):
        res["decode_siso"] = bench_decode(1000, 1, dev, siso=True)
        print(f"# SISO decode {res['decode_siso']['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)
        res["decode_slots"] = bench_decode(1000, 1, dev, slots=True)
        print(f"# decode with slots {res['decode_slots']['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)

    if args.only in ("long", "all"):
        res["long"] = bench_long(max(3, K // 4), max(1, W // 4), dev)
        print(f"# long sequence: plain {res['long']['plain']['ms']:.3f} ms, segmented "
              f"{res['long']['segmented']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["packed_segmented"] = bench_packed_segmented(max(3, K // 4), max(1, W // 4), dev)
        print("# packed segmented: " + ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in res["packed_segmented"].items()
                                                 if isinstance(v, dict)), file=sys.stderr, flush=True)

    peaks = measured_peaks(dev) if args.only == "all" else None

    # the oracle on the host, beside each forward workload (a baseline, not a target)
    cpu = {}
    if not args.no_cpu_baseline:
        if "packed" in res:
            cpu["packed"] = cpu_baseline(4)
        if "siso" in res:
            cpu["siso"] = cpu_baseline(1, target_s=5.0, seqlen=4096)
        if "mimo" in res:
            cpu["mimo"] = cpu_baseline(2, target_s=5.0, seqlen=4096)
        if "tiny" in res:
            cpu["tiny"] = cpu_baseline_tiny()
        if "decode" in res:
            cpu["decode"] = cpu_baseline_decode()
        print("# oracle timed", file=sys.stderr, flush=True)

    if "packed" in res:
        r = res["packed"]
        c = m3_config(4)
        line = {
            "metric": METRIC,
            "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, device-generated)",
            "config": {"workload": r["workload"], "batch": 1, "seqlen": c["seqlen"], "nseq": c["nseq"],
                       "nheads": c["nheads"], "headdim": c["headdim"], "dstate": c["dstate"], "rank": c["rank"],
                       "ngroups": c["nheads"], "chunk": c["chunk"], "parallelism": "single GPU"},
            "roofline": dict(scan_roofline(r, "scan_bf16_packed", "scan_bf16_packed"), kernel=r["kernel"]),
            "cpu_baseline": cpu.get("packed"),
        }
    else:
        line = {"metric": METRIC, "value": None}
    sec = {}
    for k, tk in (("siso", "scan_bf16"), ("mimo", "scan_bf16_mimo"), ("tiny", None), ("mimo_g1", None),
                  ("packed_g1", None), ("siso_block", "scan_bf16_block"), ("mimo_block", None),
                  ("packed_block", None)):
        if k in res:
            r = res[k]
            sec[k] = {"workload": r["workload"], "ms": r["ms"], "tokens_per_s": r["tokens_per_s"],
                      "kernel": r["kernel"], "roofline": scan_roofline(r, tk, tk)}
            if k in cpu:
                sec[k]["oracle"] = cpu[k]
    for k in ("siso_bwd", "mimo_bwd"):
        if k in res:
            r = res[k]
            # binding roofline: the kernel's arithmetic (bf16 MFMA, or fp32 vector for the VALU
            # kernel) or HBM bytes, whichever needs more time at peak
            cpeak, cname = (MFMA_BF16_PEAK_TFS, "mfma") if r["mfma"] else (VALU_F32_PEAK_TFS, "alu")
            c_bound = r["flops"] / (cpeak * 1e12) > r["bytes"] / (HBM_PEAK_GBS * 1e9)
            roof = ({"bound": cname, "achieved": r["alu_tfs"], "peak": cpeak, "unit": "TFLOP/s",
                     "frac": r["alu_tfs"] / cpeak, "hbm_gbs": r["hbm_gbs"]} if c_bound else
                    {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["hbm_gbs"] / HBM_PEAK_GBS, "tflops": r["alu_tfs"], "tflops_peak": cpeak})
            roof.update(bytes_per_launch=r["bytes"], flops_per_launch=r["flops"], chunk=r["chunk"])
            if k == "siso_bwd":
                # the whole backward: the state-only forward scan that writes the chunk states,
                # then the backward kernel
                tb, ts = traffic_record("scan_bwd"), traffic_record("scan_bwd_states")
                roof["traffic"] = tb + ts if tb is not None and ts is not None else None
            sec[k] = {"workload": r["workload"], "ms": r["ms"], "tokens_per_s": r["tokens_per_s"],
                      "workspace_bytes": r["workspace_bytes"], "roofline": roof}
    for k in ("decode", "decode_block", "decode_siso", "decode_slots"):
        if k in res:
            r = res[k]
            sec[k] = {"workload": r["workload"], "us_per_step": r["us_per_step"], "median_us": r["median_us"],
                      "graph_wall_us": r["graph_wall_us"], "steps": r["steps"],
                      "roofline": {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": r["hbm_gbs"] / HBM_PEAK_GBS,
                                   "bytes_per_launch": r["bytes_per_step"],
                                   "traffic": traffic_record(k)}}
            if k in cpu:
                sec[k]["oracle"] = cpu[k]
    if "long" in res:
        sec["long_sequence"] = res["long"]
    if "packed_segmented" in res:
        sec["packed_segmented"] = res["packed_segmented"]
    line["secondary"] = sec
    if peaks:
        line["measured_peaks"] = peaks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
