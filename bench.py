#!/usr/bin/env python3
"""Bench of the Mamba-3 SSM recurrence on one MI355X.

Headline: prefill throughput (tokens/s) of the bf16 chunked scan on the SISO
layer workload (batch 8 x 4096 tokens, 64 heads, head dim 64, state 128,
rank 1, chunk 64). One step = one whole scan of that batch (every step of the
hot path: chunk-local prefixes and rotations, score and output MFMAs, state
update, outputs). Inputs are synthetic (seeded, device-generated) and resident
in HBM before timing starts. The same JSON line also carries the decode step
(batch 256, 64 heads, N=64, R=4, fp32 state updated in place, 1000
consecutive steps over a ring of 64 token-input sets) and the MIMO and packed
MIMO scans as secondary figures, each with its roofline.

Timing: HIP events recorded on the stream the kernels are launched on (torch's
current stream, which the binding passes to the library), W untimed warmup
steps, then exactly K timed steps between device synchronisations.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published


def scan_bytes(c):
    """Algorithmic HBM bytes of one scan: every input read once, y and the
    final state written once (token inputs bf16, A/D/state fp32)."""
    b, L, H, P, N, R = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    T = b * L
    S = c.get("nseq", b) if c.get("packed") else b
    es = 2
    tok = T * (H * P * R * es * 2          # x, y
               + H * es * 2                # dt, lam
               + H * (N // 2) * es         # theta
               + 2 * G * N * R * es)       # B, C
    return tok + S * H * N * P * 4 + 2 * H * 4


def scan_flops(c):
    """Algorithmic FLOPs of the chunked method per token-head (causal half of
    the score and output contractions, inter-chunk output and chunk-state
    update): R^2 (N + P)(Q + 1) + 4 R N P."""
    L, H, P, N, R, Q = c["seqlen"], c["nheads"], c["headdim"], c["dstate"], c["rank"], c["chunk"]
    return c["batch"] * L * H * (R * R * (N + P) * (Q + 1) + 4 * R * N * P)


def decode_bytes(c):
    b, H, P, N, R = c["batch"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
    G = c.get("ngroups", H)
    es = 2
    return (b * H * N * P * 4 * 2                       # state read + write
            + b * H * P * R * es * 3                    # x, xprev, y
            + b * G * N * R * es * 3                    # B, C, Bprev
            + b * H * (N // 2) * es + b * H * es * 2)   # theta, dt, lam


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


def bench_scan(cfg, steps, warmup, dev):
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    c = synth.CONFIGS[cfg]
    d = synth.torch_scan_inputs(cfg, dev, seed=cfg)
    y = torch.empty_like(d["x"])
    S = int(d["cu_seqlens"].numel()) - 1 if "cu_seqlens" in d else c["batch"]
    h = torch.empty((S, c["nheads"], c["dstate"], c["headdim"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        m3.mamba3_scan_fwd(d["x"], d["dt"], d["lam"], d["theta"], d["B"], d["C"], d["A"], d["D"], y=y, h_out=h,
                           cu_seqlens=d.get("cu_seqlens"), chunk=c["chunk"], stream=stream)

    ms, wall = timed(step, steps, warmup, stream)
    tokens = c["batch"] * c["seqlen"]
    nbytes, flops = scan_bytes(c), scan_flops(c)
    out = dict(workload=c["name"], ms=ms, tokens_per_s=tokens / (ms * 1e-3), bytes=nbytes, flops=flops,
               hbm_gbs=nbytes / (ms * 1e-3) / 1e9, mfma_tfs=flops / (ms * 1e-3) / 1e12, wall_s=wall)
    del d, y, h
    torch.cuda.empty_cache()
    return out


def bench_decode(steps_per_rep, reps, dev):
    import torch
    import state_space_sequence_mamba3_amd as m3
    from state_space_sequence_mamba3_amd import synth
    c = synth.CONFIGS[3]
    ring = c["ring"]
    b, H, P, N, R = c["batch"], c["nheads"], c["headdim"], c["dstate"], c["rank"]
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
    h = nrm((b, H, N, P))
    ys = torch.empty((ring, b, H, R, P), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    state = {"k": 0}

    def step():
        k = state["k"]
        i, j = k % ring, (k - 1) % ring
        m3.mamba3_decode_step(x[i], dt[i], lam[i], th[i], B[i], C[i], A, D, h=h, y=ys[i], Bprev=B[j], xprev=x[j],
                              stream=stream)
        state["k"] = k + 1

    ms, wall = timed(step, steps_per_rep, 10, stream)
    nbytes = decode_bytes(c)
    us = ms * 1e3
    return dict(workload=c["name"], us_per_step=us, steps=steps_per_rep, bytes_per_step=nbytes,
                hbm_gbs=nbytes / (us * 1e-6) / 1e9, wall_s=wall)


def cpu_baseline(target_s=12.0):
    """The fp64 oracle (O1, C + OpenMP over (sequence, head) slabs) on whole
    slabs of the headline workload (4096 tokens, N=128, P=64, R=1); its
    throughput is scaled to the whole batch (8 sequences x 64 heads)."""
    from oracle import oracle as o
    from state_space_sequence_mamba3_amd import synth
    import numpy as np
    c = synth.CONFIGS[1]
    threads = o.max_threads()
    total_slabs = c["batch"] * c["nheads"]
    nslab = min(total_slabs, 2 * threads)
    inp = synth.scan_inputs(1, seed=500, batch=1, nheads=nslab)
    inp = {k: v for k, v in inp.items() if k != "meta"}
    done, spent = 0, 0.0
    while spent < target_s and done < 8 * total_slabs:
        t0 = time.perf_counter()
        o.scan(inp, form=1, nthreads=threads)
        spent += time.perf_counter() - t0
        done += nslab
    tokens = c["batch"] * c["seqlen"]
    whole_job_s = spent * total_slabs / done
    return dict(value=tokens / whole_job_s, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{done} (sequence, head) slabs of the 8x4096 SISO workload ({nslab} distinct, "
                       f"4096 tokens each; the batch has {total_slabs}) in {spent:.1f} s; rate scaled to the "
                       f"whole batch")


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["scan", "decode", "all"], default="all")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the scan and decode shard over (sequence, head) with no communication, see DESIGN.md", file=sys.stderr)
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

    res = {}
    if args.only in ("scan", "all"):
        res["siso"] = bench_scan(1, args.steps, args.warmup, dev)
        print(f"# siso scan {res['siso']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only == "all":
        res["mimo"] = bench_scan(2, args.steps, args.warmup, dev)
        print(f"# mimo scan {res['mimo']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["packed"] = bench_scan(4, max(2, args.steps // 2), max(1, args.warmup // 2), dev)
        print(f"# packed scan {res['packed']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only in ("decode", "all"):
        res["decode"] = bench_decode(1000, 1, dev)
        print(f"# decode {res['decode']['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline and args.only in ("scan", "all"):
        cpu = cpu_baseline()

    if "siso" in res:
        s = res["siso"]
        tr = traffic_record("scan_bf16")
        line = {
            "metric": "Mamba-3 SSM prefill tokens/s (SISO scan) + decode step us; % of HBM/MFMA roofline",
            "value": s["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": s["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, device-generated)",
            "config": {"workload": s["workload"], "batch": 8, "seqlen": 4096, "nheads": 64, "headdim": 64,
                       "dstate": 128, "rank": 1, "chunk": 64, "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": s["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": s["hbm_gbs"] / HBM_PEAK_GBS, "traffic": tr,
                         "kernel": "k_scan_bf16<N=128,P=64,R=1,Q=64>", "bytes_per_launch": s["bytes"],
                         "launch_ms": s["ms"], "mfma_tflops": s["mfma_tfs"],
                         "mfma_frac": s["mfma_tfs"] / MFMA_BF16_PEAK_TFS},
            "cpu_baseline": cpu,
        }
    else:
        line = {"metric": "Mamba-3 SSM decode step us", "value": None}
    sec = {}
    for k in ("mimo", "packed"):
        if k in res:
            r = res[k]
            sec[k] = {"workload": r["workload"], "ms": r["ms"], "tokens_per_s": r["tokens_per_s"],
                      "roofline": {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": r["hbm_gbs"] / HBM_PEAK_GBS, "mfma_tflops": r["mfma_tfs"],
                                   "mfma_frac": r["mfma_tfs"] / MFMA_BF16_PEAK_TFS}}
    if "decode" in res:
        r = res["decode"]
        sec["decode"] = {"workload": r["workload"], "us_per_step": r["us_per_step"], "steps": r["steps"],
                         "roofline": {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": r["hbm_gbs"] / HBM_PEAK_GBS,
                                      "bytes_per_launch": r["bytes_per_step"],
                                      "traffic": traffic_record("decode")}}
    line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
