"""The allocation-free segmented scan (mamba3_scan_segmented_noalloc) against the
segmented scan with a caller workspace (mamba3_scan_segmented), through the C ABI:
two calls in a row, the second on a smaller input, each bitwise equal to the
workspace entry point's result (same kernels, same inputs). Its argument errors
and size limit are checked on the CPU (tests/test_abi.py)."""
import numpy as np
import pytest

import state_space_sequence_mamba3_amd as m3
from state_space_sequence_mamba3_amd import synth
from tests.gpu_util import device, note, upload

pytestmark = pytest.mark.gpu


def _both(inp, nseg, chunk):
    import torch
    d = upload(inp, device())
    args = [d[k] for k in ("x", "dt", "lam", "theta", "B", "C", "A", "D")]
    kw = dict(nseg=nseg, chunk=chunk, h_in=d.get("h_in"), Bprev=d.get("Bprev"), xprev=d.get("xprev"))
    y0, h0 = m3.mamba3_scan_segmented(*args, **kw)
    y1, h1 = m3.mamba3_scan_segmented_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return (y0, h0), (y1, h1)


def _bits(t):
    import torch
    return t.contiguous().view(-1).view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("cfg", [1, 2])
def test_noalloc_matches_workspace_entry_twice(cfg):
    # first call: a larger input; second call: a smaller one (the array keeps the first call's
    # contents, and the second must not depend on them)
    for i, (batch, seqlen, nheads, nseg) in enumerate(((2, 1024, 4, 8), (1, 256, 2, 4))):
        inp = synth.resume_inputs(synth.scan_inputs(cfg, seed=90 + 10 * cfg + i, batch=batch, seqlen=seqlen,
                                                    nheads=nheads), seed=91 + i)
        note(f"no-alloc segmented scan cfg{cfg} call {i}: batch {batch} x {seqlen}, {nheads} heads, {nseg} segments")
        (y0, h0), (y1, h1) = _both(inp, nseg, inp["meta"]["chunk"])
        assert np.array_equal(_bits(y0), _bits(y1))
        assert np.array_equal(_bits(h0), _bits(h1))


def test_noalloc_packed_matches_workspace_entry_twice():
    """Packed batches (segments of seg_tokens tokens, the segment table in the array too): two
    calls in a row, the second smaller, each bitwise equal to the workspace entry point's."""
    import torch
    for i, (cu, L) in enumerate((([0, 1, 1, 129, 130, 400, 700, 700], 100), ([0, 37, 37, 250], 64))):
        cu = np.array(cu, dtype=np.int32)
        inp = synth.scan_inputs(4, seed=95 + i, seqlen=int(cu[-1]), nheads=2, packed=False)
        inp["cu_seqlens"] = cu
        inp = synth.resume_inputs(inp, seed=96 + i)
        note(f"no-alloc packed segmented scan call {i}: {len(cu) - 1} sequences, {cu[-1]} tokens, segments of {L}")
        d = upload(inp, device())
        args = [d[k] for k in ("x", "dt", "lam", "theta", "B", "C", "A", "D")]
        kw = dict(seg_tokens=L, cu_seqlens=d["cu_seqlens"], chunk=inp["meta"]["chunk"], h_in=d["h_in"],
                  Bprev=d["Bprev"], xprev=d["xprev"])
        y0, h0 = m3.mamba3_scan_segmented(*args, **kw)
        y1, h1 = m3.mamba3_scan_segmented_noalloc(*args, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y0), _bits(y1))
        assert np.array_equal(_bits(h0), _bits(h1))
