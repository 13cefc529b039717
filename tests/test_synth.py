"""Seeded input generator: determinism, bf16 rounding, packed lengths, shapes."""
import numpy as np

from state_space_sequence_mamba3_amd import synth


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = synth.bf16_bits(vals)
    back = synth.bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert back[1] == 1.0
    # 1 + 1.5*2^-8 rounds up to 1 + 2^-7
    assert back[2] == np.float32(1.0078125)
    assert back[3] == np.float32(1.0078125)
    assert back[4] == -2.5
    # round trip of representable values is exact
    assert np.array_equal(synth.bits_to_f32(synth.bf16_bits(back)), back)


def test_determinism_and_shapes():
    a = synth.scan_inputs(2, batch=1, seqlen=16, nheads=2)
    b = synth.scan_inputs(2, batch=1, seqlen=16, nheads=2)
    for k in ("x", "dt", "lam", "theta", "B", "C", "A", "D"):
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (1, 16, 2, 4, 64) and a["x"].dtype == np.uint16
    assert a["B"].shape == (1, 16, 2, 4, 64)
    assert a["theta"].shape == (1, 16, 2, 32)
    c = synth.scan_inputs(2, seed=7, batch=1, seqlen=16, nheads=2)
    assert not np.array_equal(a["x"], c["x"])


def test_distributions():
    inp = synth.scan_inputs(0, batch=4, seqlen=4096)
    dt = inp["dt"]
    assert 0.10 < np.median(dt) < 0.16 and dt.min() > 0
    assert 0 < inp["lam"].min() and inp["lam"].max() < 1
    assert np.all(np.abs(inp["theta"]) <= np.pi + 1e-6)
    assert abs(inp["B"].std() * np.sqrt(16) - 1) < 0.02
    assert np.all(inp["A"] < 0)


def test_packed_lengths():
    inp = synth.scan_inputs(4, seqlen=65536, nheads=1, headdim=4, dstate=4, rank=1)
    cu = inp["cu_seqlens"]
    ln = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == 65536 and len(ln) == 8
    assert ln.min() >= 65536 * 1024 // (8 * 16384) and ln.max() <= 16384 * 65536 // (8 * 1024)
