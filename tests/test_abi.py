"""C ABI on the CPU: the library loads, exports every declared symbol, and its
pure host-side validation returns the documented status codes. No compute
call is made here (no GPU in this tier)."""
import ctypes
import os
import re

import pytest

import state_space_sequence_mamba3_amd as m3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m3.LIB_PATH):
        from state_space_sequence_mamba3_amd import build
        build.build()
    return m3.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mamba3.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba3_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m3.EXPORTS)


def test_binding_declares_every_signature(lib):
    # a pointer argument passed without a declared signature would be truncated to a C int
    l = m3.lib()
    for name in m3.EXPORTS:
        if name != "mamba3_version":
            assert getattr(l, name).argtypes is not None, name


def test_status_strings(lib):
    assert m3.status_string(m3.MAMBA3_OK) == "ok"
    for s in range(6):
        assert m3.status_string(s)
    assert lib.mamba3_version() == 10500


BASE = 0x7F0000000000


def fake(i):
    return BASE + i * 0x100000000


def good_scan(**over):
    a = m3.ScanArgs(batch=2, seqlen=100, nheads=4, headdim=16, dstate=16, rank=1, ngroups=4, chunk=64,
                    dtype=m3.MAMBA3_F32, cu_seqlens=None, nseq=0, x=fake(1), dt=fake(2), lam=fake(3),
                    theta=fake(4), B=fake(5), C=fake(6), A=fake(7), D=fake(8), h_in=None, Bprev=None,
                    xprev=None, y=fake(9), h_out=fake(10), workspace=None, workspace_bytes=0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_scan_validate_ok(lib):
    assert m3.mamba3_scan_validate(good_scan()) == m3.MAMBA3_OK
    assert m3.mamba3_scan_validate(good_scan(h_in=fake(11), Bprev=fake(12), xprev=fake(13))) == m3.MAMBA3_OK
    # h_out may alias h_in
    assert m3.mamba3_scan_validate(good_scan(h_in=fake(10))) == m3.MAMBA3_OK
    assert m3.mamba3_scan_workspace_size(good_scan()) == 0
    # empty inputs are valid
    assert m3.mamba3_scan_validate(good_scan(seqlen=0)) == m3.MAMBA3_OK
    assert m3.mamba3_scan_validate(good_scan(batch=0)) == m3.MAMBA3_OK


@pytest.mark.parametrize("field,value,status", [
    ("dstate", 15, m3.MAMBA3_EINVAL),
    ("dstate", 0, m3.MAMBA3_EINVAL),
    ("ngroups", 3, m3.MAMBA3_EINVAL),
    ("rank", 0, m3.MAMBA3_EINVAL),
    ("chunk", 0, m3.MAMBA3_EINVAL),
    ("headdim", 0, m3.MAMBA3_EINVAL),
    ("dtype", 7, m3.MAMBA3_EINVAL),
    ("x", None, m3.MAMBA3_EINVAL),
    ("A", None, m3.MAMBA3_EINVAL),
    ("y", None, m3.MAMBA3_EINVAL),
    ("Bprev", BASE + 0x5000000000, m3.MAMBA3_EINVAL),      # Bprev without xprev
    ("x", BASE + 0x100000008, m3.MAMBA3_EALIGN),
    ("theta", BASE + 0x400000004, m3.MAMBA3_EALIGN),
    ("dt", BASE + 0x200000002, m3.MAMBA3_EALIGN),           # fp32 needs 4-byte alignment
    ("h_out", BASE + 0xA00000004, m3.MAMBA3_EALIGN),
    ("y", BASE + 0x100000000, m3.MAMBA3_EINVAL),            # y aliases x
    ("h_out", BASE + 0x500000000, m3.MAMBA3_EINVAL),        # h_out overlaps B
    ("workspace_bytes", 64, m3.MAMBA3_EWORKSPACE),
    ("chunk", 100000, m3.MAMBA3_EUNSUPPORTED),              # fp32 tile does not fit LDS
])
def test_scan_validate_errors(lib, field, value, status):
    assert m3.mamba3_scan_validate(good_scan(**{field: value})) == status


@pytest.mark.parametrize("over,status", [
    (dict(bc_norm=1, bc_eps=1e-5), m3.MAMBA3_OK),
    (dict(bc_norm=1, bc_eps=0.0), m3.MAMBA3_OK),
    (dict(B_bias=fake(14), C_bias=fake(15), z=fake(16)), m3.MAMBA3_OK),
    (dict(bc_norm=2), m3.MAMBA3_EINVAL),
    (dict(bc_norm=-1), m3.MAMBA3_EINVAL),
    (dict(bc_norm=1, bc_eps=-1e-6), m3.MAMBA3_EINVAL),
    (dict(bc_norm=1, bc_eps=float("nan")), m3.MAMBA3_EINVAL),
    (dict(bc_norm=1, bc_eps=float("inf")), m3.MAMBA3_EINVAL),
    (dict(bc_norm=0, bc_eps=float("nan")), m3.MAMBA3_OK),       # eps unused without the norm
    (dict(z=fake(16) + 8), m3.MAMBA3_EALIGN),
    (dict(B_bias=fake(14) + 4), m3.MAMBA3_EALIGN),
    (dict(C_bias=fake(15) + 12), m3.MAMBA3_EALIGN),
    (dict(z=fake(9)), m3.MAMBA3_EINVAL),                        # y aliases z
    (dict(B_bias=fake(9) + 64), m3.MAMBA3_EINVAL),              # bias inside y
    (dict(C_bias=fake(10)), m3.MAMBA3_EINVAL),                  # h_out aliases a bias
])
def test_scan_validate_prologue(lib, over, status):
    assert m3.mamba3_scan_validate(good_scan(**over)) == status


def test_validate_variants(lib):
    # per-token decay rate: A may then be absent; fixed trapezoid weight: lam may be absent
    assert m3.mamba3_scan_validate(good_scan(A_tok=fake(17))) == m3.MAMBA3_OK
    assert m3.mamba3_scan_validate(good_scan(A_tok=fake(17), A=None)) == m3.MAMBA3_OK
    assert m3.mamba3_scan_validate(good_scan(A=None)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_scan_validate(good_scan(lam=None, lam_fixed=0.5)) == m3.MAMBA3_OK
    assert m3.mamba3_scan_validate(good_scan(lam=None, lam_fixed=float("nan"))) == m3.MAMBA3_EINVAL
    assert m3.mamba3_scan_validate(good_scan(A_tok=fake(17) + 2)) == m3.MAMBA3_EALIGN    # fp32 element alignment
    assert m3.mamba3_scan_validate(good_scan(A_tok=fake(9))) == m3.MAMBA3_EINVAL         # y aliases A_tok
    assert m3.mamba3_decode_validate(good_decode(A_tok=fake(17), A=None)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(A=None)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(lam=None, lam_fixed=1.0)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(lam=None, lam_fixed=float("inf"))) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(A_tok=fake(11))) == m3.MAMBA3_EINVAL     # h aliases A_tok
    # backward: dA_tok with a per-token A (and no dA), no dlam with a fixed weight
    b = good_bwd(dA=None, dA_tok=fake(39))
    b.fwd.A_tok = fake(17)
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_OK
    b.dA_tok = None
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_EINVAL
    assert m3.mamba3_scan_bwd_validate(good_bwd(dA_tok=fake(39))) == m3.MAMBA3_EINVAL     # no A_tok in the forward
    b = good_bwd(dlam=None)
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_EINVAL
    b.fwd.lam = None
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_OK


def test_validate_shared_angles_and_slots(lib):
    # angle rows shared by groups of heads: theta_groups divides nheads (0 = one row per head)
    for gth, st in ((0, m3.MAMBA3_OK), (1, m3.MAMBA3_OK), (2, m3.MAMBA3_OK), (3, m3.MAMBA3_EINVAL),
                    (-1, m3.MAMBA3_EINVAL)):
        assert m3.mamba3_scan_validate(good_scan(theta_groups=gth)) == st
        assert m3.mamba3_decode_validate(good_decode(theta_groups=gth if gth != 3 else 3)) == st
        b = good_bwd()
        b.fwd.theta_groups = gth
        assert m3.mamba3_scan_bwd_validate(b) == st
    # slot-indexed states: the pool holds nslots states; slots is a 4-byte aligned int32 array
    assert m3.mamba3_decode_validate(good_decode(slots=fake(13), nslots=16)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(slots=fake(13), nslots=0)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(slots=fake(13), nslots=-1)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(slots=fake(13) + 2, nslots=16)) == m3.MAMBA3_EALIGN
    assert m3.mamba3_decode_validate(good_decode(slots=fake(12), nslots=16)) == m3.MAMBA3_EINVAL   # y aliases slots
    assert m3.mamba3_decode_validate(good_decode(slots=fake(11) + 64, nslots=16)) == m3.MAMBA3_EINVAL  # slots in h
    # a pool of 10^6 states (8 heads of 64 x 64 fp32) reaches past y at the next fake address
    assert m3.mamba3_decode_validate(good_decode(slots=fake(13), nslots=1_000_000)) == m3.MAMBA3_EINVAL


def good_sp(**over):
    fwd = good_scan(y=None, h_out=None, h_in=fake(11), Bprev=fake(12), xprev=fake(13))
    a = m3.StatePassingArgs(fwd=fwd, nseg=4, U=fake(20), seg_h_in=fake(21), seg_Bprev=fake(22), seg_xprev=fake(23),
                            h_out=fake(24))
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_state_passing_validate(lib):
    assert m3.mamba3_state_passing_validate(good_sp()) == m3.MAMBA3_OK
    assert m3.mamba3_state_passing_validate(good_sp(h_out=None)) == m3.MAMBA3_OK
    assert m3.mamba3_state_passing_validate(good_sp(nseg=3)) == m3.MAMBA3_EINVAL      # 100 tokens, 3 segments
    assert m3.mamba3_state_passing_validate(good_sp(nseg=0)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_state_passing_validate(good_sp(U=None)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_state_passing_validate(good_sp(seg_xprev=None)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_state_passing_validate(good_sp(seg_h_in=fake(21) + 4)) == m3.MAMBA3_EALIGN
    assert m3.mamba3_state_passing_validate(good_sp(seg_h_in=fake(20))) == m3.MAMBA3_EINVAL   # aliases U
    assert m3.mamba3_state_passing_validate(good_sp(seg_Bprev=fake(5))) == m3.MAMBA3_EINVAL   # aliases B
    assert m3.mamba3_state_passing_validate(good_sp(h_out=fake(23))) == m3.MAMBA3_EINVAL      # aliases seg_xprev
    a = good_sp()
    a.fwd.y, a.fwd.z = fake(9), fake(10)                                                       # ignored: not read
    assert m3.mamba3_state_passing_validate(a) == m3.MAMBA3_OK
    a = good_sp()
    a.fwd.seqlen = 0
    assert m3.mamba3_state_passing_validate(a) == m3.MAMBA3_EINVAL
    assert m3.mamba3_state_passing_validate(good_sp(seg_tokens=32)) == m3.MAMBA3_EINVAL   # padded: nseg alone


def packed_sp(**over):
    """Packed batch of 3 sequences, 100 tokens, segments of 32 tokens: at most 3 + 4 = 7 rows."""
    a = good_sp(nseg=0, seg_tokens=32)
    a.fwd.cu_seqlens, a.fwd.batch, a.fwd.nseq = fake(30), 1, 3
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_state_passing_validate_packed(lib):
    a = packed_sp()
    assert lib.mamba3_segment_rows(ctypes.byref(a.fwd), 0, 32) == 7
    assert lib.mamba3_segment_rows(ctypes.byref(a.fwd), 0, 100) == 4
    assert lib.mamba3_segment_rows(ctypes.byref(a.fwd), 4, 32) == 0          # packed: nseg must be 0
    assert lib.mamba3_segment_rows(ctypes.byref(good_scan()), 4, 0) == 8     # padded: batch * nseg
    assert lib.mamba3_segment_rows(ctypes.byref(good_scan()), 4, 32) == 0
    assert m3.mamba3_state_passing_validate(a) == m3.MAMBA3_OK
    assert m3.mamba3_state_passing_validate(packed_sp(nseg=4)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_state_passing_validate(packed_sp(seg_tokens=0)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_state_passing_validate(packed_sp(seg_h_in=fake(30))) == m3.MAMBA3_EINVAL   # aliases cu_seqlens
    # h_in / h_out are per sequence (3 rows), the segment arrays per segment row (7)
    b = packed_sp()
    b.fwd.h_in = fake(31)
    assert m3.mamba3_state_passing_validate(b) == m3.MAMBA3_OK
    b.fwd.h_in = fake(24) - 3 * 4 * 16 * 16 * 4 + 256                       # its 3 rows reach into h_out
    assert m3.mamba3_state_passing_validate(b) == m3.MAMBA3_EINVAL


def test_segment_table_validate(lib):
    """The segment table's host checks (no launch: every case fails before one)."""
    t = lib.mamba3_segment_table
    assert t(None, 3, 100, 32, fake(2), None) == m3.MAMBA3_EINVAL
    assert t(fake(1), 3, 100, 32, None, None) == m3.MAMBA3_EINVAL
    assert t(fake(1), -1, 100, 32, fake(2), None) == m3.MAMBA3_EINVAL
    assert t(fake(1), 3, 100, 0, fake(2), None) == m3.MAMBA3_EINVAL
    assert t(fake(1) + 2, 3, 100, 32, fake(2), None) == m3.MAMBA3_EALIGN
    assert t(fake(1), 3, 100, 32, fake(1) + 8, None) == m3.MAMBA3_EINVAL   # overlaps cu_seqlens
    assert t(fake(1), 2 ** 31 - 2, 2 ** 31 - 1, 1, fake(2), None) == m3.MAMBA3_EINVAL   # rows + 1 > INT32_MAX


def good_seg(**over):
    fwd = good_scan(h_in=fake(11), Bprev=fake(12), xprev=fake(13))
    a = m3.ScanSegmentedArgs(fwd=fwd, nseg=4, workspace=fake(30), workspace_bytes=1 << 32)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_scan_segmented_validate(lib):
    need = m3.lib().mamba3_scan_segmented_workspace_size(ctypes.byref(good_seg()))
    # U and the entering states (2 x 8 rows x 4 heads x 16 x 16 fp32) and the previous tokens
    assert need == 2 * 8 * 4 * 16 * 16 * 4 + 8 * 4 * 16 * 4 + 8 * 4 * 16 * 4
    assert m3.mamba3_scan_segmented_validate(good_seg()) == m3.MAMBA3_OK
    assert m3.mamba3_scan_segmented_validate(good_seg(workspace_bytes=need)) == m3.MAMBA3_OK
    assert m3.mamba3_scan_segmented_validate(good_seg(workspace_bytes=need - 1)) == m3.MAMBA3_EWORKSPACE
    assert m3.mamba3_scan_segmented_validate(good_seg(workspace=None)) == m3.MAMBA3_EWORKSPACE
    assert m3.mamba3_scan_segmented_validate(good_seg(workspace=fake(30) + 128)) == m3.MAMBA3_EALIGN
    assert m3.mamba3_scan_segmented_validate(good_seg(workspace=fake(9) + 256)) == m3.MAMBA3_EINVAL   # inside y
    assert m3.mamba3_scan_segmented_validate(good_seg(nseg=3)) == m3.MAMBA3_EINVAL          # 100 tokens
    a = good_seg()
    a.fwd.workspace, a.fwd.workspace_bytes = fake(31), 256
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_EINVAL
    a = good_seg()
    a.fwd.cu_seqlens, a.fwd.batch, a.fwd.nseq = fake(32), 1, 2
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_EINVAL                # packed: nseg must be 0
    a.nseg, a.seg_tokens = 0, 32
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_OK
    # packed: 2 + ceil(100 / 32) = 6 rows, and the segment table (7 int32) in its own region
    need = m3.lib().mamba3_scan_segmented_workspace_size(ctypes.byref(a))
    assert need == 2 * 6 * 4 * 16 * 16 * 4 + 6 * 4 * 16 * 4 + 6 * 4 * 16 * 4 + 256
    a.workspace_bytes = need - 1
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_EWORKSPACE
    a.workspace, a.workspace_bytes = fake(32) - 256, need                          # overlaps cu_seqlens
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_EINVAL
    assert m3.mamba3_scan_segmented_validate(good_seg(seg_tokens=32)) == m3.MAMBA3_EINVAL   # padded: nseg alone
    a = good_seg()
    a.fwd.h_out = fake(11)                                                          # h_out may be h_in
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_OK
    a = good_seg(nseg=2)
    a.fwd.dtype, a.fwd.dstate, a.fwd.headdim, a.fwd.chunk = m3.MAMBA3_BF16, 48, 48, 64   # no bf16 kernel
    assert m3.mamba3_scan_segmented_validate(a) == m3.MAMBA3_EUNSUPPORTED


def test_decode_validate_prologue(lib):
    ok = dict(B_bias=fake(14), C_bias=fake(15), z=fake(16), bc_norm=1, bc_eps=1e-6)
    assert m3.mamba3_decode_validate(good_decode(**ok)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(bc_norm=3)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(bc_norm=1, bc_eps=-0.5)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(z=fake(16) + 2)) == m3.MAMBA3_EALIGN
    assert m3.mamba3_decode_validate(good_decode(z=fake(12))) == m3.MAMBA3_EINVAL       # y aliases z
    assert m3.mamba3_decode_validate(good_decode(B_bias=fake(11))) == m3.MAMBA3_EINVAL  # h aliases a bias


def good_bwd(**over):
    fwd = good_scan(y=None, h_out=None, h_in=fake(11), Bprev=fake(12), xprev=fake(13))
    b = m3.ScanBwdArgs(fwd=fwd, dy=fake(20), dh_out=fake(21), dx=fake(22), ddt=fake(23), dlam=fake(24),
                       dtheta=fake(25), dB=fake(26), dC=fake(27), dA=fake(28), dD=fake(29), dh_in=fake(30),
                       dBprev=fake(31), dxprev=fake(32), dB_bias=None, dC_bias=None, dz=None,
                       workspace=fake(40), workspace_bytes=1 << 40)
    for k, v in over.items():
        setattr(b, k, v)
    return b


def test_scan_bwd_validate(lib):
    b = good_bwd()
    need = m3.mamba3_scan_bwd_workspace_size(b)
    assert 0 < need < 1 << 40
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_OK
    b.workspace_bytes = need
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_OK
    b.workspace_bytes = need - 1
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_EWORKSPACE
    assert m3.mamba3_scan_bwd_validate(good_bwd(workspace=None)) == m3.MAMBA3_EWORKSPACE
    assert m3.mamba3_scan_bwd_validate(good_bwd(workspace=fake(40) + 128)) == m3.MAMBA3_EALIGN
    # optional outputs may be left out
    assert m3.mamba3_scan_bwd_validate(good_bwd(dD=None, dh_in=None, dh_out=None, dBprev=None, dxprev=None)) == m3.MAMBA3_OK


@pytest.mark.parametrize("field,value,status", [
    ("dy", None, m3.MAMBA3_EINVAL),
    ("dA", None, m3.MAMBA3_EINVAL),
    ("dx", None, m3.MAMBA3_EINVAL),
    ("dBprev", None, m3.MAMBA3_EINVAL),                     # dxprev without dBprev
    ("dz", BASE + 0x3300000000, m3.MAMBA3_EINVAL),          # no gate in the forward
    ("dB_bias", BASE + 0x3400000000, m3.MAMBA3_EINVAL),     # no bias in the forward
    ("dx", BASE + 0x100000000, m3.MAMBA3_EINVAL),           # dx aliases x
    ("dB", BASE + 0x1900000000, m3.MAMBA3_EINVAL),          # dB aliases dtheta
    ("dA", BASE + 0x1500000000, m3.MAMBA3_EINVAL),          # dA aliases dh_out
    ("dx", BASE + 0x1600000008, m3.MAMBA3_EALIGN),
    ("dA", BASE + 0x1C00000002, m3.MAMBA3_EALIGN),
    ("workspace", BASE + 0x700000000, m3.MAMBA3_EINVAL),    # workspace overlaps A
])
def test_scan_bwd_validate_errors(lib, field, value, status):
    assert m3.mamba3_scan_bwd_validate(good_bwd(**{field: value})) == status


def test_scan_bwd_validate_shapes(lib):
    b = good_bwd()
    b.fwd.dstate, b.fwd.headdim = 1024, 512       # the state and its gradient do not fit in LDS
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_EUNSUPPORTED
    assert m3.mamba3_scan_bwd_workspace_size(b) == 0
    b = good_bwd()
    b.fwd.dtype = m3.MAMBA3_BF16                  # bf16 shapes without a forward kernel are fine here
    b.fwd.dstate, b.fwd.headdim = 24, 40
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_OK
    b.fwd.dstate = 23
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_EINVAL
    assert lib.mamba3_scan_bwd_validate(None) == m3.MAMBA3_EINVAL


def test_scan_validate_packed(lib):
    a = good_scan(batch=1, seqlen=500, nseq=3)
    a.cu_seqlens = fake(20)
    assert m3.mamba3_scan_validate(a) == m3.MAMBA3_OK
    a.batch = 2
    assert m3.mamba3_scan_validate(a) == m3.MAMBA3_EINVAL
    a.batch, a.nseq = 1, 0
    assert m3.mamba3_scan_validate(a) == m3.MAMBA3_EINVAL


def test_scan_validate_null_args(lib):
    assert lib.mamba3_scan_validate(None) == m3.MAMBA3_EINVAL
    assert lib.mamba3_decode_validate(None) == m3.MAMBA3_EINVAL


def good_decode(**over):
    a = m3.DecodeArgs(batch=4, nheads=8, headdim=64, dstate=64, rank=4, ngroups=8, dtype=m3.MAMBA3_BF16,
                      x=fake(1), dt=fake(2), lam=fake(3), theta=fake(4), B=fake(5), C=fake(6), Bprev=fake(7),
                      xprev=fake(8), A=fake(9), D=fake(10), h=fake(11), y=fake(12))
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_decode_validate(lib):
    assert m3.mamba3_decode_validate(good_decode()) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(Bprev=None, xprev=None)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(Bprev=None)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(dstate=63)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(h=None)) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(y=fake(11))) == m3.MAMBA3_EINVAL
    assert m3.mamba3_decode_validate(good_decode(h=BASE + 0xB00000002)) == m3.MAMBA3_EALIGN
    assert m3.mamba3_decode_validate(good_decode(dstate=40)) == m3.MAMBA3_EUNSUPPORTED
    # dt / lam need only element alignment
    assert m3.mamba3_decode_validate(good_decode(dt=BASE + 0x200000002)) == m3.MAMBA3_OK
    assert m3.mamba3_decode_validate(good_decode(dt=BASE + 0x200000001)) == m3.MAMBA3_EALIGN
    assert m3.mamba3_decode_validate(good_decode(batch=0)) == m3.MAMBA3_OK


def test_binding_refuses_host_and_strided_tensors():
    # every ABI pointer is a dense device array: a host tensor or a strided view never reaches the library
    import torch
    x = torch.zeros((2, 8, 4, 1, 16))
    with pytest.raises(ValueError, match="device memory"):
        m3._ptr(x)
    with pytest.raises(ValueError, match="device memory"):
        m3.mamba3_scan_fwd(x, x[..., 0, 0], x[..., 0, 0], x[..., 0, :8], x, x, torch.zeros(4))
    assert m3._ptr(None) is None and m3._ptr(fake(3)) == fake(3)


def _device_count():
    import torch
    return torch.cuda.device_count()   # counts devices without initialising one


def test_no_device_returns_ehip(lib):
    """With no GPU visible, every entry point that would enqueue work returns MAMBA3_EHIP after
    its validation passes, instead of crashing. The pointers are fake device addresses, so this
    runs only where no device exists (on a GPU machine a launch would read them)."""
    if _device_count() > 0:
        pytest.skip("a device is visible: the fake pointers would be dereferenced by a real launch")
    st = lib.mamba3_scan_fwd(ctypes.byref(good_scan()), None)
    assert st == m3.MAMBA3_EHIP
    bf = good_scan(dtype=m3.MAMBA3_BF16, dstate=128, headdim=64)
    assert m3.mamba3_scan_validate(bf) == m3.MAMBA3_OK
    assert lib.mamba3_scan_fwd(ctypes.byref(bf), None) == m3.MAMBA3_EHIP
    d = good_decode()
    assert m3.mamba3_decode_validate(d) == m3.MAMBA3_OK
    assert lib.mamba3_decode_step(ctypes.byref(d), None) == m3.MAMBA3_EHIP
    b = good_bwd()
    assert m3.mamba3_scan_bwd_validate(b) == m3.MAMBA3_OK
    assert lib.mamba3_scan_bwd(ctypes.byref(b), None) == m3.MAMBA3_EHIP
    sp = good_sp()
    assert m3.mamba3_state_passing_validate(sp) == m3.MAMBA3_OK
    assert lib.mamba3_state_passing(ctypes.byref(sp), None) == m3.MAMBA3_EHIP
    sg = good_seg()
    assert m3.mamba3_scan_segmented_validate(sg) == m3.MAMBA3_OK
    assert lib.mamba3_scan_segmented(ctypes.byref(sg), None) == m3.MAMBA3_EHIP
    sg.workspace, sg.workspace_bytes = None, 0
    assert lib.mamba3_scan_segmented_noalloc(ctypes.byref(sg), None) == m3.MAMBA3_EHIP


def test_scan_segmented_noalloc_limits(lib):
    """The allocation-free segmented scan refuses a caller workspace and a problem whose
    workspace exceeds its array; both before any HIP call (so this runs without a device)."""
    a = good_seg()
    assert lib.mamba3_scan_segmented_noalloc(ctypes.byref(a), None) == m3.MAMBA3_EINVAL   # caller workspace
    big = good_seg(workspace=None, workspace_bytes=0, nseg=64)
    big.fwd.seqlen, big.fwd.nheads, big.fwd.ngroups, big.fwd.dstate, big.fwd.headdim = 64 * 16, 64, 64, 128, 64
    need = lib.mamba3_scan_segmented_workspace_size(ctypes.byref(big))
    assert need > m3.MAMBA3_NOALLOC_SCRATCH_BYTES
    assert lib.mamba3_scan_segmented_noalloc(ctypes.byref(big), None) == m3.MAMBA3_EWORKSPACE
    assert lib.mamba3_scan_segmented_noalloc(None, None) == m3.MAMBA3_EINVAL
