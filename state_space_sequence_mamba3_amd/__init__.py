"""Mamba-3 SSM layer recurrence on AMD MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libmamba3.so`` (declared in
``include/mamba3.h``). It only marshals arguments: torch tensors provide the
device memory and the current HIP stream; every step of the computation runs
in the library's HIP kernels. If the library is missing the binding raises;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmamba3.so")

MAMBA3_OK, MAMBA3_EINVAL, MAMBA3_EUNSUPPORTED, MAMBA3_EALIGN, MAMBA3_EHIP, MAMBA3_EWORKSPACE = range(6)
MAMBA3_F32, MAMBA3_BF16 = 0, 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class ScanArgs(ctypes.Structure):
    """Mirror of ``mamba3_scan_args``."""
    _fields_ = [
        ("batch", _i32), ("seqlen", _i32), ("nheads", _i32), ("headdim", _i32), ("dstate", _i32),
        ("rank", _i32), ("ngroups", _i32), ("chunk", _i32), ("dtype", _i32),
        ("cu_seqlens", _vp), ("nseq", _i32),
        ("x", _vp), ("dt", _vp), ("lam", _vp), ("theta", _vp), ("B", _vp), ("C", _vp),
        ("A", _vp), ("D", _vp), ("h_in", _vp), ("Bprev", _vp), ("xprev", _vp),
        ("y", _vp), ("h_out", _vp), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("B_bias", _vp), ("C_bias", _vp), ("z", _vp), ("bc_norm", _i32), ("bc_eps", ctypes.c_float),
        ("A_tok", _vp), ("lam_fixed", ctypes.c_float), ("theta_groups", _i32),
    ]


class DecodeArgs(ctypes.Structure):
    """Mirror of ``mamba3_decode_args``."""
    _fields_ = [
        ("batch", _i32), ("nheads", _i32), ("headdim", _i32), ("dstate", _i32), ("rank", _i32),
        ("ngroups", _i32), ("dtype", _i32),
        ("x", _vp), ("dt", _vp), ("lam", _vp), ("theta", _vp), ("B", _vp), ("C", _vp),
        ("Bprev", _vp), ("xprev", _vp), ("A", _vp), ("D", _vp), ("h", _vp), ("y", _vp),
        ("B_bias", _vp), ("C_bias", _vp), ("z", _vp), ("bc_norm", _i32), ("bc_eps", ctypes.c_float),
        ("A_tok", _vp), ("lam_fixed", ctypes.c_float), ("theta_groups", _i32), ("slots", _vp), ("nslots", _i32),
    ]


class ScanBwdArgs(ctypes.Structure):
    """Mirror of ``mamba3_scan_bwd_args``."""
    _fields_ = [
        ("fwd", ScanArgs), ("dy", _vp), ("dh_out", _vp),
        ("dx", _vp), ("ddt", _vp), ("dlam", _vp), ("dtheta", _vp), ("dB", _vp), ("dC", _vp),
        ("dA", _vp), ("dD", _vp), ("dh_in", _vp), ("dBprev", _vp), ("dxprev", _vp),
        ("dB_bias", _vp), ("dC_bias", _vp), ("dz", _vp), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("dA_tok", _vp),
    ]


class StatePassingArgs(ctypes.Structure):
    """Mirror of ``mamba3_state_passing_args``."""
    _fields_ = [
        ("fwd", ScanArgs), ("nseg", _i32), ("U", _vp), ("seg_h_in", _vp), ("seg_Bprev", _vp), ("seg_xprev", _vp),
        ("h_out", _vp), ("seg_tokens", _i32),
    ]


class ScanSegmentedArgs(ctypes.Structure):
    """Mirror of ``mamba3_scan_segmented_args``."""
    _fields_ = [("fwd", ScanArgs), ("nseg", _i32), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("seg_tokens", _i32)]


EXPORTS = ("mamba3_scan_validate", "mamba3_scan_workspace_size", "mamba3_scan_fwd", "mamba3_scan_bwd_validate",
           "mamba3_scan_bwd_workspace_size", "mamba3_scan_bwd", "mamba3_state_passing_validate",
           "mamba3_state_passing", "mamba3_segment_rows", "mamba3_segment_table",
           "mamba3_scan_segmented_workspace_size", "mamba3_scan_segmented_validate",
           "mamba3_scan_segmented", "mamba3_scan_segmented_noalloc", "mamba3_decode_validate", "mamba3_decode_step",
           "mamba3_status_string", "mamba3_version")

# Size of the library-owned workspace of mamba3_scan_segmented_noalloc (bytes, per GPU).
MAMBA3_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class Mamba3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib():
    """Loads libmamba3.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m state_space_sequence_mamba3_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        l.mamba3_scan_validate.argtypes = [ctypes.POINTER(ScanArgs)]
        l.mamba3_scan_validate.restype = ctypes.c_int
        l.mamba3_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs)]
        l.mamba3_scan_workspace_size.restype = ctypes.c_size_t
        l.mamba3_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        l.mamba3_scan_fwd.restype = ctypes.c_int
        l.mamba3_scan_bwd_validate.argtypes = [ctypes.POINTER(ScanBwdArgs)]
        l.mamba3_scan_bwd_validate.restype = ctypes.c_int
        l.mamba3_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ScanBwdArgs)]
        l.mamba3_scan_bwd_workspace_size.restype = ctypes.c_size_t
        l.mamba3_scan_bwd.argtypes = [ctypes.POINTER(ScanBwdArgs), _vp]
        l.mamba3_scan_bwd.restype = ctypes.c_int
        l.mamba3_state_passing_validate.argtypes = [ctypes.POINTER(StatePassingArgs)]
        l.mamba3_state_passing_validate.restype = ctypes.c_int
        l.mamba3_state_passing.argtypes = [ctypes.POINTER(StatePassingArgs), _vp]
        l.mamba3_state_passing.restype = ctypes.c_int
        l.mamba3_segment_rows.argtypes = [ctypes.POINTER(ScanArgs), _i32, _i32]
        l.mamba3_segment_rows.restype = ctypes.c_int64
        l.mamba3_segment_table.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp]
        l.mamba3_segment_table.restype = ctypes.c_int
        l.mamba3_scan_segmented_workspace_size.argtypes = [ctypes.POINTER(ScanSegmentedArgs)]
        l.mamba3_scan_segmented_workspace_size.restype = ctypes.c_size_t
        l.mamba3_scan_segmented_validate.argtypes = [ctypes.POINTER(ScanSegmentedArgs)]
        l.mamba3_scan_segmented_validate.restype = ctypes.c_int
        l.mamba3_scan_segmented.argtypes = [ctypes.POINTER(ScanSegmentedArgs), _vp]
        l.mamba3_scan_segmented.restype = ctypes.c_int
        l.mamba3_scan_segmented_noalloc.argtypes = [ctypes.POINTER(ScanSegmentedArgs), _vp]
        l.mamba3_scan_segmented_noalloc.restype = ctypes.c_int
        l.mamba3_decode_validate.argtypes = [ctypes.POINTER(DecodeArgs)]
        l.mamba3_decode_validate.restype = ctypes.c_int
        l.mamba3_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        l.mamba3_decode_step.restype = ctypes.c_int
        l.mamba3_status_string.argtypes = [ctypes.c_int]
        l.mamba3_status_string.restype = ctypes.c_char_p
        l.mamba3_version.restype = ctypes.c_int32
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().mamba3_status_string(status).decode()


def _ptr(t):
    """Device address of a tensor (or an int address as is). Every pointer of the ABI is a device
    pointer into a dense row-major array, so a host tensor or a strided view is refused here
    rather than read as if it were dense device memory."""
    if t is None:
        return None
    if not hasattr(t, "data_ptr"):
        return int(t)
    if not t.is_cuda:
        raise ValueError("mamba3: tensors must be in device memory")
    if not t.is_contiguous():
        raise ValueError("mamba3: tensors must be contiguous (dense row-major); call .contiguous()")
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MAMBA3_BF16
    if t.dtype == torch.float32:
        return MAMBA3_F32
    raise TypeError(f"token inputs must be float32 or bfloat16, got {t.dtype}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def scan_args(x, dt, lam, theta, B, C, A, D=None, *, y, h_in=None, h_out=None, Bprev=None, xprev=None,
              cu_seqlens=None, chunk=64, B_bias=None, C_bias=None, z=None, bc_norm=False,
              bc_eps=1e-5, A_tok=None, lam_fixed=0.5) -> ScanArgs:
    """Builds a ScanArgs from tensors in the library's layouts (see mamba3.h)."""
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    nseq = int(cu_seqlens.numel()) - 1 if cu_seqlens is not None else 0
    return ScanArgs(b, L, H, P, N, R, G, chunk, _dtype_code(x), _ptr(cu_seqlens), nseq,
                    _ptr(x), _ptr(dt), _ptr(lam), _ptr(theta), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
                    _ptr(h_in), _ptr(Bprev), _ptr(xprev), _ptr(y), _ptr(h_out), None, 0,
                    _ptr(B_bias), _ptr(C_bias), _ptr(z), int(bool(bc_norm)), float(bc_eps), _ptr(A_tok),
                    float(lam_fixed), int(theta.shape[2]) if theta is not None else 0)


def mamba3_scan_validate(args: ScanArgs) -> int:
    return lib().mamba3_scan_validate(ctypes.byref(args))


def mamba3_scan_workspace_size(args: ScanArgs) -> int:
    return lib().mamba3_scan_workspace_size(ctypes.byref(args))


def mamba3_scan_fwd(x, dt, lam, theta, B, C, A, D=None, *, y=None, h_in=None, h_out=None, Bprev=None,
                    xprev=None, cu_seqlens=None, chunk=64, want_state=True, stream=None, B_bias=None,
                    C_bias=None, z=None, bc_norm=False, bc_eps=1e-5, A_tok=None, lam_fixed=0.5):
    """Chunked scan over whole sequences. Tensors are device tensors in the
    layouts of mamba3.h; y and h_out are allocated when not given. Returns
    (y, h_out). B_bias, C_bias ([H, N] fp32), z (layout of x) and bc_norm /
    bc_eps switch on the fused B/C normalisation, B/C biases and output gate;
    A_tok (layout of dt) replaces A with a per-token decay rate, lam=None
    uses lam_fixed for every token, and a theta of shape [b,L,Gth,N/2] with
    Gth < H shares each angle row among H/Gth consecutive heads."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    if h_out is None and want_state:
        S = int(cu_seqlens.numel()) - 1 if cu_seqlens is not None else x.shape[0]
        h_out = torch.empty((S, x.shape[2], B.shape[4], x.shape[4]), dtype=torch.float32, device=x.device)
    a = scan_args(x, dt, lam, theta, B, C, A, D, y=y, h_in=h_in, h_out=h_out, Bprev=Bprev, xprev=xprev,
                  cu_seqlens=cu_seqlens, chunk=chunk, B_bias=B_bias, C_bias=C_bias, z=z, bc_norm=bc_norm,
                  bc_eps=bc_eps, A_tok=A_tok, lam_fixed=lam_fixed)
    st = lib().mamba3_scan_fwd(ctypes.byref(a), _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_scan_fwd")
    return y, h_out


def mamba3_scan_bwd_validate(args: ScanBwdArgs) -> int:
    return lib().mamba3_scan_bwd_validate(ctypes.byref(args))


def mamba3_scan_bwd_workspace_size(args: ScanBwdArgs) -> int:
    return lib().mamba3_scan_bwd_workspace_size(ctypes.byref(args))


def mamba3_scan_bwd(x, dt, lam, theta, B, C, A, D=None, *, dy, dh_out=None, h_in=None, Bprev=None, xprev=None,
                    cu_seqlens=None, chunk=64, B_bias=None, C_bias=None, z=None, bc_norm=False, bc_eps=1e-5,
                    A_tok=None, lam_fixed=0.5, want_dD=True, want_dh_in=True, workspace=None, stream=None):
    """Gradients of the scan. Takes the forward's inputs plus dy (layout of
    x) and dh_out ([S,H,N,P] fp32 or None); returns a dict of gradients shaped
    like the inputs (dx, ddt, dlam, dtheta, dB, dC; dA, dD fp32 [H]; dh_in;
    dBprev, dxprev, dB_bias, dC_bias, dz where the input exists). The
    workspace is allocated unless given (a uint8 device tensor)."""
    import torch
    fwd = scan_args(x, dt, lam, theta, B, C, A, D, y=None, h_in=h_in, h_out=None, Bprev=Bprev, xprev=xprev,
                    cu_seqlens=cu_seqlens, chunk=chunk, B_bias=B_bias, C_bias=C_bias, z=z, bc_norm=bc_norm,
                    bc_eps=bc_eps, A_tok=A_tok, lam_fixed=lam_fixed)
    S = int(cu_seqlens.numel()) - 1 if cu_seqlens is not None else x.shape[0]
    H, N, P = x.shape[2], B.shape[4], x.shape[4]
    f32 = dict(dtype=torch.float32, device=x.device)
    g = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dtheta=torch.empty_like(theta),
             dB=torch.empty_like(B), dC=torch.empty_like(C))
    if lam is not None:
        g["dlam"] = torch.empty_like(lam)
    if A_tok is not None:
        g["dA_tok"] = torch.empty_like(A_tok)
    else:
        g["dA"] = torch.empty((H,), **f32)
    if want_dD:
        g["dD"] = torch.empty((H,), **f32)
    if want_dh_in:
        g["dh_in"] = torch.empty((S, H, N, P), **f32)
    if Bprev is not None:
        g["dBprev"], g["dxprev"] = torch.empty_like(Bprev), torch.empty_like(xprev)
    if B_bias is not None:
        g["dB_bias"] = torch.empty_like(B_bias)
    if C_bias is not None:
        g["dC_bias"] = torch.empty_like(C_bias)
    if z is not None:
        g["dz"] = torch.empty_like(z)
    a = ScanBwdArgs(fwd, _ptr(dy), _ptr(dh_out), *[_ptr(g.get(k)) for k in (
        "dx", "ddt", "dlam", "dtheta", "dB", "dC", "dA", "dD", "dh_in", "dBprev", "dxprev", "dB_bias", "dC_bias",
        "dz")], None, 0, _ptr(g.get("dA_tok")))
    need = lib().mamba3_scan_bwd_workspace_size(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    st = lib().mamba3_scan_bwd(ctypes.byref(a), _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_scan_bwd")
    return g


def mamba3_state_passing_validate(args: StatePassingArgs) -> int:
    return lib().mamba3_state_passing_validate(ctypes.byref(args))


def mamba3_segment_rows(args: ScanArgs, nseg: int = 0, seg_tokens: int = 0) -> int:
    return lib().mamba3_segment_rows(ctypes.byref(args), int(nseg), int(seg_tokens))


def mamba3_segment_table(cu_seqlens, seqlen: int, seg_tokens: int, stream=None):
    """The segment table of a packed batch (int32 device tensor of rows + 1
    entries, rows = nseq + ceil(seqlen / seg_tokens)): segment row r holds
    tokens [t[r], t[r+1])."""
    import torch
    nseq = int(cu_seqlens.numel()) - 1
    rows = nseq + (int(seqlen) + int(seg_tokens) - 1) // int(seg_tokens) if seg_tokens >= 1 else 0
    seg_cu = torch.empty((max(rows, 0) + 1,), dtype=torch.int32, device=cu_seqlens.device)
    st = lib().mamba3_segment_table(_ptr(cu_seqlens), nseq, int(seqlen), int(seg_tokens), _ptr(seg_cu),
                                    _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_segment_table")
    return seg_cu


def mamba3_state_passing(x, dt, lam, theta, B, C, A, *, nseg=0, U, h_in=None, Bprev=None, xprev=None, B_bias=None,
                         C_bias=None, bc_norm=False, bc_eps=1e-5, A_tok=None, lam_fixed=0.5, want_state=True,
                         cu_seqlens=None, seg_tokens=0, stream=None):
    """The state entering each segment row, from U ([rows,H,N,P], the
    segments scanned from a zero state with no previous token). Padded
    batches: nseg segments per sequence, rows = batch*nseg. Packed batches
    (cu_seqlens): segments of seg_tokens tokens, rows as mamba3_segment_rows.
    Returns (seg_h_in [rows,H,N,P] fp32, seg_Bprev, seg_xprev (token before
    each segment), h_out [S,H,N,P] or None)."""
    import torch
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    fwd = scan_args(x, dt, lam, theta, B, C, A, None, y=None, h_in=h_in, h_out=None, Bprev=Bprev, xprev=xprev,
                    cu_seqlens=cu_seqlens, B_bias=B_bias, C_bias=C_bias, bc_norm=bc_norm, bc_eps=bc_eps,
                    A_tok=A_tok, lam_fixed=lam_fixed)
    SR = mamba3_segment_rows(fwd, nseg, seg_tokens)
    S = int(cu_seqlens.numel()) - 1 if cu_seqlens is not None else b
    seg_h = torch.empty((SR, H, N, P), dtype=torch.float32, device=x.device)
    seg_B = torch.empty((SR, G, R, N), dtype=x.dtype, device=x.device)
    seg_x = torch.empty((SR, H, R, P), dtype=x.dtype, device=x.device)
    h_out = torch.empty((S, H, N, P), dtype=torch.float32, device=x.device) if want_state else None
    a = StatePassingArgs(fwd, int(nseg), _ptr(U), _ptr(seg_h), _ptr(seg_B), _ptr(seg_x), _ptr(h_out),
                         int(seg_tokens))
    st = lib().mamba3_state_passing(ctypes.byref(a), _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_state_passing")
    return seg_h, seg_B, seg_x, h_out


def mamba3_scan_segmented_validate(args: ScanSegmentedArgs) -> int:
    return lib().mamba3_scan_segmented_validate(ctypes.byref(args))


def mamba3_scan_segmented(x, dt, lam, theta, B, C, A, D=None, *, nseg=0, y=None, h_in=None, h_out=None, Bprev=None,
                          xprev=None, chunk=64, want_state=True, workspace=None, stream=None, B_bias=None,
                          C_bias=None, z=None, bc_norm=False, bc_eps=1e-5, A_tok=None, lam_fixed=0.5,
                          cu_seqlens=None, seg_tokens=0):
    """mamba3_scan_segmented: the whole-sequence scan run as independent
    segments (scan, state passing, scan, all in the library): nseg segments
    per sequence of a padded batch, or segments of seg_tokens tokens of a
    packed batch (cu_seqlens). Same results as mamba3_scan_fwd up to rounding.
    The workspace is allocated when not given. Returns (y, h_out)."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    if h_out is None and want_state:
        S = int(cu_seqlens.numel()) - 1 if cu_seqlens is not None else x.shape[0]
        h_out = torch.empty((S, x.shape[2], B.shape[4], x.shape[4]), dtype=torch.float32, device=x.device)
    fwd = scan_args(x, dt, lam, theta, B, C, A, D, y=y, h_in=h_in, h_out=h_out, Bprev=Bprev, xprev=xprev,
                    cu_seqlens=cu_seqlens, chunk=chunk, B_bias=B_bias, C_bias=C_bias, z=z, bc_norm=bc_norm,
                    bc_eps=bc_eps, A_tok=A_tok, lam_fixed=lam_fixed)
    a = ScanSegmentedArgs(fwd, int(nseg), None, 0, int(seg_tokens))
    need = lib().mamba3_scan_segmented_workspace_size(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    st = lib().mamba3_scan_segmented(ctypes.byref(a), _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_scan_segmented")
    return y, h_out


def mamba3_scan_segmented_noalloc(x, dt, lam, theta, B, C, A, D=None, *, nseg=0, y=None, h_in=None, h_out=None,
                                  Bprev=None, xprev=None, chunk=64, want_state=True, stream=None, B_bias=None,
                                  C_bias=None, z=None, bc_norm=False, bc_eps=1e-5, A_tok=None, lam_fixed=0.5,
                                  cu_seqlens=None, seg_tokens=0):
    """mamba3_scan_segmented_noalloc: the segmented scan with the library's own workspace (the
    library allocates nothing; y and h_out are allocated here by torch when not given, as by the
    other entry points). Returns (y, h_out)."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    if h_out is None and want_state:
        S = int(cu_seqlens.numel()) - 1 if cu_seqlens is not None else x.shape[0]
        h_out = torch.empty((S, x.shape[2], B.shape[4], x.shape[4]), dtype=torch.float32, device=x.device)
    fwd = scan_args(x, dt, lam, theta, B, C, A, D, y=y, h_in=h_in, h_out=h_out, Bprev=Bprev, xprev=xprev,
                    cu_seqlens=cu_seqlens, chunk=chunk, B_bias=B_bias, C_bias=C_bias, z=z, bc_norm=bc_norm,
                    bc_eps=bc_eps, A_tok=A_tok, lam_fixed=lam_fixed)
    a = ScanSegmentedArgs(fwd, int(nseg), None, 0, int(seg_tokens))
    st = lib().mamba3_scan_segmented_noalloc(ctypes.byref(a), _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_scan_segmented_noalloc")
    return y, h_out


def decode_args(x, dt, lam, theta, B, C, A, D=None, *, h, y, Bprev=None, xprev=None, B_bias=None, C_bias=None,
                z=None, bc_norm=False, bc_eps=1e-5, A_tok=None, lam_fixed=0.5, slots=None) -> DecodeArgs:
    b, H, R, P = x.shape
    G, N = B.shape[1], B.shape[3]
    return DecodeArgs(b, H, P, N, R, G, _dtype_code(x), _ptr(x), _ptr(dt), _ptr(lam), _ptr(theta), _ptr(B),
                      _ptr(C), _ptr(Bprev), _ptr(xprev), _ptr(A), _ptr(D), _ptr(h), _ptr(y),
                      _ptr(B_bias), _ptr(C_bias), _ptr(z), int(bool(bc_norm)), float(bc_eps), _ptr(A_tok),
                      float(lam_fixed), int(theta.shape[1]) if theta is not None else 0, _ptr(slots),
                      int(h.shape[0]) if slots is not None else 0)


def mamba3_decode_validate(args: DecodeArgs) -> int:
    return lib().mamba3_decode_validate(ctypes.byref(args))


def mamba3_decode_step(x, dt, lam, theta, B, C, A, D=None, *, h, y=None, Bprev=None, xprev=None, stream=None,
                       B_bias=None, C_bias=None, z=None, bc_norm=False, bc_eps=1e-5, A_tok=None, lam_fixed=0.5,
                       slots=None):
    """One decode step; h (fp32 [batch,H,N,P]) is updated in place. Returns y.
    The prologue / epilogue keywords are those of mamba3_scan_fwd. theta may
    be [batch,Gth,N/2] (angle rows shared by groups of heads). With slots
    (int32 [batch] on the device), h is a pool [nslots,H,N,P] and row i
    updates h[slots[i]]; rows with an out-of-range slot are skipped (their y
    rows are left as they were)."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    a = decode_args(x, dt, lam, theta, B, C, A, D, h=h, y=y, Bprev=Bprev, xprev=xprev, B_bias=B_bias,
                    C_bias=C_bias, z=z, bc_norm=bc_norm, bc_eps=bc_eps, A_tok=A_tok, lam_fixed=lam_fixed,
                    slots=slots)
    st = lib().mamba3_decode_step(ctypes.byref(a), _stream(stream))
    if st != MAMBA3_OK:
        raise Mamba3Error(st, "mamba3_decode_step")
    return y
