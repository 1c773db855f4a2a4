"""Python binding of libm3scan.so: argument marshalling only.

Every step of the scan runs in the library's HIP kernels; PyTorch supplies the
device memory and the current HIP stream.  There is no fallback: if the library
is missing or a call fails, these functions raise.

Layouts are those of include/m3scan.h (contiguous, last index fastest):
  x, y (b, L, H, R, P)   dt, lam (b, L, H)   A, D (H,)   theta (b, L, G, N/2)
  B, C (b, L, G, R, N)   state h (b, H, N, P) fp32 or bf16 (the state dtype)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm3scan.so")

M3_F32, M3_BF16 = 0, 1
_IO = {torch.float32: M3_F32, torch.bfloat16: M3_BF16}
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape or dtype",
          -3: "workspace too small", -4: "HIP runtime error"}


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("rank", ctypes.c_int64), ("chunk", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32)]


class State(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("b_last", ctypes.c_void_p), ("x_last", ctypes.c_void_p)]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "ddt", "dA", "dlambda", "dtheta", "dB", "dC", "dD", "dh0", "db_last", "dx_last")]


class Fusion(ctypes.Structure):
    _fields_ = [("A_t", ctypes.c_void_p), ("b_norm_w", ctypes.c_void_p), ("c_norm_w", ctypes.c_void_p),
                ("b_bias", ctypes.c_void_p), ("c_bias", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("out_norm_w", ctypes.c_void_p), ("theta_groups", ctypes.c_int32)]


class M3Error(RuntimeError):
    def __init__(self, where: str, code: int):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({code})")
        self.code = code


_lib = None


def lib(path: str = LIB_PATH):
    """Load libm3scan.so once and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m state_space_sequence_scan_amd.build`")
    L = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.m3_status_string.restype = ctypes.c_char_p
    L.m3_status_string.argtypes = [ctypes.c_int]
    L.m3_version.restype = ctypes.c_int32
    L.m3_version.argtypes = []
    L.m3_prefill_workspace_size.restype = ctypes.c_int
    L.m3_prefill_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(sz)]
    L.m3_prefill_chunked.restype = ctypes.c_int
    L.m3_prefill_chunked.argtypes = ([ctypes.POINTER(Dims)] + [vp] * 8 +
                                     [ctypes.POINTER(State), ctypes.POINTER(State), vp, vp, sz, vp])
    L.m3_prefill_chunked_noalloc.restype = ctypes.c_int
    L.m3_prefill_chunked_noalloc.argtypes = ([ctypes.POINTER(Dims)] + [vp] * 8 +
                                             [ctypes.POINTER(State), ctypes.POINTER(State), vp, vp])
    L.m3_prefill_varlen.restype = ctypes.c_int
    L.m3_prefill_varlen.argtypes = ([ctypes.POINTER(Dims), vp, ctypes.c_int64] + [vp] * 8 +
                                    [ctypes.POINTER(State), ctypes.POINTER(State), vp, vp, sz, vp])
    L.m3_decode_step.restype = ctypes.c_int
    L.m3_decode_step.argtypes = [ctypes.POINTER(Dims)] + [vp] * 13
    L.m3_prefill_fused_workspace_size.restype = ctypes.c_int
    L.m3_prefill_fused_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Fusion), ctypes.POINTER(sz)]
    L.m3_prefill_fused.restype = ctypes.c_int
    L.m3_prefill_fused.argtypes = ([ctypes.POINTER(Dims)] + [vp] * 8 + [ctypes.POINTER(Fusion)] +
                                   [ctypes.POINTER(State), ctypes.POINTER(State), vp, vp, sz, vp])
    L.m3_prefill_varlen_fused.restype = ctypes.c_int
    L.m3_prefill_varlen_fused.argtypes = ([ctypes.POINTER(Dims), vp, ctypes.c_int64] + [vp] * 8 +
                                          [ctypes.POINTER(Fusion), ctypes.POINTER(State), ctypes.POINTER(State),
                                           vp, vp, sz, vp])
    L.m3_decode_step_fused.restype = ctypes.c_int
    L.m3_decode_step_fused.argtypes = [ctypes.POINTER(Dims)] + [vp] * 11 + [ctypes.POINTER(Fusion), vp, vp]
    L.m3_backward_workspace_size.restype = ctypes.c_int
    L.m3_backward_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(sz)]
    L.m3_backward_workspace_size_budget.restype = ctypes.c_int
    L.m3_backward_workspace_size_budget.argtypes = [ctypes.POINTER(Dims), ctypes.c_size_t, ctypes.POINTER(sz)]
    L.m3_backward_varlen.restype = ctypes.c_int
    L.m3_backward_varlen.argtypes = ([ctypes.POINTER(Dims), vp, ctypes.c_int64] + [vp] * 8 +
                                     [ctypes.POINTER(State), vp, vp, ctypes.POINTER(Grads), vp, sz, vp])
    L.m3_backward_per_token_A.restype = ctypes.c_int
    L.m3_backward_per_token_A.argtypes = ([ctypes.POINTER(Dims), vp, ctypes.c_int64] + [vp] * 8 +
                                          [ctypes.POINTER(State), vp, vp, ctypes.POINTER(Grads), vp, sz, vp])
    L.m3_prefill_sequences_per_workgroup.restype = ctypes.c_int
    L.m3_prefill_sequences_per_workgroup.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_int32)]
    L.m3_backward_parts.restype = ctypes.c_int
    L.m3_backward_parts.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int64)]
    L.m3_backward.restype = ctypes.c_int
    L.m3_backward.argtypes = ([ctypes.POINTER(Dims)] + [vp] * 8 + [ctypes.POINTER(State), vp, vp,
                              ctypes.POINTER(Grads), vp, sz, vp])
    _lib = L
    return L


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclasses.dataclass
class DecodeState:
    """Scan state: h (b,H,N,P) in fp32 or bf16 (its dtype is the state dtype of
    every call that reads or writes it), and the previous token's B (b,G,R,N) and
    X (b,H,R,P) in the io dtype (the trapezoid carry; None = zero)."""
    h: torch.Tensor
    b_last: Optional[torch.Tensor] = None
    x_last: Optional[torch.Tensor] = None


def make_dims(batch, seqlen, nheads, ngroups, headdim, dstate, rank, chunk, io_dtype,
              state_dtype: int = M3_F32) -> Dims:
    return Dims(batch, seqlen, nheads, ngroups, headdim, dstate, rank, chunk, io_dtype, state_dtype)


def workspace_size(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    rc = lib().m3_prefill_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != 0:
        raise M3Error("m3_prefill_workspace_size", rc)
    return int(n.value)


def prefill(x, dt, A, lam, theta, B, C, D, chunk: int, state_in: Optional[DecodeState] = None,
            out_state: bool = True, y: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None):
    """Chunked prefill.  Returns (y, DecodeState or None).

    state_dtype: dtype of the state read (state_in.h) and written (the returned
    h): torch.float32 or torch.bfloat16; default that of state_in.h, else fp32."""
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    dev = x.device
    io = x.dtype
    if io not in _IO:
        raise ValueError(f"x dtype {io} not supported (fp32 or bf16)")
    _check(x, "x", (b, L, H, R, P), io, dev)
    _check(dt, "dt", (b, L, H), torch.float32, dev)
    _check(lam, "lam", (b, L, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", (b, L, G, N // 2), torch.float32, dev)
    _check(B, "B", (b, L, G, R, N), io, dev)
    _check(C, "C", (b, L, G, R, N), io, dev)
    if state_dtype is None:
        state_dtype = state_in.h.dtype if state_in is not None else torch.float32
    if state_dtype not in _IO:
        raise ValueError(f"state dtype {state_dtype} not supported (fp32 or bf16)")
    dims = make_dims(b, L, H, G, P, N, R, chunk, _IO[io], _IO[state_dtype])
    if y is None:
        y = torch.empty_like(x)
    else:
        _check(y, "y", x.shape, io, dev)
    sin = None
    if state_in is not None:
        _check(state_in.h, "state_in.h", (b, H, N, P), state_dtype, dev)
        if state_in.b_last is not None:
            _check(state_in.b_last, "state_in.b_last", (b, G, R, N), io, dev)
            _check(state_in.x_last, "state_in.x_last", (b, H, R, P), io, dev)
        sin = State(state_in.h.data_ptr(),
                    None if state_in.b_last is None else state_in.b_last.data_ptr(),
                    None if state_in.x_last is None else state_in.x_last.data_ptr())
    sout = st = None
    if out_state:
        st = DecodeState(torch.empty((b, H, N, P), dtype=state_dtype, device=dev),
                         torch.empty((b, G, R, N), dtype=io, device=dev),
                         torch.empty((b, H, R, P), dtype=io, device=dev))
        sout = State(st.h.data_ptr(), st.b_last.data_ptr(), st.x_last.data_ptr())
    ws = workspace_size(dims)
    if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    rc = lib().m3_prefill_chunked(ctypes.byref(dims), _p(x), _p(dt), _p(A), _p(lam), _p(theta),
                                  _p(B), _p(C), _p(D),
                                  None if sin is None else ctypes.byref(sin),
                                  None if sout is None else ctypes.byref(sout), _p(y),
                                  _p(workspace) if ws > 0 else None,
                                  ws, _stream(dev))
    if rc != 0:
        raise M3Error("m3_prefill_chunked", rc)
    return y, st


NOALLOC_SCRATCH_BYTES = 64 << 20   # M3_NOALLOC_SCRATCH_BYTES of include/m3scan.h


def prefill_noalloc(x, dt, A, lam, theta, B, C, D, chunk: int, state_in: Optional[DecodeState] = None,
                    y: Optional[torch.Tensor] = None, state_out: Optional[DecodeState] = None):
    """``prefill`` through m3_prefill_chunked_noalloc: no workspace argument (the library's
    static scratch array serves as one).  The caller's y and state_out are used when given
    (nothing is allocated then); else they are allocated here.  Returns (y, state_out)."""
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    dev, io = x.device, x.dtype
    if io not in _IO:
        raise ValueError(f"x dtype {io} not supported (fp32 or bf16)")
    _check(x, "x", (b, L, H, R, P), io, dev)
    _check(dt, "dt", (b, L, H), torch.float32, dev)
    _check(lam, "lam", (b, L, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", (b, L, G, N // 2), torch.float32, dev)
    _check(B, "B", (b, L, G, R, N), io, dev)
    _check(C, "C", (b, L, G, R, N), io, dev)
    state_dtype = state_in.h.dtype if state_in is not None else (
        state_out.h.dtype if state_out is not None else torch.float32)
    dims = make_dims(b, L, H, G, P, N, R, chunk, _IO[io], _IO[state_dtype])
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.shape, io, dev)
    sin = None
    if state_in is not None:
        _check(state_in.h, "state_in.h", (b, H, N, P), state_dtype, dev)
        if state_in.b_last is not None:
            _check(state_in.b_last, "state_in.b_last", (b, G, R, N), io, dev)
            _check(state_in.x_last, "state_in.x_last", (b, H, R, P), io, dev)
        sin = State(state_in.h.data_ptr(),
                    None if state_in.b_last is None else state_in.b_last.data_ptr(),
                    None if state_in.x_last is None else state_in.x_last.data_ptr())
    if state_out is None:
        state_out = DecodeState(torch.empty((b, H, N, P), dtype=state_dtype, device=dev),
                                torch.empty((b, G, R, N), dtype=io, device=dev),
                                torch.empty((b, H, R, P), dtype=io, device=dev))
    _check(state_out.h, "state_out.h", (b, H, N, P), state_dtype, dev)
    sout = State(state_out.h.data_ptr(),
                 None if state_out.b_last is None else state_out.b_last.data_ptr(),
                 None if state_out.x_last is None else state_out.x_last.data_ptr())
    rc = lib().m3_prefill_chunked_noalloc(ctypes.byref(dims), _p(x), _p(dt), _p(A), _p(lam), _p(theta),
                                          _p(B), _p(C), _p(D), None if sin is None else ctypes.byref(sin),
                                          ctypes.byref(sout), _p(y), _stream(dev))
    if rc != 0:
        raise M3Error("m3_prefill_chunked_noalloc", rc)
    return y, state_out


def decode_step(state: DecodeState, x_t, dt_t, A, lam_t, theta_t, B_t, C_t, D,
                y_t: Optional[torch.Tensor] = None, advance: bool = True):
    """One decode step: updates state.h in place and returns y_t (b,H,R,P).

    With advance=True the state's carry becomes (B_t, x_t) -- references to the
    caller's tensors, no copy."""
    b, H, R, P = x_t.shape
    G, N = B_t.shape[1], B_t.shape[3]
    dev, io = x_t.device, x_t.dtype
    if io not in _IO:
        raise ValueError(f"x_t dtype {io} not supported (fp32 or bf16)")
    if state.h.dtype not in _IO:
        raise ValueError(f"state.h dtype {state.h.dtype} not supported (fp32 or bf16)")
    _check(state.h, "state.h", (b, H, N, P), state.h.dtype, dev)
    _check(x_t, "x_t", (b, H, R, P), io, dev)
    _check(dt_t, "dt_t", (b, H), torch.float32, dev)
    _check(lam_t, "lam_t", (b, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta_t, "theta_t", (b, G, N // 2), torch.float32, dev)
    _check(B_t, "B_t", (b, G, R, N), io, dev)
    _check(C_t, "C_t", (b, G, R, N), io, dev)
    if state.b_last is not None:
        _check(state.b_last, "state.b_last", (b, G, R, N), io, dev)
        _check(state.x_last, "state.x_last", (b, H, R, P), io, dev)
    if y_t is None:
        y_t = torch.empty_like(x_t)
    dims = make_dims(b, 1, H, G, P, N, R, 1, _IO[io], _IO[state.h.dtype])
    rc = lib().m3_decode_step(ctypes.byref(dims), _p(state.h), _p(state.b_last), _p(state.x_last),
                              _p(x_t), _p(dt_t), _p(A), _p(lam_t), _p(theta_t), _p(B_t), _p(C_t),
                              _p(D), _p(y_t), _stream(dev))
    if rc != 0:
        raise M3Error("m3_decode_step", rc)
    if advance:
        state.b_last, state.x_last = B_t, x_t
    return y_t


def prefill_varlen(x, dt, A, lam, theta, B, C, D, cu_seqlens, max_seqlen: int, chunk: int,
                   state_in: Optional[DecodeState] = None, out_state: bool = True,
                   y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   state_dtype: Optional[torch.dtype] = None):
    """Chunked prefill of a packed batch of variable-length sequences.

    x (T,H,R,P), dt/lam (T,H), theta (T,G,N/2), B/C (T,G,R,N) hold the sequences
    one after another; cu_seqlens (nseq+1,) int64 on the device gives their starts
    (cu_seqlens[0] = 0, cu_seqlens[-1] = T); max_seqlen bounds every length.
    Each sequence is scanned from its own state_in slice (else from zero).
    Returns (y (T,H,R,P), DecodeState with (nseq, ...) tensors or None)."""
    return _prefill_packed(x, dt, A, lam, theta, B, C, D, cu_seqlens, max_seqlen, chunk, state_in, out_state,
                           y, workspace, state_dtype, None)


def prefill_varlen_fused(x, dt, A, lam, theta, B, C, D, cu_seqlens, max_seqlen: int, chunk: int, A_t=None,
                         b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None, z=None, eps: float = 1e-6,
                         state_in: Optional[DecodeState] = None, out_state: bool = True,
                         y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         state_dtype: Optional[torch.dtype] = None, out_norm_w=None):
    """``prefill_varlen`` with the fused layer prologue/epilogue (m3_prefill_varlen_fused):
    per-token A (T,H), RMSNorm weights and biases of B and C (R,N), gate z (laid out as y),
    output norm weight (H,P); theta may carry finer angle groups (T, Gt, N/2)."""
    T, H, R, P = x.shape
    G, N = B.shape[1], B.shape[3]
    fu = _fusion(x.device, (R, N, (T, H), (T, H, R, P), (H, P)), A_t, b_norm_w, c_norm_w, b_bias, c_bias, z, eps,
                 x.dtype, out_norm_w, _theta_groups(theta, 1, G, H))
    return _prefill_packed(x, dt, A, lam, theta, B, C, D, cu_seqlens, max_seqlen, chunk, state_in, out_state,
                           y, workspace, state_dtype, fu)


def _prefill_packed(x, dt, A, lam, theta, B, C, D, cu_seqlens, max_seqlen, chunk, state_in, out_state, y,
                    workspace, state_dtype, fu):
    T, H, R, P = x.shape
    G, N = B.shape[1], B.shape[3]
    nseq = cu_seqlens.shape[0] - 1
    dev, io = x.device, x.dtype
    if io not in _IO:
        raise ValueError(f"x dtype {io} not supported (fp32 or bf16)")
    if nseq < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    _check(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int64, dev)
    _check(x, "x", (T, H, R, P), io, dev)
    _check(dt, "dt", (T, H), torch.float32, dev)
    _check(lam, "lam", (T, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", (T, fu.theta_groups if fu is not None and fu.theta_groups else G, N // 2),
           torch.float32, dev)
    _check(B, "B", (T, G, R, N), io, dev)
    _check(C, "C", (T, G, R, N), io, dev)
    if state_dtype is None:
        state_dtype = state_in.h.dtype if state_in is not None else torch.float32
    if state_dtype not in _IO:
        raise ValueError(f"state dtype {state_dtype} not supported (fp32 or bf16)")
    dims = make_dims(nseq, max_seqlen, H, G, P, N, R, chunk, _IO[io], _IO[state_dtype])
    if y is None:
        y = torch.empty_like(x)
    else:
        _check(y, "y", x.shape, io, dev)
    sin = None
    if state_in is not None:
        _check(state_in.h, "state_in.h", (nseq, H, N, P), state_dtype, dev)
        if state_in.b_last is not None:
            _check(state_in.b_last, "state_in.b_last", (nseq, G, R, N), io, dev)
            _check(state_in.x_last, "state_in.x_last", (nseq, H, R, P), io, dev)
        sin = State(state_in.h.data_ptr(),
                    None if state_in.b_last is None else state_in.b_last.data_ptr(),
                    None if state_in.x_last is None else state_in.x_last.data_ptr())
    sout = st = None
    if out_state:
        st = DecodeState(torch.empty((nseq, H, N, P), dtype=state_dtype, device=dev),
                         torch.empty((nseq, G, R, N), dtype=io, device=dev),
                         torch.empty((nseq, H, R, P), dtype=io, device=dev))
        sout = State(st.h.data_ptr(), st.b_last.data_ptr(), st.x_last.data_ptr())
    ws = workspace_size(dims) if fu is None else fused_workspace_size(dims, fu)
    if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    common = (ctypes.byref(dims), _p(cu_seqlens), ctypes.c_int64(T), _p(x), _p(dt), _p(A), _p(lam), _p(theta),
              _p(B), _p(C), _p(D))
    tail = (None if sin is None else ctypes.byref(sin), None if sout is None else ctypes.byref(sout), _p(y),
            _p(workspace) if ws > 0 else None, ws, _stream(dev))
    if fu is None:
        rc, name = lib().m3_prefill_varlen(*common, *tail), "m3_prefill_varlen"
    else:
        rc, name = lib().m3_prefill_varlen_fused(*common, ctypes.byref(fu), *tail), "m3_prefill_varlen_fused"
    if rc != 0:
        raise M3Error(name, rc)
    return y, st


def backward_workspace_size(dims: Dims, checkpoint_bytes: Optional[int] = None) -> int:
    """Workspace bytes of the backward calls: for the default checkpoint budget
    (m3_backward_workspace_size), or for ``checkpoint_bytes`` of kept states
    (m3_backward_workspace_size_budget)."""
    n = ctypes.c_size_t(0)
    if checkpoint_bytes is None:
        rc = lib().m3_backward_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    else:
        rc = lib().m3_backward_workspace_size_budget(ctypes.byref(dims), int(checkpoint_bytes), ctypes.byref(n))
    if rc != 0:
        raise M3Error("m3_backward_workspace_size", rc)
    return int(n.value)


def prefill_sequences_per_workgroup(dims: Dims) -> int:
    """How many sequences one workgroup of m3_prefill_chunked sweeps one after another."""
    n = ctypes.c_int32(0)
    rc = lib().m3_prefill_sequences_per_workgroup(ctypes.byref(dims), ctypes.byref(n))
    if rc != 0:
        raise M3Error("m3_prefill_sequences_per_workgroup", rc)
    return int(n.value)


def backward_parts(dims: Dims):
    """(parts, tokens_per_part): how m3_backward splits each (b, h) sequence."""
    n = ctypes.c_int32(0)
    t = ctypes.c_int64(0)
    rc = lib().m3_backward_parts(ctypes.byref(dims), ctypes.byref(n), ctypes.byref(t))
    if rc != 0:
        raise M3Error("m3_backward_parts", rc)
    return int(n.value), int(t.value)


def _backward_state(state_in, nb, H, G, N, P, R, io, dev):
    """The state_in argument of a backward call (nb sequences) and its state dtype."""
    state_dtype = state_in.h.dtype if state_in is not None else torch.float32
    if state_in is None:
        return None, state_dtype
    _check(state_in.h, "state_in.h", (nb, H, N, P), state_dtype, dev)
    if state_in.b_last is not None:
        _check(state_in.b_last, "state_in.b_last", (nb, G, R, N), io, dev)
        _check(state_in.x_last, "state_in.x_last", (nb, H, R, P), io, dev)
    return State(state_in.h.data_ptr(),
                 None if state_in.b_last is None else state_in.b_last.data_ptr(),
                 None if state_in.x_last is None else state_in.x_last.data_ptr()), state_dtype


def _backward_grads(lead, nb, H, G, N, P, R, want_state_grads, grads, dev, dA_per_token=False):
    """Output tensors of a backward call (per-token ones with leading shape `lead`)."""
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"dx": lead + (H, R, P), "ddt": lead + (H,), "dA": lead + (H,) if dA_per_token else (H,),
              "dlam": lead + (H,),
              "dtheta": lead + (G, N // 2), "dB": lead + (G, R, N), "dC": lead + (G, R, N), "dD": (H,)}
    if want_state_grads:
        shapes.update({"dh0": (nb, H, N, P), "db_last": (nb, G, R, N), "dx_last": (nb, H, R, P)})
    out = {} if grads is None else dict(grads)
    for k, shp in shapes.items():
        if k not in out:
            out[k] = torch.empty(shp, **f32)
        _check(out[k], k, shp, torch.float32, dev)
    gs = Grads(*[out[k].data_ptr() if k in out else None for k in
                 ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0", "db_last", "dx_last")])
    return out, gs


def _backward_workspace(dims, workspace, dev, checkpoint_bytes):
    """(bytes, tensor): a caller's workspace whole when it holds what the budget needs (the
    call keeps as many states as it allows), else a new one of that size."""
    ws = backward_workspace_size(dims, checkpoint_bytes)
    if workspace is not None and workspace.numel() * workspace.element_size() >= ws:
        return workspace.numel() * workspace.element_size(), workspace
    if ws > 0:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    return ws, workspace


def backward(x, dt, A, lam, theta, B, C, D, dy, dh_out=None, state_in: Optional[DecodeState] = None,
             want_state_grads: bool = True, workspace: Optional[torch.Tensor] = None,
             grads: Optional[dict] = None, checkpoint_bytes: Optional[int] = None):
    """Backward pass of the scan: gradients of sum <dy, y> + <dh_out, h_L>.

    Returns a dict of fp32 tensors dx, ddt, dA, dlam, dtheta, dB, dC, dD and, with
    want_state_grads, dh0 (b,H,N,P), db_last (b,G,R,N), dx_last (b,H,R,P).
    ``grads`` may hold preallocated output tensors of those names; ``checkpoint_bytes``
    bounds the states kept for the reverse sweep (default 4 GiB)."""
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    dev = x.device
    io = x.dtype
    if io not in _IO:
        raise ValueError(f"x dtype {io} not supported (fp32 or bf16)")
    _check(x, "x", (b, L, H, R, P), io, dev)
    _check(dy, "dy", (b, L, H, R, P), io, dev)
    _check(dt, "dt", (b, L, H), torch.float32, dev)
    _check(lam, "lam", (b, L, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", (b, L, G, N // 2), torch.float32, dev)
    _check(B, "B", (b, L, G, R, N), io, dev)
    _check(C, "C", (b, L, G, R, N), io, dev)
    if dh_out is not None:
        _check(dh_out, "dh_out", (b, H, N, P), torch.float32, dev)
    sin, state_dtype = _backward_state(state_in, b, H, G, N, P, R, io, dev)
    dims = make_dims(b, L, H, G, P, N, R, 1, _IO[io], _IO[state_dtype])
    out, gs = _backward_grads((b, L), b, H, G, N, P, R, want_state_grads, grads, dev)
    ws, workspace = _backward_workspace(dims, workspace, dev, checkpoint_bytes)
    rc = lib().m3_backward(ctypes.byref(dims), _p(x), _p(dt), _p(A), _p(lam), _p(theta), _p(B), _p(C),
                           _p(D), None if sin is None else ctypes.byref(sin), _p(dy), _p(dh_out),
                           ctypes.byref(gs), _p(workspace) if ws > 0 else None, ws, _stream(dev))
    if rc != 0:
        raise M3Error("m3_backward", rc)
    return out


def backward_varlen(x, dt, A, lam, theta, B, C, D, dy, cu_seqlens, max_seqlen: int, dh_out=None,
                    state_in: Optional[DecodeState] = None, want_state_grads: bool = True,
                    workspace: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
                    checkpoint_bytes: Optional[int] = None):
    """Backward pass of prefill_varlen (m3_backward_varlen): the packed layouts of
    prefill_varlen for the inputs, dy and the per-token gradients (T, ...), per-sequence
    dh_out, state_in and state gradients (nseq, ...).  Returns the dict of ``backward``."""
    T, H, R, P = x.shape
    G, N = B.shape[1], B.shape[3]
    nseq = cu_seqlens.shape[0] - 1
    dev, io = x.device, x.dtype
    if io not in _IO:
        raise ValueError(f"x dtype {io} not supported (fp32 or bf16)")
    if nseq < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    _check(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int64, dev)
    _check(x, "x", (T, H, R, P), io, dev)
    _check(dy, "dy", (T, H, R, P), io, dev)
    _check(dt, "dt", (T, H), torch.float32, dev)
    _check(lam, "lam", (T, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", (T, G, N // 2), torch.float32, dev)
    _check(B, "B", (T, G, R, N), io, dev)
    _check(C, "C", (T, G, R, N), io, dev)
    if dh_out is not None:
        _check(dh_out, "dh_out", (nseq, H, N, P), torch.float32, dev)
    sin, state_dtype = _backward_state(state_in, nseq, H, G, N, P, R, io, dev)
    dims = make_dims(nseq, max_seqlen, H, G, P, N, R, 1, _IO[io], _IO[state_dtype])
    out, gs = _backward_grads((T,), nseq, H, G, N, P, R, want_state_grads, grads, dev)
    ws, workspace = _backward_workspace(dims, workspace, dev, checkpoint_bytes)
    rc = lib().m3_backward_varlen(ctypes.byref(dims), _p(cu_seqlens), T, _p(x), _p(dt), _p(A), _p(lam),
                                  _p(theta), _p(B), _p(C), _p(D), None if sin is None else ctypes.byref(sin),
                                  _p(dy), _p(dh_out), ctypes.byref(gs), _p(workspace) if ws > 0 else None, ws,
                                  _stream(dev))
    if rc != 0:
        raise M3Error("m3_backward_varlen", rc)
    return out


def _fusion(dev, shapes, A_t=None, b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None, z=None,
            eps: float = 1e-6, io=None, out_norm_w=None, theta_groups: int = 0):
    """Checks the fusion tensors against the call's shapes and packs them.  shapes is
    (R, N, A_t shape, z shape, (H, P)); theta_groups is the angle-group count (0: that of B, C)."""
    R, N, at_shape, z_shape, hp = shapes
    for t, name in ((b_norm_w, "b_norm_w"), (c_norm_w, "c_norm_w"), (b_bias, "b_bias"), (c_bias, "c_bias")):
        if t is not None:
            _check(t, name, (R, N), torch.float32, dev)
    if A_t is not None:
        _check(A_t, "A_t", at_shape, torch.float32, dev)
    if z is not None:
        _check(z, "z", z_shape, io, dev)
    if out_norm_w is not None:
        _check(out_norm_w, "out_norm_w", hp, torch.float32, dev)
    return Fusion(*[None if t is None else t.data_ptr() for t in (A_t, b_norm_w, c_norm_w, b_bias, c_bias, z)],
                  float(eps), None if out_norm_w is None else out_norm_w.data_ptr(), int(theta_groups))


def _theta_groups(theta, axis, G, H):
    """Angle groups of a fused call from theta's shape: 0 when they are B and C's G."""
    Gt = theta.shape[axis]
    if Gt == G:
        return 0
    if Gt % G != 0 or H % Gt != 0:
        raise ValueError(f"theta has {Gt} angle groups: not a multiple of G={G} dividing H={H}")
    return Gt


def fused_workspace_size(dims: Dims, fu: Fusion) -> int:
    n = ctypes.c_size_t(0)
    rc = lib().m3_prefill_fused_workspace_size(ctypes.byref(dims), ctypes.byref(fu), ctypes.byref(n))
    if rc != 0:
        raise M3Error("m3_prefill_fused_workspace_size", rc)
    return int(n.value)


def prefill_fused(x, dt, A, lam, theta, B, C, D, chunk: int, A_t=None, b_norm_w=None, c_norm_w=None,
                  b_bias=None, c_bias=None, z=None, eps: float = 1e-6,
                  state_in: Optional[DecodeState] = None, out_state: bool = True,
                  y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  state_dtype: Optional[torch.dtype] = None, out_norm_w=None):
    """``prefill`` with the fused layer prologue/epilogue (m3_prefill_fused): per-token A
    (b,L,H), RMSNorm weights and biases of B and C (R,N), gate z (laid out as y), output
    norm weight (H,P); theta may carry finer angle groups than B and C, (b, L, Gt, N/2)
    (Gt = H: angles per head)."""
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    dev = x.device
    io = x.dtype
    Gt = _theta_groups(theta, 2, G, H)
    _check(x, "x", (b, L, H, R, P), io, dev)
    _check(dt, "dt", (b, L, H), torch.float32, dev)
    _check(lam, "lam", (b, L, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", (b, L, Gt or G, N // 2), torch.float32, dev)
    _check(B, "B", (b, L, G, R, N), io, dev)
    _check(C, "C", (b, L, G, R, N), io, dev)
    fu = _fusion(dev, (R, N, (b, L, H), (b, L, H, R, P), (H, P)), A_t, b_norm_w, c_norm_w, b_bias, c_bias, z, eps,
                 io, out_norm_w, Gt)
    if state_dtype is None:
        state_dtype = state_in.h.dtype if state_in is not None else torch.float32
    dims = make_dims(b, L, H, G, P, N, R, chunk, _IO[io], _IO[state_dtype])
    if y is None:
        y = torch.empty_like(x)
    sin = None
    if state_in is not None:
        _check(state_in.h, "state_in.h", (b, H, N, P), state_dtype, dev)
        if state_in.b_last is not None:
            _check(state_in.b_last, "state_in.b_last", (b, G, R, N), io, dev)
            _check(state_in.x_last, "state_in.x_last", (b, H, R, P), io, dev)
        sin = State(state_in.h.data_ptr(),
                    None if state_in.b_last is None else state_in.b_last.data_ptr(),
                    None if state_in.x_last is None else state_in.x_last.data_ptr())
    sout = st = None
    if out_state:
        st = DecodeState(torch.empty((b, H, N, P), dtype=state_dtype, device=dev),
                         torch.empty((b, G, R, N), dtype=io, device=dev),
                         torch.empty((b, H, R, P), dtype=io, device=dev))
        sout = State(st.h.data_ptr(), st.b_last.data_ptr(), st.x_last.data_ptr())
    ws = fused_workspace_size(dims, fu)
    if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    rc = lib().m3_prefill_fused(ctypes.byref(dims), _p(x), _p(dt), _p(A), _p(lam), _p(theta), _p(B), _p(C),
                                _p(D), ctypes.byref(fu), None if sin is None else ctypes.byref(sin),
                                None if sout is None else ctypes.byref(sout), _p(y),
                                _p(workspace) if ws > 0 else None, ws, _stream(dev))
    if rc != 0:
        raise M3Error("m3_prefill_fused", rc)
    return y, st


def decode_step_fused(state: DecodeState, x_t, dt_t, A, lam_t, theta_t, B_t, C_t, D, A_t=None,
                      b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None, z=None, eps: float = 1e-6,
                      y_t: Optional[torch.Tensor] = None, advance: bool = True, out_norm_w=None):
    """``decode_step`` with the fused prologue/epilogue (m3_decode_step_fused): A_t (b,H),
    norm weights and biases (R,N), gate z (b,H,R,P), output norm weight (H,P); theta_t may
    carry finer angle groups (b, Gt, N/2).  The carry stays raw."""
    b, H, R, P = x_t.shape
    G, N = B_t.shape[1], B_t.shape[3]
    dev = x_t.device
    io = x_t.dtype
    _check(state.h, "state.h", (b, H, N, P), state.h.dtype, dev)
    Gt = _theta_groups(theta_t, 1, G, H)
    _check(theta_t, "theta_t", (b, Gt or G, N // 2), torch.float32, dev)
    fu = _fusion(dev, (R, N, (b, H), (b, H, R, P), (H, P)), A_t, b_norm_w, c_norm_w, b_bias, c_bias, z, eps, io,
                 out_norm_w, Gt)
    dims = make_dims(b, 1, H, G, P, N, R, 1, _IO[io], _IO[state.h.dtype])
    if y_t is None:
        y_t = torch.empty_like(x_t)
    rc = lib().m3_decode_step_fused(ctypes.byref(dims), _p(state.h), _p(state.b_last), _p(state.x_last), _p(x_t),
                                    _p(dt_t), _p(A), _p(lam_t), _p(theta_t), _p(B_t), _p(C_t), _p(D),
                                    ctypes.byref(fu), _p(y_t), _stream(dev))
    if rc != 0:
        raise M3Error("m3_decode_step_fused", rc)
    if advance:
        state.b_last, state.x_last = B_t, x_t
    return y_t


def backward_per_token_A(x, dt, A_t, lam, theta, B, C, D, dy, cu_seqlens=None, max_seqlen: Optional[int] = None,
                         dh_out=None, state_in: Optional[DecodeState] = None, want_state_grads: bool = True,
                         workspace: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
                         checkpoint_bytes: Optional[int] = None):
    """Backward pass with a per-token decay rate A_t (m3_backward_per_token_A): the
    layouts of ``backward`` (cu_seqlens None) or ``backward_varlen`` (cu_seqlens and
    max_seqlen given), with A_t fp32 shaped like dt; dA is returned per token, shaped
    like A_t.  Returns the dict of ``backward``."""
    packed = cu_seqlens is not None
    lead = tuple(x.shape[:-3])
    if len(lead) != (1 if packed else 2):
        raise ValueError(f"x: {x.dim()} dimensions, expected {4 if packed else 5}")
    H, R, P = x.shape[-3:]
    G, N = B.shape[-3], B.shape[-1]
    dev, io = x.device, x.dtype
    if io not in _IO:
        raise ValueError(f"x dtype {io} not supported (fp32 or bf16)")
    if packed:
        nseq = cu_seqlens.shape[0] - 1
        if nseq < 1:
            raise ValueError("cu_seqlens needs at least two entries")
        if max_seqlen is None:
            raise ValueError("max_seqlen is needed with cu_seqlens")
        _check(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int64, dev)
        nb, L = nseq, max_seqlen
    else:
        nb, L = lead
    _check(x, "x", lead + (H, R, P), io, dev)
    _check(dy, "dy", lead + (H, R, P), io, dev)
    _check(dt, "dt", lead + (H,), torch.float32, dev)
    _check(A_t, "A_t", lead + (H,), torch.float32, dev)
    _check(lam, "lam", lead + (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(theta, "theta", lead + (G, N // 2), torch.float32, dev)
    _check(B, "B", lead + (G, R, N), io, dev)
    _check(C, "C", lead + (G, R, N), io, dev)
    if dh_out is not None:
        _check(dh_out, "dh_out", (nb, H, N, P), torch.float32, dev)
    sin, state_dtype = _backward_state(state_in, nb, H, G, N, P, R, io, dev)
    dims = make_dims(nb, L, H, G, P, N, R, 1, _IO[io], _IO[state_dtype])
    out, gs = _backward_grads(lead, nb, H, G, N, P, R, want_state_grads, grads, dev, dA_per_token=True)
    ws, workspace = _backward_workspace(dims, workspace, dev, checkpoint_bytes)
    rc = lib().m3_backward_per_token_A(ctypes.byref(dims), _p(cu_seqlens), lead[0] if packed else 0, _p(x),
                                       _p(dt), _p(A_t), _p(lam), _p(theta), _p(B), _p(C), _p(D),
                                       None if sin is None else ctypes.byref(sin), _p(dy), _p(dh_out),
                                       ctypes.byref(gs), _p(workspace) if ws > 0 else None, ws, _stream(dev))
    if rc != 0:
        raise M3Error("m3_backward_per_token_A", rc)
    return out
