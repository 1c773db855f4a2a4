"""CPU oracle for the Mamba-3 SSM scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it shares no code with the HIP library.

Contents
  * ``scan``          -- ctypes front end of ``m3_oracle.c``: the sequential
                         fp64 loop over t (the definition written out).
  * ``scan_fused``    -- the scan with the fused prologue/epilogue of a Mamba-3
                         layer written out around it: RMSNorm and bias of B and C
                         (``bc_norm``), per-token A, angles per head over shared B and
                         C (``expand_groups``), the output gate (``gate``) and the
                         output RMSNorm (``out_norm``).
  * ``scan_backward`` -- its reverse-mode derivative (the adjoint loop of
                         ``m3_oracle.c``), pinned by finite differences of ``scan``.
  * ``m3_oracle_np``  -- two independent numpy formulations used to pin it:
                         complex modes (``scan_complex``) and the dense
                         semiseparable matrix (``scan_dense``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB = os.path.join(_HERE, "libm3_oracle.so")
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "ngroups", "headdim", "dstate", "rank")]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (-O2, IEEE fp64: no fast-math)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-fno-fast-math", "-Wall", "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def load(path: str = _LIB):
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(force=False, out=path)
    lib = ctypes.CDLL(path)
    f = lib.m3o_scan
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(_Dims)] + [ctypes.c_void_p] * 13 + [ctypes.c_int]
    f = lib.m3o_scan_rounded
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(_Dims)] + [ctypes.c_void_p] * 14 + [ctypes.c_int]
    f = lib.m3o_scan_ex
    f.restype = ctypes.c_int
    f.argtypes = ([ctypes.POINTER(_Dims)] + [ctypes.c_void_p] * 3 + [ctypes.c_int] +
                  [ctypes.c_void_p] * 11 + [ctypes.c_int])
    f = lib.m3o_scan_backward
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(_Dims)] + [ctypes.c_void_p] * 24 + [ctypes.c_int]
    f = lib.m3o_scan_backward_ex
    f.restype = ctypes.c_int
    f.argtypes = ([ctypes.POINTER(_Dims)] + [ctypes.c_void_p] * 3 + [ctypes.c_int] +
                  [ctypes.c_void_p] * 21 + [ctypes.c_int])
    lib.m3o_round_bf16.restype = ctypes.c_double
    lib.m3o_round_bf16.argtypes = [ctypes.c_double]
    lib.m3o_max_threads.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def max_threads() -> int:
    return int(load().m3o_max_threads())


def _f64(a):
    """Inputs are widened to fp64 (exact for fp32 and bf16 values)."""
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def round_bf16(v: float) -> float:
    """Nearest bf16 value of a float (ties to even), as the oracle rounds a state."""
    return float(load().m3o_round_bf16(float(v)))


def scan(x, dt, A, lam, theta, B, C, D, state_in=None, nthreads: int = 0, lib_path: str = _LIB,
         round_after=None):
    """Sequential fp64 scan.

    Shapes: x (b,L,H,R,P), dt/lam (b,L,H), A (H,) or per token (b,L,H), D (H,), theta (b,L,G,N/2),
    B/C (b,L,G,R,N).  ``state_in`` is None or a tuple (h0 (b,H,N,P),
    b_last (b,G,R,N), x_last (b,H,R,P)); b_last/x_last may be None.
    ``round_after``: None (full-precision state) or L booleans; after each
    flagged token the state is replaced by its nearest bf16 value (the output
    of that token still reads the unrounded state).
    Returns (y (b,L,H,R,P) float64, h_out (b,H,N,P) float64).
    """
    x, dt, A, lam, theta, B, C, D = map(_f64, (x, dt, A, lam, theta, B, C, D))
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    assert dt.shape == (b, L, H) and lam.shape == (b, L, H)
    assert (A.shape == (H,) or A.shape == (b, L, H)) and D.shape == (H,)
    a_tok = int(A.shape != (H,))
    assert theta.shape == (b, L, G, N // 2)
    assert B.shape == (b, L, G, R, N) and C.shape == (b, L, G, R, N)
    h0 = bl = xl = None
    if state_in is not None:
        h0, bl, xl = state_in
        if h0 is not None:
            h0 = _f64(h0)
            assert h0.shape == (b, H, N, P)
        if bl is not None:
            bl = _f64(bl)
            assert bl.shape == (b, G, R, N)
        if xl is not None:
            xl = _f64(xl)
            assert xl.shape == (b, H, R, P)
    y = np.empty((b, L, H, R, P), dtype=np.float64)
    h_out = np.empty((b, H, N, P), dtype=np.float64)
    d = _Dims(b, L, H, G, P, N, R)
    if round_after is None and not a_tok:
        rc = load(lib_path).m3o_scan(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(lam),
                                     _ptr(theta), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(bl),
                                     _ptr(xl), _ptr(y), _ptr(h_out), int(nthreads))
    else:
        ra = None
        if round_after is not None:
            ra = np.ascontiguousarray(np.asarray(round_after, dtype=bool), dtype=np.uint8)
            assert ra.shape == (L,)
        rc = load(lib_path).m3o_scan_ex(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), a_tok,
                                        _ptr(lam), _ptr(theta), _ptr(B), _ptr(C), _ptr(D),
                                        _ptr(h0), _ptr(bl), _ptr(xl), _ptr(ra), _ptr(y),
                                        _ptr(h_out), int(nthreads))
    if rc != 0:
        raise ValueError(f"m3o_scan failed with code {rc}")
    return y, h_out


def scan_backward(x, dt, A, lam, theta, B, C, D, dy, dh_out=None, state_in=None, nthreads: int = 0,
                  lib_path: str = _LIB):
    """Gradient of sum_t <dy_t, y_t> + <dh_out, h_L> with respect to every input of ``scan``.

    Same shapes and ``state_in`` as ``scan``; ``dy`` has the shape of y and ``dh_out``
    (optional) that of the final state.  Returns a dict with dx, ddt, dA, dlam, dtheta,
    dB, dC, dD (shapes of the inputs; dB, dC and dtheta summed over the heads of a
    group, dA and dD over batch and tokens), dh0 (b,H,N,P) and, when the state carries
    a previous input, db_last (b,G,R,N) and dx_last (b,H,R,P).  A per-token decay rate
    A (b, L, H) gives dA per token, (b, L, H).
    """
    x, dt, A, lam, theta, B, C, D, dy = map(_f64, (x, dt, A, lam, theta, B, C, D, dy))
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    assert dy.shape == x.shape
    h0 = bl = xl = None
    if state_in is not None:
        h0, bl, xl = state_in
        h0 = None if h0 is None else _f64(h0)
        bl = None if bl is None else _f64(bl)
        xl = None if xl is None else _f64(xl)
    dho = None if dh_out is None else _f64(dh_out)
    if dho is not None:
        assert dho.shape == (b, H, N, P)
    carry = bl is not None and xl is not None
    a_tok = A.ndim == 3
    if a_tok:
        assert A.shape == (b, L, H)
    out = {"dx": np.empty_like(x), "ddt": np.empty_like(dt), "dA": np.empty((b, L, H) if a_tok else (H,)),
           "dlam": np.empty_like(lam), "dtheta": np.empty_like(theta), "dB": np.empty_like(B),
           "dC": np.empty_like(C), "dD": np.empty((H,)), "dh0": np.empty((b, H, N, P))}
    if carry:
        out["db_last"] = np.empty((b, G, R, N))
        out["dx_last"] = np.empty((b, H, R, P))
    d = _Dims(b, L, H, G, P, N, R)
    rc = load(lib_path).m3o_scan_backward_ex(
        ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), int(a_tok), _ptr(lam), _ptr(theta), _ptr(B), _ptr(C),
        _ptr(D), _ptr(h0), _ptr(bl), _ptr(xl), _ptr(dy), _ptr(dho), _ptr(out["dx"]),
        _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dlam"]), _ptr(out["dtheta"]), _ptr(out["dB"]),
        _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]), _ptr(out.get("db_last")),
        _ptr(out.get("dx_last")), int(nthreads))
    if rc != 0:
        raise ValueError(f"m3o_scan_backward failed with code {rc}")
    return out


def bc_norm(M, weight=None, bias=None, eps: float = 1e-6):
    """BCNorm of B or C (b, L, G, R, N): each length-N vector M[b, t, g, r, :] divided by its
    root mean square (sqrt(mean(M^2) + eps)) and scaled by weight[r, :] when a weight is given,
    then bias[r, :] added when a bias is given (the bias of B and C follows BCNorm: Mamba-3
    blog, part 1, "Normalization" and "Removing the short convolution").  fp64."""
    M = _f64(M)
    if weight is not None:
        rms = np.sqrt(np.mean(M * M, axis=-1, keepdims=True) + eps)
        M = M / rms * _f64(weight)[None, None, None]
    if bias is not None:
        M = M + _f64(bias)[None, None, None]
    return M


def gate(y, z):
    """Output gate y * silu(z), silu(v) = v / (1 + exp(-v)).  fp64."""
    y, z = _f64(y), _f64(z)
    return y * z / (1.0 + np.exp(-z))


def out_norm(y, weight, eps: float = 1e-6):
    """RMSNorm of the scan's output before the out-projection (the Mamba-3 paper note,
    "Architecture": kept in hybrid models): each row y[b, t, h, r, :] of P values divided by
    its root mean square sqrt(mean(y^2) + eps) and multiplied by weight[h, :] (one weight per
    channel of the head, shared by its R rows).  fp64."""
    y = _f64(y)
    rms = np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return y / rms * _f64(weight)[None, None, :, None, :]


def expand_groups(M, groups: int):
    """Repeat each group of M (b, L, G, ...) over groups // G consecutive groups: the B or C
    a finer grouping of heads sees (group j of the finer grouping holds group j // (groups // G))."""
    G = M.shape[2]
    assert groups % G == 0
    return np.repeat(_f64(M), groups // G, axis=2)


def scan_fused(x, dt, A, lam, theta, B, C, D, b_norm_w=None, c_norm_w=None, b_bias=None,
               c_bias=None, eps: float = 1e-6, z=None, state_in=None, round_after=None,
               out_norm_w=None):
    """``scan`` with the layer's prologue and epilogue around it: B and C through
    ``bc_norm`` (the carried previous B of state_in as well), A per head (H,) or per token
    (b,L,H), y through ``gate`` when z is given and then through ``out_norm`` when
    out_norm_w (H, P) is given.

    theta (b, L, Gt, N/2) may have more groups than B and C (G): G divides Gt, Gt divides H,
    head h turns with angle group h // (H/Gt) and reads B, C group h // (H/G); with Gt = H
    every head has its own angles over shared B and C.  Each head then sees exactly the
    grouped scan of B and C repeated over the angle groups (``expand_groups``).
    Returns (y, h_out)."""
    Bn = bc_norm(B, b_norm_w, b_bias, eps)
    Cn = bc_norm(C, c_norm_w, c_bias, eps)
    st = state_in
    bl = None
    if state_in is not None and state_in[1] is not None:
        bl = bc_norm(_f64(state_in[1])[:, None], b_norm_w, b_bias, eps)[:, 0]
        st = (state_in[0], bl, state_in[2])
    Gt = theta.shape[2]
    if Gt != B.shape[2]:
        Bn = expand_groups(Bn, Gt)
        Cn = expand_groups(Cn, Gt)
        if bl is not None:
            st = (st[0], expand_groups(bl[:, None], Gt)[:, 0], st[2])
    y, h = scan(x, dt, A, lam, theta, Bn, Cn, D, state_in=st, round_after=round_after)
    if z is not None:
        y = gate(y, z)
    if out_norm_w is not None:
        y = out_norm(y, out_norm_w, eps)
    return y, h
