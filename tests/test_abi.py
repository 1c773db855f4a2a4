"""The C-ABI library loads and exports what include/m3scan.h declares; argument
errors come back as status codes before anything is launched (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from state_space_sequence_scan_amd import m3scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3scan.h")


def declared_symbols():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(m3_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m3scan.LIB_PATH):
        from state_space_sequence_scan_amd import build
        build.build()
    return m3scan.lib()


def test_header_declares_the_entry_points():
    assert declared_symbols() == ["m3_backward", "m3_backward_parts", "m3_backward_per_token_A", "m3_backward_varlen",
                                  "m3_backward_workspace_size", "m3_decode_step",
                                  "m3_decode_step_fused", "m3_prefill_chunked", "m3_prefill_fused",
                                  "m3_prefill_varlen", "m3_prefill_varlen_fused", "m3_prefill_workspace_size", "m3_status_string",
                                  "m3_version"]


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", m3scan.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (m3_\w+)$", out, re.M))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(lib, s)


def test_status_strings_and_version(lib):
    for code, text in m3scan.STATUS.items():
        assert lib.m3_status_string(code).decode() == text
    assert lib.m3_status_string(99).decode() == "unknown status"
    assert lib.m3_version() >= 100


def _dims(**kw):
    base = dict(batch=2, seqlen=64, nheads=4, ngroups=2, headdim=16, dstate=16, rank=2, chunk=16,
                io_dtype=m3scan.M3_F32)
    base.update(kw)
    return m3scan.Dims(**base)


BAD_DIMS = [dict(batch=0), dict(seqlen=-1), dict(nheads=0), dict(ngroups=3), dict(dstate=15),
            dict(headdim=0), dict(rank=0), dict(chunk=0), dict(io_dtype=7), dict(state_dtype=5)]


@pytest.mark.parametrize("kw", BAD_DIMS, ids=lambda k: next(iter(k)))
def test_workspace_size_rejects_bad_dims(lib, kw):
    n = ctypes.c_size_t(123)
    assert lib.m3_prefill_workspace_size(ctypes.byref(_dims(**kw)), ctypes.byref(n)) == -1
    assert lib.m3_prefill_workspace_size(None, ctypes.byref(n)) == -1
    assert lib.m3_prefill_workspace_size(ctypes.byref(_dims()), None) == -1


def test_workspace_size_ok(lib):
    n = ctypes.c_size_t(123)
    assert lib.m3_prefill_workspace_size(ctypes.byref(_dims()), ctypes.byref(n)) == 0
    assert n.value >= 0
    d = _dims(state_dtype=m3scan.M3_BF16)       # bf16 state: accepted, same workspace
    m = ctypes.c_size_t(123)
    assert lib.m3_prefill_workspace_size(ctypes.byref(d), ctypes.byref(m)) == 0
    assert m.value == n.value


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its checks first


@pytest.mark.parametrize("kw", BAD_DIMS, ids=lambda k: next(iter(k)))
def test_prefill_rejects_bad_dims(lib, kw):
    d = _dims(**kw)
    rc = lib.m3_prefill_chunked(ctypes.byref(d), *[FAKE] * 8, None, None, FAKE, None, 0, None)
    assert rc == -1


def test_prefill_rejects_null_inputs(lib):
    d = _dims()
    for i in range(8):
        args = [FAKE] * 8
        args[i] = None
        assert lib.m3_prefill_chunked(ctypes.byref(d), *args, None, None, FAKE, None, 0, None) == -1
    # y missing
    assert lib.m3_prefill_chunked(ctypes.byref(d), *[FAKE] * 8, None, None, None, None, 0, None) == -1
    # state_in without h, or with half a carry
    s = m3scan.State(None, None, None)
    assert lib.m3_prefill_chunked(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(s), None, FAKE, None, 0,
                                  None) == -1
    s = m3scan.State(0x1000, 0x1000, None)
    assert lib.m3_prefill_chunked(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(s), None, FAKE, None, 0,
                                  None) == -1


def test_prefill_rejects_unsupported(lib):
    d = _dims(rank=9, dstate=512, headdim=512, chunk=256)
    n = ctypes.c_size_t(0)
    assert lib.m3_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == -2
    assert lib.m3_prefill_chunked(ctypes.byref(d), *[FAKE] * 8, None, None, FAKE, None, 0, None) == -2


@pytest.mark.parametrize("kw", [k for k in BAD_DIMS if "seqlen" not in k and "chunk" not in k],
                         ids=lambda k: next(iter(k)))
def test_decode_rejects_bad_dims(lib, kw):
    d = _dims(**kw)
    assert lib.m3_decode_step(ctypes.byref(d), *[FAKE] * 13) == -1


def test_decode_rejects_null_and_half_carry(lib):
    d = _dims()
    for i in [0, 3, 4, 5, 6, 7, 8, 9, 10, 11]:
        args = [FAKE] * 13
        args[i] = None
        assert lib.m3_decode_step(ctypes.byref(d), *args) == -1, i
    args = [FAKE] * 13
    args[1] = None          # b_last without x_last
    assert lib.m3_decode_step(ctypes.byref(d), *args) == -1


def test_binding_raises_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(m3scan, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        m3scan.lib(str(tmp_path / "missing.so"))


def test_varlen_rejects_bad_arguments(lib):
    d = _dims()
    T = ctypes.c_int64(100)
    # no offsets, negative token count
    assert lib.m3_prefill_varlen(ctypes.byref(d), None, T, *[FAKE] * 8, None, None, FAKE, None, 0,
                                 None) == -1
    assert lib.m3_prefill_varlen(ctypes.byref(d), FAKE, ctypes.c_int64(-1), *[FAKE] * 8, None, None,
                                 FAKE, None, 0, None) == -1
    # bad dims and missing per-token inputs fail like the uniform prefill
    for kw in BAD_DIMS:
        bd = _dims(**kw)
        assert lib.m3_prefill_varlen(ctypes.byref(bd), FAKE, T, *[FAKE] * 8, None, None, FAKE, None, 0,
                                     None) == -1, kw
    for i in range(8):
        args = [FAKE] * 8
        args[i] = None
        assert lib.m3_prefill_varlen(ctypes.byref(d), FAKE, T, *args, None, None, FAKE, None, 0,
                                     None) == -1
    # workspace too small (the MFMA path needs one)
    big = _dims(headdim=64, dstate=128, rank=2, chunk=32, io_dtype=m3scan.M3_BF16)
    n = ctypes.c_size_t(0)
    assert lib.m3_prefill_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0 and n.value > 0
    assert lib.m3_prefill_varlen(ctypes.byref(big), FAKE, T, *[FAKE] * 8, None, None, FAKE, FAKE, 16,
                                 None) == -3


def _bwd(lib, d, grads, ws=None, nbytes=0, args=None, dy=FAKE, state=None):
    args = [FAKE] * 8 if args is None else args
    return lib.m3_backward(ctypes.byref(d), *args, state, dy, None,
                           None if grads is None else ctypes.byref(grads), ws, nbytes, None)


def _grads(**none):
    names = ("dx", "ddt", "dA", "dlambda", "dtheta", "dB", "dC", "dD", "dh0", "db_last", "dx_last")
    return m3scan.Grads(*[None if n in none else 0x1000 for n in names])


def test_backward_rejects_bad_arguments(lib):
    big = _dims(headdim=64, dstate=128, rank=4, io_dtype=m3scan.M3_BF16)
    n = ctypes.c_size_t(0)
    assert lib.m3_backward_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0 and n.value > 0
    # unsupported shape (N = 16, P = 16) and rank 3
    small = _dims()
    assert lib.m3_backward_workspace_size(ctypes.byref(small), ctypes.byref(n)) == -2
    assert _bwd(lib, small, _grads()) == -2
    r3 = _dims(headdim=64, dstate=128, rank=3)
    assert _bwd(lib, r3, _grads()) == -2
    # bad dims
    for kw in BAD_DIMS:
        bd = _dims(**{"headdim": 64, "dstate": 128, **kw})
        assert _bwd(lib, bd, _grads()) == -1, kw
    # missing grads struct, inputs, dy, or a required gradient
    assert _bwd(lib, big, None) == -1
    for i in range(8):
        args = [FAKE] * 8
        args[i] = None
        assert _bwd(lib, big, _grads(), args=args) == -1, i
    assert _bwd(lib, big, _grads(), dy=None) == -1
    for k in ("dx", "ddt", "dA", "dlambda", "dtheta", "dB", "dC", "dD"):
        assert _bwd(lib, big, _grads(**{k: 1})) == -1, k
    # a state without h
    st = m3scan.State(None, None, None)
    assert _bwd(lib, big, _grads(), state=ctypes.byref(st)) == -1
    # workspace too small
    assert _bwd(lib, big, _grads(), ws=FAKE, nbytes=n.value - 1) == -3
    assert _bwd(lib, big, _grads(), ws=None, nbytes=0) == -3


def test_fused_entry_points_reject_bad_arguments(lib):
    d = _dims()
    fu = m3scan.Fusion(None, None, None, None, None, None, 1e-6)
    # a NULL fusion
    assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, None, None, None, FAKE, None, 0, None) == -1
    assert lib.m3_decode_step_fused(ctypes.byref(d), *[FAKE] * 11, None, FAKE, None) == -1
    # a norm weight with a non-positive epsilon
    bad = m3scan.Fusion(None, 0x1000, None, None, None, None, 0.0)
    assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(bad), None, None, FAKE, None, 0,
                                None) == -1
    assert lib.m3_decode_step_fused(ctypes.byref(d), *[FAKE] * 11, ctypes.byref(bad), FAKE, None) == -1
    # bad dims, missing inputs: as the plain entry points
    for kw in BAD_DIMS:
        bd = _dims(**kw)
        assert lib.m3_prefill_fused(ctypes.byref(bd), *[FAKE] * 8, ctypes.byref(fu), None, None, FAKE, None, 0,
                                    None) == -1, kw
    assert lib.m3_prefill_fused(ctypes.byref(d), *([FAKE] * 7 + [None]), ctypes.byref(fu), None, None, FAKE,
                                None, 0, None) == -1
    # the workspace reserves room for the normalised carry: none given is too small
    assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(fu), None, None, FAKE, None, 0,
                                None) == -3


def test_backward_parts(lib):
    """The split of the backward is a function of the dims: none when the (b, h)
    pairs fill the CUs or the sequence is a single segment, otherwise pieces of
    whole 3-token segments that cover the sequence, every piece non-empty; the
    workspace grows by the pieces' states."""
    P, N = 64, 128
    nb = ctypes.c_size_t(0)
    # 256 (b, h) pairs: no split
    d = _dims(batch=8, nheads=32, ngroups=8, headdim=P, dstate=N, rank=1, seqlen=40)
    assert m3scan.backward_parts(d) == (1, 40)
    # a single segment
    for L in (0, 1, 3):
        assert m3scan.backward_parts(_dims(batch=1, nheads=2, headdim=P, dstate=N, seqlen=L)) == (1, L)
    # few pairs: split
    for b, H, L in [(4, 24, 2048), (2, 64, 16384), (4, 24, 200), (2, 4, 37), (1, 1, 100000)]:
        d = _dims(batch=b, nheads=H, ngroups=1, headdim=P, dstate=N, rank=2, seqlen=L)
        parts, tpp = m3scan.backward_parts(d)
        assert parts > 1 and tpp % 3 == 0, (b, H, L)
        assert (parts - 1) * tpp < L <= parts * tpp, (b, H, L, parts, tpp)
        assert lib.m3_backward_workspace_size(ctypes.byref(d), ctypes.byref(nb)) == 0
        assert nb.value >= 2 * b * H * parts * N * P * 4
    n32, n64 = ctypes.c_int32(0), ctypes.c_int64(0)
    good = _dims(headdim=P, dstate=N)
    assert lib.m3_backward_parts(ctypes.byref(good), None, ctypes.byref(n64)) == -1
    assert lib.m3_backward_parts(ctypes.byref(good), ctypes.byref(n32), None) == -1
    assert lib.m3_backward_parts(ctypes.byref(_dims(batch=0, headdim=P, dstate=N)), ctypes.byref(n32),
                                 ctypes.byref(n64)) == -1
    assert lib.m3_backward_parts(ctypes.byref(_dims()), ctypes.byref(n32), ctypes.byref(n64)) == -2


def test_launch_size_limits(lib):
    """Shapes whose launches would exceed 2^32 work-items are refused before anything
    is launched (M3_ERR_UNSUPPORTED), and a batch too large for the matrix-core
    prefill's grid falls back to the generic path while that one fits."""
    P, N = 64, 128
    n = ctypes.c_size_t(0)
    # decode: one workgroup per (b, h)
    d = _dims(batch=1 << 18, nheads=64, ngroups=1, headdim=P, dstate=N, rank=4, io_dtype=m3scan.M3_BF16)
    args = [FAKE] * 12
    assert lib.m3_decode_step(ctypes.byref(d), *args, None) == -2
    # prefill: 2^24 (b, h) pairs fit neither path
    assert lib.m3_prefill_workspace_size(ctypes.byref(_dims(batch=1 << 18, nheads=64, ngroups=1, headdim=P,
                                                            dstate=N, rank=1, chunk=64, seqlen=64,
                                                            io_dtype=m3scan.M3_BF16)), ctypes.byref(n)) == -2
    # 70000 sequences of one head: past the matrix-core grid, still the generic path
    small = _dims(batch=70000, nheads=1, ngroups=1, headdim=P, dstate=N, rank=1, chunk=64, seqlen=64,
                  io_dtype=m3scan.M3_BF16)
    assert lib.m3_prefill_workspace_size(ctypes.byref(small), ctypes.byref(n)) == 0
    # backward: one workgroup per (b, h, piece)
    bd = _dims(batch=1 << 17, nheads=64, ngroups=1, headdim=P, dstate=N, rank=1, seqlen=3)
    assert _bwd(lib, bd, _grads(), ws=FAKE, nbytes=1 << 62) == -2


def test_backward_varlen_rejects_bad_arguments(lib):
    """Packed-batch backward: a NULL cu_seqlens, a negative token count or more tokens than
    batch * seqlen (the workspace's per-token room) are argument errors; everything else is
    checked as for m3_backward.  No call here reaches a launch."""
    d = _dims(batch=3, seqlen=10, nheads=4, ngroups=2, headdim=64, dstate=128, rank=2, io_dtype=m3scan.M3_BF16)
    def call(cu=FAKE, T=20, grads=None, args=None, dy=FAKE):
        args = [FAKE] * 8 if args is None else args
        g = _grads() if grads is None else grads
        return lib.m3_backward_varlen(ctypes.byref(d), cu, T, *args, None, dy, None, ctypes.byref(g),
                                      None, 0, None)
    assert call(cu=None) == -1
    assert call(T=-1) == -1
    assert call(T=31) == -1                   # 3 sequences of at most 10 tokens
    assert call(dy=None) == -1
    assert call(grads=_grads(dx=1)) == -1
    args = [FAKE] * 8
    args[5] = None                            # B
    assert call(args=args) == -1
    assert call(T=30) == -3                   # valid: the missing workspace is the only error
    small = _dims(batch=3, seqlen=10)         # N = 16, P = 16: no backward kernel
    assert lib.m3_backward_varlen(ctypes.byref(small), FAKE, 20, *([FAKE] * 8), None, FAKE, None,
                                  ctypes.byref(_grads()), None, 0, None) == -2


def test_backward_per_token_A_rejects_bad_arguments(lib):
    """Backward with a per-token decay rate: a NULL A_t is an argument error; without
    cu_seqlens the token count is ignored, with it the packed-batch bounds apply.  No call
    here reaches a launch."""
    d = _dims(batch=3, seqlen=10, nheads=4, ngroups=2, headdim=64, dstate=128, rank=2, io_dtype=m3scan.M3_BF16)
    def call(cu=FAKE, T=20, args=None):
        args = [FAKE] * 8 if args is None else args
        return lib.m3_backward_per_token_A(ctypes.byref(d), cu, T, *args, None, FAKE, None,
                                           ctypes.byref(_grads()), None, 0, None)
    args = [FAKE] * 8
    args[2] = None                            # A_t
    assert call(args=args) == -1
    assert call(cu=None, args=args) == -1
    assert call(T=-1) == -1
    assert call(T=31) == -1
    assert call(cu=None, T=-1) == -3          # T unused without cu_seqlens: only the workspace is missing
    assert call(T=30) == -3
