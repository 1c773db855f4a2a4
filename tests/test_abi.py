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
                                  "m3_backward_workspace_size", "m3_backward_workspace_size_budget", "m3_decode_step",
                                  "m3_decode_step_fused", "m3_prefill_chunked", "m3_prefill_chunked_noalloc", "m3_prefill_fused",
                                  "m3_prefill_fused_workspace_size", "m3_prefill_sequences_per_workgroup",
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
    s = ctypes.c_int32(0)
    assert lib.m3_prefill_sequences_per_workgroup(ctypes.byref(d), ctypes.byref(s)) == -2
    # a state too large for LDS whatever the block size
    d = _dims(rank=1, dstate=512, headdim=512, chunk=1)
    assert lib.m3_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == -2


@pytest.mark.parametrize("R,Q", [(4, 64), (2, 64), (4, 128)])
def test_fp32_chunks_larger_than_lds_are_split(lib, R, Q):
    """fp32 io at the 1.5B head shape (N=128, P=64): chunks whose arrays exceed LDS run as
    smaller blocks instead of being refused (the chunked result does not depend on the block
    size beyond rounding); no workspace is asked for, except by a fused call with a B norm
    or bias, which normalises the carried B into it."""
    d = m3scan.make_dims(2, 300, 4, 1, 64, 128, R, Q, m3scan.M3_F32)
    n = ctypes.c_size_t(1)
    assert lib.m3_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 0
    fu = m3scan.Fusion(None, 0x1000, None, None, None, None, 1e-6, None, 0)   # a B norm weight
    assert lib.m3_prefill_fused_workspace_size(ctypes.byref(d), ctypes.byref(fu), ctypes.byref(n)) == 0
    assert n.value == 2 * 1 * R * 128 * 4   # batch x G x R x N fp32: the normalised carried B


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
    # shapes no backward kernel takes: P above 256, rank 9, N / 2 * P above 4096 off the
    # fast kernel's shape
    for kw in (dict(headdim=300), dict(rank=9), dict(headdim=64, dstate=256)):
        un = _dims(**kw)
        assert lib.m3_backward_workspace_size(ctypes.byref(un), ctypes.byref(n)) == -2, kw
        assert _bwd(lib, un, _grads()) == -2, kw
    # the generic kernel's shapes (N = P = 16; rank 3 at N = 128, P = 64): valid calls whose
    # only error is the missing workspace
    for kw in (dict(), dict(headdim=64, dstate=128, rank=3)):
        gen = _dims(**kw)
        assert lib.m3_backward_workspace_size(ctypes.byref(gen), ctypes.byref(n)) == 0 and n.value > 0, kw
        assert _bwd(lib, gen, _grads()) == -3, kw
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
    fu = m3scan.Fusion(None, None, None, None, None, None, 1e-6, None, 0)
    # a NULL fusion
    assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, None, None, None, FAKE, None, 0, None) == -1
    assert lib.m3_decode_step_fused(ctypes.byref(d), *[FAKE] * 11, None, FAKE, None) == -1
    # a norm weight with a non-positive epsilon
    bad = m3scan.Fusion(None, 0x1000, None, None, None, None, 0.0, None, 0)
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
    # with a norm weight the workspace reserves room for the normalised carry: none given is
    # too small
    fn = m3scan.Fusion(None, 0x1000, None, None, None, None, 1e-6, None, 0)
    assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(fn), None, None, FAKE, None, 0,
                                None) == -3
    # an output-norm weight with a non-positive epsilon
    bad = m3scan.Fusion(None, None, None, None, None, None, 0.0, 0x1000, 0)
    assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(bad), None, None, FAKE, None, 0,
                                None) == -1
    assert lib.m3_decode_step_fused(ctypes.byref(d), *[FAKE] * 11, ctypes.byref(bad), FAKE, None) == -1
    # angle groups must be a multiple of G (2 here) dividing H (4): 1, 3, 8 and -2 are refused
    for gt in (1, 3, 8, -2):
        bad = m3scan.Fusion(None, None, None, None, None, None, 1e-6, None, gt)
        assert lib.m3_prefill_fused(ctypes.byref(d), *[FAKE] * 8, ctypes.byref(bad), None, None, FAKE, None, 0,
                                    None) == -1, gt
        assert lib.m3_decode_step_fused(ctypes.byref(d), *[FAKE] * 11, ctypes.byref(bad), FAKE, None) == -1, gt
        n = ctypes.c_size_t(0)
        assert lib.m3_prefill_fused_workspace_size(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(n)) == -1, gt


def test_fused_workspace_grows_with_angle_groups(lib):
    """Angles per head over shared B and C prepare the rotated operands per angle group:
    the matrix-core path's workspace holds Gt / G times the per-group share; 0 or G angle
    groups give the plain size."""
    d = m3scan.make_dims(2, 640, 8, 2, 64, 128, 2, 32, m3scan.M3_BF16)
    n0, n2, n8 = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    for gt, n in ((0, n0), (2, n2), (8, n8)):
        fu = m3scan.Fusion(None, None, None, None, None, None, 1e-6, None, gt)
        assert lib.m3_prefill_fused_workspace_size(ctypes.byref(d), ctypes.byref(fu), ctypes.byref(n)) == 0
    assert n0.value == n2.value == m3scan.workspace_size(d)
    assert n8.value > n0.value


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
    assert lib.m3_backward_parts(ctypes.byref(_dims(headdim=300)), ctypes.byref(n32), ctypes.byref(n64)) == -2
    # the generic kernel (off the fast shape) never splits
    for L in (0, 5, 5000):
        assert m3scan.backward_parts(_dims(batch=1, nheads=2, seqlen=L)) == (1, L)


def test_prefill_sequences_per_workgroup(lib):
    """The matrix-core prefill sweeps several sequences per workgroup only for equal-length
    batches of one to four whole chunks, at 64 or 256 rows per chunk, whose (b, h) pairs fill
    at least eight rounds of workgroups (two sequences each, four rounds), about 16 chunks
    per workgroup, never more than the batch; everything else runs one sequence per
    workgroup."""
    def seqs(**kw):
        base = dict(batch=4096, seqlen=64, nheads=64, ngroups=1, headdim=64, dstate=128, rank=4, chunk=64,
                    io_dtype=m3scan.M3_BF16)
        base.update(kw)
        return m3scan.prefill_sequences_per_workgroup(m3scan.Dims(**base))
    assert seqs() == 16                                   # one chunk each: 16 per workgroup
    assert seqs(seqlen=128) == 8 and seqs(seqlen=256) == 4
    assert seqs(seqlen=320) == 1                          # five chunks
    assert seqs(seqlen=100) == 1                          # a partial chunk
    assert seqs(batch=32) == 2                            # 2048 pairs at one workgroup per CU: 8 rounds
    assert seqs(batch=31) == 1
    assert seqs(rank=1, batch=64) == 2                    # two workgroups per CU at 64 rows: 512 slots
    assert seqs(rank=1, batch=63) == 1
    assert seqs(ngroups=8) == 16                          # groups of heads sharing B and C
    assert seqs(chunk=32) == 1 and seqs(rank=2) == 1      # 128-row chunks: two workgroups per CU already
    assert seqs(rank=2, chunk=32, batch=128) == 4 and seqs(rank=1, chunk=32) == 8   # two chunks each
    assert seqs(headdim=16, dstate=16, io_dtype=m3scan.M3_F32) == 1   # not the matrix-core path
    n = ctypes.c_int32(0)
    good = _dims()
    assert lib.m3_prefill_sequences_per_workgroup(ctypes.byref(good), None) == -1
    assert lib.m3_prefill_sequences_per_workgroup(ctypes.byref(_dims(batch=0)), ctypes.byref(n)) == -1


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
    un = _dims(batch=3, seqlen=10, headdim=300)   # P above 256: no backward kernel
    assert lib.m3_backward_varlen(ctypes.byref(un), FAKE, 20, *([FAKE] * 8), None, FAKE, None,
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


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    """m3_prefill_chunked_noalloc checks the workspace its plan needs against its static
    array before any HIP call: the batch-256 MIMO layer needs about 514 MiB and is refused
    with M3_ERR_WORKSPACE; bad dims give M3_ERR_INVALID_ARG."""
    null8 = [None] * 8
    big = m3scan.make_dims(256, 1024, 64, 1, 64, 128, 4, 64, m3scan.M3_BF16)
    assert m3scan.workspace_size(big) > m3scan.NOALLOC_SCRATCH_BYTES
    assert lib.m3_prefill_chunked_noalloc(ctypes.byref(big), *null8, None, None, None, None) == -3
    bad = _dims(ngroups=3)
    assert lib.m3_prefill_chunked_noalloc(ctypes.byref(bad), *null8, None, None, None, None) == -1
    assert lib.m3_prefill_chunked_noalloc(None, *null8, None, None, None, None) == -1


def _bwd_ws(lib, d, budget=None):
    n = ctypes.c_size_t(0)
    if budget is None:
        assert lib.m3_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    else:
        assert lib.m3_backward_workspace_size_budget(ctypes.byref(d), ctypes.c_size_t(budget), ctypes.byref(n)) == 0
    return n.value


def test_backward_checkpoint_budget(lib):
    """Checkpoints stay one per 3-token segment while they fit the budget (4 GiB by default,
    else the one passed to m3_backward_workspace_size_budget); above it the workspace holds
    about 2 sqrt(L/3) states per (b, h) instead of L/3 -- checked against the sizes that
    layout implies."""
    P, N, state = 64, 128, 64 * 128 * 4
    # nanomamba3-shaped: 2.15 GB of checkpoints, under the budget: one level
    d = _dims(batch=4, nheads=24, ngroups=1, headdim=P, dstate=N, rank=2, seqlen=2048)
    parts, tpp = m3scan.backward_parts(d)
    one = _bwd_ws(lib, d)
    assert one >= 4 * 24 * parts * (tpp // 3) * state
    assert _bwd_ws(lib, d, 4 << 30) == one
    # a budget below that: groups of ceil(sqrt(segments per piece)) segments
    two = _bwd_ws(lib, d, 1 << 20)
    segs = tpp // 3
    g = -(-segs // 1)
    import math
    g = math.ceil(math.sqrt(segs))
    ck_one = 4 * 24 * parts * segs * state
    ck_two = 4 * 24 * parts * (-(-segs // g) + g) * state
    assert one - two == ck_one - ck_two, (one, two, ck_one, ck_two)
    # the 1.5B SISO layer (44.8 GB of one-level checkpoints) is grouped by default
    d = _dims(batch=8, nheads=64, ngroups=1, headdim=P, dstate=N, rank=1, seqlen=8192)
    assert m3scan.backward_parts(d) == (1, 8192)
    segs = -(-8192 // 3)
    g = math.ceil(math.sqrt(segs))
    ws = _bwd_ws(lib, d)
    partials = 8 * 8192 * 64 * (2 * 1 * N + N // 2) * 4 + 8 * 64 * 1 * N * 4
    assert ws < 8 * 64 * segs * state
    assert ws >= 8 * 64 * (-(-segs // g) + g) * state + partials
    # a budget above it restores one level
    assert _bwd_ws(lib, d, 64 << 30) >= 8 * 64 * segs * state


def test_serial_prefill_needs_no_workspace(lib):
    """Small states are scanned token by token: no workspace (the chunked paths need one
    only for their prepared operands and segment states)."""
    n = ctypes.c_size_t(1)
    for N, P, R, io in [(16, 16, 1, m3scan.M3_F32), (2, 4, 6, m3scan.M3_F32), (32, 16, 4, m3scan.M3_BF16),
                        (128, 2, 8, m3scan.M3_F32)]:
        d = m3scan.make_dims(2, 300, 4, 2, P, N, R, 32, io)
        assert lib.m3_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
        assert n.value == 0, (N, P, R)


@pytest.mark.parametrize("shape", [dict(headdim=64, dstate=128, rank=2), dict(headdim=12, dstate=24, rank=3)],
                         ids=["fast", "generic"])
def test_backward_workspace_below_every_level_is_refused(lib, shape):
    """The backward keeps states at the first level whose workspace fits the bytes passed;
    below the smallest level (the size a budget of one byte asks for) it returns
    M3_ERR_WORKSPACE before any launch, and the budgeted sizes shrink with the budget."""
    d = _dims(batch=2, seqlen=1000, nheads=4, ngroups=1, io_dtype=m3scan.M3_BF16, **shape)
    smallest = _bwd_ws(lib, d, 1)
    assert 0 < smallest <= _bwd_ws(lib, d, 1 << 20) <= _bwd_ws(lib, d) <= _bwd_ws(lib, d, 1 << 62)
    assert _bwd(lib, d, _grads(), ws=FAKE, nbytes=smallest - 1) == -3
    assert _bwd(lib, d, _grads(), ws=None, nbytes=smallest) == -3
    n = ctypes.c_size_t(0)
    assert lib.m3_backward_workspace_size_budget(ctypes.byref(d), 1, None) == -1
    assert lib.m3_backward_workspace_size_budget(None, 1, ctypes.byref(n)) == -1
    un = _dims(batch=2, seqlen=10, headdim=300)
    assert lib.m3_backward_workspace_size_budget(ctypes.byref(un), 1, ctypes.byref(n)) == -2


def test_generic_backward_workspace(lib):
    """Off the fast kernel's shape the backward keeps every state of the sequence (one
    segment: L rounded up to 16, plus 2 states per (b, h)) while those fit the checkpoint
    budget; else the state before every 16-token segment plus one segment's 17 states; else
    segments of ceil(sqrt(L)) tokens rounded up to a multiple of 16 (fewer bytes each time,
    the same gradients); per-head copies of the group-shared gradients are added when H > G."""
    import math
    b, H, N, P, R, L = 2, 4, 24, 12, 3, 1000
    state = N * P * 4
    slack = 4 * 256 + 2 * b * H * 4 + 1024
    d1 = _dims(batch=b, nheads=H, ngroups=H, headdim=P, dstate=N, rank=R, seqlen=L)
    wall = _bwd_ws(lib, d1)
    keep = 16 * math.ceil(L / 16) + 2
    assert b * H * keep * state <= wall < b * H * keep * state + slack
    # below every state, above 16-token segments
    w16 = _bwd_ws(lib, d1, 2 << 20)
    seg16 = math.ceil(L / 16) + 17
    assert b * H * seg16 * state <= w16 < b * H * seg16 * state + slack
    ks = 16 * math.ceil(math.ceil(math.sqrt(L)) / 16)
    wsq = _bwd_ws(lib, d1, 1)
    assert wsq >= b * H * (math.ceil(L / ks) + ks + 1) * state and wsq < w16 < wall
    d2 = _dims(batch=b, nheads=H, ngroups=1, headdim=P, dstate=N, rank=R, seqlen=L)
    per_head = b * L * H * (2 * R * N + N // 2) * 4 + b * H * R * N * 4
    assert _bwd_ws(lib, d2) >= wall + per_head


def test_binding_backward_workspace_choice(lib):
    """The binding's backward workspace (host-side marshalling, CPU tensors here): a new one
    of the size the budget asks for; a caller's larger one whole (the call then keeps as many
    states as it holds); a caller's smaller one replaced."""
    import torch
    d = _dims(batch=2, seqlen=1000, nheads=4, ngroups=1, headdim=12, dstate=24, rank=3)
    need = m3scan.backward_workspace_size(d, 1)
    n, ws = m3scan._backward_workspace(d, None, "cpu", 1)
    assert n == need and ws.numel() == need and ws.dtype == torch.uint8
    big = torch.empty(need * 3, dtype=torch.uint8)
    n, ws = m3scan._backward_workspace(d, big, "cpu", 1)
    assert n == need * 3 and ws is big
    small = torch.empty(need - 1, dtype=torch.uint8)
    n, ws = m3scan._backward_workspace(d, small, "cpu", 1)
    assert n == need and ws is not small and ws.numel() == need
    assert m3scan.backward_workspace_size(d) == m3scan.backward_workspace_size(d, 4 << 30)
