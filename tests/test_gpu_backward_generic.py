"""GPU parity of the backward pass at shapes off the fast kernel's N = 128, P = 64 (the
generic token-serial kernel, m3_backward_generic.hip), through the C ABI, against the
oracle's adjoint loop (oracle.scan_backward, pinned by finite differences of the forward
oracle), gradient by gradient: the small fp32 SISO layer's shape (N = P = 16, L = 256),
odd and uneven dims (N = 24, P = 12), the smallest state (N = 2), the largest state rows
and columns the kernel takes (N = 256; P = 256), rank up to 8, groups shared by several
heads and one head per group, fp32 and bf16 io, a state and carry passed in, a final-state
cotangent, a single token and none; packed variable-length batches (per sequence), a
per-token decay rate, and the checkpoint budget (bit-identical gradients for any segment
length), with the reverse sweep's sums taken in batches of 1 to 16 tokens (full and ragged).
Bar: 1e-3 max relative error per gradient tensor, as for the fast kernel."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import draw, np64, say
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-3
NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")


def _rel(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30))


def _inputs(b, L, H, G, P, N, R, io, seed, with_state, with_dh):
    d = draw(b, L, H, G, P, N, R, io, 2.0, seed=seed)
    gen = torch.Generator(device="cpu").manual_seed(seed + 1)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    dy = torch.randn((b, L, H, R, P), generator=gen).to(tdt).cuda()
    dh = torch.randn((b, H, N, P), generator=gen).cuda() if with_dh else None
    st = None
    if with_state:
        st = m3scan.DecodeState(torch.randn((b, H, N, P), generator=gen).cuda(),
                                torch.randn((b, G, R, N), generator=gen).to(tdt).cuda(),
                                torch.randn((b, H, R, P), generator=gen).to(tdt).cuda())
    return d, dy, dh, st


def _state_np(st):
    return None if st is None else (np64(st.h), np64(st.b_last), np64(st.x_last))


# b, L, H, G, P, N, R, io, with state_in, with dh_out
CASES = [
    (1, 256, 4, 1, 16, 16, 1, "fp32", False, True),    # the small fp32 SISO layer's shape
    (2, 37, 4, 2, 12, 24, 3, "fp32", True, True),
    (1, 50, 2, 2, 32, 64, 8, "bf16", True, False),
    (2, 33, 2, 1, 128, 64, 2, "bf16", False, True),    # 4096 element pairs: 16 per thread; 8-token blocks
    (1, 21, 2, 1, 128, 64, 8, "fp32", True, True),     # 2-token blocks (LDS)
    (1, 1, 2, 1, 8, 4, 1, "fp32", True, True),
    (1, 100, 2, 1, 4, 2, 5, "fp32", False, False),     # N = 2: one rotation pair
    (1, 40, 2, 1, 256, 32, 1, "bf16", True, True),     # P = 256
    (1, 45, 3, 3, 16, 256, 2, "fp32", True, True),     # N = 256
    (2, 45, 2, 1, 64, 32, 2, "fp32", True, True),      # 16-token blocks, sums in batches of 4 (ragged: 13 = 4+4+4+1)
]


def _id(c):
    return "b{}L{}H{}G{}P{}N{}R{}-{}{}{}".format(*c[:8], "-state" if c[8] else "", "-dh" if c[9] else "")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_generic_backward_matches_oracle(case):
    b, L, H, G, P, N, R, io, ws, wd = case
    say("generic backward", _id(case))
    d, dy, dh, st = _inputs(b, L, H, G, P, N, R, io, L * 3 + N + R, ws, wd)
    gr = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    ref = oracle.scan_backward(*[np64(d[k]) for k in NAMES], np64(dy),
                               dh_out=None if dh is None else np64(dh), state_in=_state_np(st))
    errs = {k: _rel(np64(gr[k]), ref[k]) for k in ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0")}
    if ws:
        errs["db_last"] = _rel(np64(gr["db_last"]), ref["db_last"])
        errs["dx_last"] = _rel(np64(gr["dx_last"]), ref["dx_last"])
    else:
        assert float(gr["db_last"].abs().max()) == 0.0 and float(gr["dx_last"].abs().max()) == 0.0
    say("  " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL_BWD}
    assert not bad, bad


def test_generic_backward_empty_sequence():
    """L = 0: the final-state cotangent passes to h_0; every other gradient is zero."""
    b, H, G, P, N, R = 1, 2, 1, 16, 16, 1
    d = draw(b, 1, H, G, P, N, R, "fp32", 1.0, seed=3)
    d = {k: (v[:, :0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    dy = torch.zeros((b, 0, H, R, P), device="cuda")
    dh = torch.randn((b, H, N, P), device="cuda")
    gr = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=m3scan.DecodeState(torch.randn((b, H, N, P), device="cuda")))
    torch.cuda.synchronize()
    assert torch.equal(gr["dh0"], dh)
    assert float(gr["dA"].abs().max()) == 0.0 and float(gr["dD"].abs().max()) == 0.0


def test_generic_backward_is_deterministic_and_budget_independent():
    """Two calls give the same bits, and so do 16-token segments and segments of about
    sqrt(L) tokens, forced by smaller checkpoint budgets, against every state kept (the
    default here): the recomputed states come from the same steps.  A workspace of exactly
    the smaller size is passed each time, so the call must pick that level to fit it."""
    b, L, H, G, P, N, R = 2, 1000, 2, 1, 16, 32, 2   # every state: 1010 states; 16-token segments: 80; 32: 65
    d, dy, dh, st = _inputs(b, L, H, G, P, N, R, "fp32", 61, True, True)
    dims = m3scan.make_dims(b, L, H, G, P, N, R, 1, 0)
    w16 = m3scan.backward_workspace_size(dims)
    g1 = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st)
    g2 = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st)
    wseg = m3scan.backward_workspace_size(dims, 4 << 20)
    g4 = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st,
                         workspace=torch.empty(wseg, dtype=torch.uint8, device="cuda"))
    wsq = m3scan.backward_workspace_size(dims, 1)
    g3 = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st, checkpoint_bytes=1)
    torch.cuda.synchronize()
    say(f"generic backward workspace: {w16} bytes (every state), {wseg} (16-token segments), {wsq} (sqrt(L))")
    assert wsq < wseg < w16
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
        assert torch.equal(g1[k], g3[k]), k
        assert torch.equal(g1[k], g4[k]), k


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_generic_backward_varlen_each_sequence_matches_oracle(io):
    """A packed batch (an empty and a one-token sequence among them), each sequence against
    the oracle's adjoint on it alone, with its own state, carry and final cotangent."""
    lengths, H, G, P, N, R = [70, 0, 1, 130, 25], 4, 2, 12, 24, 2
    T, ns, Lmax = sum(lengths), len(lengths), max(lengths)
    d = draw(1, T, H, G, P, N, R, io, 2.0, seed=17)
    d = {k: (v[0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    gen = torch.Generator(device="cpu").manual_seed(5)
    dy = torch.randn((T, H, R, P), generator=gen).to(tdt).cuda()
    dh = torch.randn((ns, H, N, P), generator=gen).cuda()
    st = m3scan.DecodeState(torch.randn((ns, H, N, P), generator=gen).cuda(),
                            torch.randn((ns, G, R, N), generator=gen).to(tdt).cuda(),
                            torch.randn((ns, H, R, P), generator=gen).to(tdt).cuda())
    gr = m3scan.backward_varlen(*[d[k] for k in NAMES], dy, cu, Lmax, dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    dA, dD = np.zeros(H), np.zeros(H)
    for s, n in enumerate(lengths):
        if n == 0:
            assert np.array_equal(np64(gr["dh0"][s]), np64(dh[s]))
            assert float(gr["db_last"][s].abs().max()) == 0.0 and float(gr["dx_last"][s].abs().max()) == 0.0
            continue
        sl = lambda k: np64(d[k][c[s]:c[s + 1]])[None]
        ref = oracle.scan_backward(sl("x"), sl("dt"), np64(d["A"]), sl("lam"), sl("theta"), sl("B"), sl("C"),
                                   np64(d["D"]), np64(dy[c[s]:c[s + 1]])[None], dh_out=np64(dh[s:s + 1]),
                                   state_in=(np64(st.h[s:s + 1]), np64(st.b_last[s:s + 1]), np64(st.x_last[s:s + 1])))
        errs = {k: _rel(np64(gr[k][c[s]:c[s + 1]])[None], ref[k]) for k in ("dx", "ddt", "dlam", "dtheta", "dB", "dC")}
        for k in ("dh0", "db_last", "dx_last"):
            errs[k] = _rel(np64(gr[k][s:s + 1]), ref[k])
        dA += ref["dA"]
        dD += ref["dD"]
        say(f"  seq {s} (len {n}): " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
        bad = {k: v for k, v in errs.items() if not v <= TOL_BWD}
        assert not bad, (s, bad)
    assert _rel(np64(gr["dA"]), dA) <= TOL_BWD and _rel(np64(gr["dD"]), dD) <= TOL_BWD


def test_generic_backward_per_token_A():
    """m3_backward_per_token_A at a generic shape: dA per token against the oracle with the
    same per-token rates."""
    b, L, H, G, P, N, R = 2, 60, 3, 1, 16, 16, 2
    d, dy, dh, st = _inputs(b, L, H, G, P, N, R, "fp32", 29, True, True)
    A_t = (-torch.rand((b, L, H), generator=torch.Generator().manual_seed(7)) * 2).cuda()
    args = [d[k] for k in NAMES]
    args[2] = A_t
    gr = m3scan.backward_per_token_A(*args, dy, dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    ref_args = [np64(d[k]) for k in NAMES]
    ref_args[2] = np64(A_t)
    ref = oracle.scan_backward(*ref_args, np64(dy), dh_out=np64(dh), state_in=_state_np(st))
    errs = {k: _rel(np64(gr[k]), ref[k]) for k in ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0",
                                                   "db_last", "dx_last")}
    say("generic backward, per-token A: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL_BWD}
    assert not bad, bad
