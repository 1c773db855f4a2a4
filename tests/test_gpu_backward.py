"""GPU parity of the backward pass (m3_backward through the C ABI) against the
oracle's adjoint loop (oracle.scan_backward, pinned by finite differences of the
forward oracle), gradient by gradient: every input, the initial state, the
carried previous input, with and without a final-state cotangent; fp32 and bf16
io; ranks 1, 2 and 4; groups shared by several heads (per-head partials summed
by the second kernel) and one head per group (written directly); sequence
lengths that leave a partial recompute segment, a single token and none.

Bar: fp32 arithmetic throughout, so a max relative error per gradient tensor
(max|gpu-ref| / max|ref|) of 1e-3: the longest sums are dA and dD over
L * N * P terms, whose fp32 rounding grows like 2^-24 * sqrt(L * N * P) ~ 2e-4
at the largest size here."""
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


def _run_case(b, L, H, G, R, io, seed, with_state=False, with_dh=False, N=128, P=64):
    d = draw(b, L, H, G, P, N, R, io, 2.0, seed=seed)
    gen = torch.Generator(device="cpu").manual_seed(seed + 1)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    dy = torch.randn((b, L, H, R, P), generator=gen).to(tdt).cuda()
    dh = torch.randn((b, H, N, P), generator=gen).cuda() if with_dh else None
    st = None
    st_np = None
    if with_state:
        h0 = torch.randn((b, H, N, P), generator=gen).cuda()
        bl = torch.randn((b, G, R, N), generator=gen).to(tdt).cuda()
        xl = torch.randn((b, H, R, P), generator=gen).to(tdt).cuda()
        st = m3scan.DecodeState(h0, bl, xl)
        st_np = (np64(h0), np64(bl), np64(xl))
    gr = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    ref = oracle.scan_backward(*[np64(d[k]) for k in NAMES], np64(dy),
                               dh_out=None if dh is None else np64(dh), state_in=st_np)
    errs = {}
    for k in ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0"):
        errs[k] = _rel(np64(gr[k]), ref[k])
    if with_state:
        errs["db_last"] = _rel(np64(gr["db_last"]), ref["db_last"])
        errs["dx_last"] = _rel(np64(gr["dx_last"]), ref["dx_last"])
    else:
        assert float(gr["db_last"].abs().max()) == 0.0 and float(gr["dx_last"].abs().max()) == 0.0
    return errs


CASES = [
    # b, L, H, G, R, io, state, dh
    (2, 37, 4, 2, 4, "bf16", True, True),
    (1, 20, 2, 2, 2, "fp32", False, False),
    (2, 9, 2, 1, 1, "bf16", True, False),
    (1, 64, 4, 1, 4, "fp32", False, True),
    (1, 3, 2, 2, 4, "bf16", True, True),
    (1, 1, 2, 1, 2, "bf16", True, True),
    # split sequences (m3_backward_parts > 1): pieces of two segments, the last one a
    # single 2-token segment; and a split with a carried state and final cotangent
    (4, 200, 24, 1, 2, "bf16", False, True),
    (2, 150, 4, 2, 4, "fp32", True, True),
    # 256 (b, h) pairs: no split
    (8, 40, 32, 8, 1, "bf16", True, False),
]


def _id(c):
    return "b{}L{}H{}G{}R{}-{}{}{}".format(*c[:6], "-state" if c[6] else "", "-dh" if c[7] else "")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_matches_oracle(case):
    b, L, H, G, R, io, ws, wd = case
    say("backward", _id(case), "pieces", m3scan.backward_parts(m3scan.make_dims(b, L, H, G, 64, 128, R, 1, 0)))
    errs = _run_case(b, L, H, G, R, io, seed=L * 7 + R, with_state=ws, with_dh=wd)
    say("  " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL_BWD}
    assert not bad, bad


def test_backward_empty_sequence():
    """L = 0: the final-state cotangent passes to h_0; every other gradient is zero."""
    b, H, G, R, N, P = 1, 2, 1, 2, 128, 64
    d = draw(b, 1, H, G, P, N, R, "bf16", 1.0, seed=3)
    d = {k: (v[:, :0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    dy = torch.zeros((b, 0, H, R, P), dtype=torch.bfloat16, device="cuda")
    dh = torch.randn((b, H, N, P), device="cuda")
    h0 = torch.randn((b, H, N, P), device="cuda")
    gr = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=m3scan.DecodeState(h0))
    torch.cuda.synchronize()
    assert torch.equal(gr["dh0"], dh)
    assert float(gr["dA"].abs().max()) == 0.0 and float(gr["dD"].abs().max()) == 0.0


def test_backward_is_deterministic():
    """No atomics: two calls give bit-identical gradients."""
    b, L, H, G, R = 1, 30, 4, 1, 4
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=8)
    dy = torch.randn((b, L, H, R, 64), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).cuda()
    g1 = m3scan.backward(*[d[k] for k in NAMES], dy)
    g2 = m3scan.backward(*[d[k] for k in NAMES], dy)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_cases_cover_split_and_whole_sequences():
    """The cases above run both the split path (several pieces, some of several
    segments) and the whole-sequence path beyond a single segment."""
    plans = [(c, m3scan.backward_parts(m3scan.make_dims(c[0], c[1], c[2], c[3], 64, 128, c[4], 1, 0)))
             for c in CASES]
    assert any(p > 1 and t > 3 for _, (p, t) in plans)
    assert any(p > 1 and c[6] for c, (p, t) in plans)
    assert any(p == 1 and c[1] > 3 for c, (p, t) in plans)


def _grads(d, dy, dh=None, st=None, checkpoint_bytes=None):
    g = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st, checkpoint_bytes=checkpoint_bytes)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", [
    (4, 1200, 24, 1, 2, "bf16", False, True),   # 8 pieces of 150 tokens: groups of 8 segments, the last of 2
    (2, 900, 4, 2, 4, "fp32", True, True),      # 30 pieces, carried state, final cotangent: groups of 4, the last of 2
    (8, 40, 32, 8, 1, "bf16", True, False),     # whole sequences: groups of 4 segments, the last of 2
    (2, 500, 4, 2, 2, "fp32", True, True),      # 28 pieces: groups of 3 segments
], ids=_id)
def test_checkpoint_groups_give_the_same_bits(case):
    """With a checkpoint budget too small for one state per segment, the states inside each
    group of segments are recomputed from the group's checkpoint: the same forward steps in
    the same order, so every gradient is bit-identical to the one-level run."""
    b, L, H, G, R, io, ws, wd = case
    d = draw(b, L, H, G, 64, 128, R, io, 2.0, seed=L + 5)
    gen = torch.Generator(device="cpu").manual_seed(L)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    dy = torch.randn((b, L, H, R, 64), generator=gen).to(tdt).cuda()
    dh = torch.randn((b, H, 128, 64), generator=gen).cuda() if wd else None
    st = None
    if ws:
        st = m3scan.DecodeState(torch.randn((b, H, 128, 64), generator=gen).cuda(),
                                torch.randn((b, G, R, 128), generator=gen).to(tdt).cuda(),
                                torch.randn((b, H, R, 64), generator=gen).to(tdt).cuda())
    dims = m3scan.make_dims(b, L, H, G, 64, 128, R, 1, 0)
    ws1 = m3scan.backward_workspace_size(dims)
    g1 = _grads(d, dy, dh, st)
    ws2 = m3scan.backward_workspace_size(dims, 1)
    g2 = _grads(d, dy, dh, st, checkpoint_bytes=1)
    parts, tpp = m3scan.backward_parts(dims)
    say(f"checkpoint groups {_id(case)}: {parts} pieces of {tpp} tokens, workspace {ws1} -> {ws2} bytes")
    assert ws2 < ws1   # the grouped level: fewer states kept
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
