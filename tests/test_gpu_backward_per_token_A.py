"""GPU parity of the backward pass with a per-token decay rate A_t
(m3_backward_per_token_A through the C ABI) against the oracle's adjoint loop run
with the same A_t (oracle.scan_backward with A shaped (b, L, H), pinned by finite
differences of the forward oracle): every gradient, dA per token included, for
equal-length batches (whole and split sequences, with a carried state and a
final-state cotangent) and a packed batch checked sequence by sequence; and A_t
constant over the tokens of each head, which must give the per-head call's
gradients bit for bit, with dA_t summing to its dA.

Bar: 1e-3 max relative error per gradient tensor, as for the per-head backward."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import draw, np64, say
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-3
P, N = 64, 128
NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")
GRADS = ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0")


def _rel(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30))


def _rate(shape, seed):
    """A_t drawn like the per-head rates: -exp(U(0, ln 16))."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (-torch.exp(torch.rand(shape, generator=g, dtype=torch.float64) * np.log(16.0))).float().cuda()


def _state(nb, H, G, R, tdt, gen):
    h0 = torch.randn((nb, H, N, P), generator=gen).cuda()
    bl = torch.randn((nb, G, R, N), generator=gen).to(tdt).cuda()
    xl = torch.randn((nb, H, R, P), generator=gen).to(tdt).cuda()
    return m3scan.DecodeState(h0, bl, xl)


CASES = [
    # b, L, H, G, R, io, state, dh
    (2, 37, 4, 2, 4, "bf16", True, True),
    (1, 64, 4, 1, 1, "fp32", False, True),
    (4, 200, 24, 1, 2, "bf16", False, True),   # split into pieces
    (2, 150, 4, 2, 4, "fp32", True, True),     # split, with a carried state
]


def _id(c):
    return "b{}L{}H{}G{}R{}-{}{}{}".format(*c[:6], "-state" if c[6] else "", "-dh" if c[7] else "")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_per_token_A_matches_oracle(case):
    b, L, H, G, R, io, with_state, with_dh = case
    say("backward A_t", _id(case), "pieces", m3scan.backward_parts(m3scan.make_dims(b, L, H, G, P, N, R, 1, 0)))
    d = draw(b, L, H, G, P, N, R, io, 2.0, seed=L * 5 + R)
    At = _rate((b, L, H), seed=L + 17)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    gen = torch.Generator(device="cpu").manual_seed(L + 3)
    dy = torch.randn((b, L, H, R, P), generator=gen).to(tdt).cuda()
    dh = torch.randn((b, H, N, P), generator=gen).cuda() if with_dh else None
    st = _state(b, H, G, R, tdt, gen) if with_state else None
    gr = m3scan.backward_per_token_A(d["x"], d["dt"], At, d["lam"], d["theta"], d["B"], d["C"], d["D"], dy,
                                     dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    args = [np64(d[k]) for k in NAMES]
    args[2] = np64(At)
    ref = oracle.scan_backward(*args, np64(dy), dh_out=np64(dh),
                               state_in=(np64(st.h), np64(st.b_last), np64(st.x_last)) if with_state else None)
    assert gr["dA"].shape == (b, L, H)
    errs = {k: _rel(np64(gr[k]), ref[k]) for k in GRADS}
    if with_state:
        errs["db_last"] = _rel(np64(gr["db_last"]), ref["db_last"])
        errs["dx_last"] = _rel(np64(gr["dx_last"]), ref["dx_last"])
    say("  " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL_BWD}
    assert not bad, bad


def test_backward_per_token_A_packed_batch_matches_oracle():
    """Packed sequences (empty, one-token, split into pieces) with A_t: each sequence
    against the oracle run on it alone."""
    lengths, H, G, R = [130, 0, 64, 17, 300, 1], 4, 1, 2
    ns, Lmax, T = len(lengths), max(lengths), sum(lengths)
    d = draw(1, T, H, G, P, N, R, "bf16", 2.0, seed=T + 1)
    d = {k: (v[0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    At = _rate((T, H), seed=T + 2)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(T + 5)
    dy = torch.randn((T, H, R, P), generator=gen).to(torch.bfloat16).cuda()
    dh = torch.randn((ns, H, N, P), generator=gen).cuda()
    st = _state(ns, H, G, R, torch.bfloat16, gen)
    say("backward A_t packed", lengths, "pieces", m3scan.backward_parts(m3scan.make_dims(ns, Lmax, H, G, P, N, R, 1, 0)))
    gr = m3scan.backward_per_token_A(d["x"], d["dt"], At, d["lam"], d["theta"], d["B"], d["C"], d["D"], dy,
                                     cu_seqlens=cu, max_seqlen=Lmax, dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    assert gr["dA"].shape == (T, H)
    c = [0] + list(np.cumsum(lengths))
    dD = np.zeros(H)
    for s, n in enumerate(lengths):
        if n == 0:
            assert np.array_equal(np64(gr["dh0"][s]), np64(dh[s]))
            continue
        sl = lambda t: np64(t[c[s]:c[s + 1]])[None]
        ref = oracle.scan_backward(sl(d["x"]), sl(d["dt"]), sl(At), sl(d["lam"]), sl(d["theta"]), sl(d["B"]),
                                   sl(d["C"]), np64(d["D"]), sl(dy), dh_out=np64(dh[s:s + 1]),
                                   state_in=(np64(st.h[s:s + 1]), np64(st.b_last[s:s + 1]),
                                             np64(st.x_last[s:s + 1])))
        errs = {k: _rel(np64(gr[k][c[s]:c[s + 1]])[None], ref[k])
                for k in ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC")}
        for k in ("dh0", "db_last", "dx_last"):
            errs[k] = _rel(np64(gr[k][s:s + 1]), ref[k])
        dD += ref["dD"]
        say(f"  seq {s} (len {n}): " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
        bad = {k: v for k, v in errs.items() if not v <= TOL_BWD}
        assert not bad, (s, bad)
    eD = _rel(np64(gr["dD"]), dD)
    say(f"  dD {eD:.1e}")
    assert eD <= TOL_BWD


@pytest.mark.parametrize("L", [40, 200])
def test_constant_per_token_A_matches_per_head_call(L):
    """A_t[b, t, h] = A[h]: the same decays, so every gradient but dA is bit-identical
    to the per-head call's, and dA_t summed over batch and tokens is its dA (up to the
    order of the fp32 sums).  L = 200 splits the sequences into pieces."""
    b, H, G, R = 2, 24, 2, 2
    d = draw(b, L, H, G, P, N, R, "bf16", 2.0, seed=L + 40)
    gen = torch.Generator(device="cpu").manual_seed(L + 41)
    dy = torch.randn((b, L, H, R, P), generator=gen).to(torch.bfloat16).cuda()
    dh = torch.randn((b, H, N, P), generator=gen).cuda()
    st = _state(b, H, G, R, torch.bfloat16, gen)
    At = d["A"].view(1, 1, H).expand(b, L, H).contiguous()
    g1 = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh, state_in=st)
    g2 = m3scan.backward_per_token_A(d["x"], d["dt"], At, d["lam"], d["theta"], d["B"], d["C"], d["D"], dy,
                                     dh_out=dh, state_in=st)
    torch.cuda.synchronize()
    for k in g1:
        if k != "dA":
            assert torch.equal(g1[k], g2[k]), k
    e = _rel(np64(g2["dA"]).sum(axis=(0, 1)), np64(g1["dA"]))
    say(f"backward constant A_t L={L}: dA sum {e:.1e}")
    assert e <= 1e-4
