"""GPU parity of the packed variable-length prefill: each sequence of the pack
against its own oracle run (the scan restarts at every sequence start), zero-
length and sub-chunk sequences, incoming states per sequence, both kernel
families, and equal-length packs against the uniform-batch prefill."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, draw, np64, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu


def _pack(lengths, H, G, P, N, R, io, seed, theta_scale=1.0):
    """One draw of total length, split into sequences (token axis packed)."""
    T = int(sum(lengths))
    d = draw(1, max(T, 1), H, G, P, N, R, io, theta_scale, seed=seed)
    d = {k: (v[0, :T].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    return d, cu, T


def _oracle_seq(d, s0, s1, state_in=None, round_after=None):
    sl = lambda k: np64(d[k][s0:s1])[None]
    return oracle.scan(sl("x"), sl("dt"), np64(d["A"]), sl("lam"), sl("theta"), sl("B"), sl("C"),
                       np64(d["D"]), state_in=state_in, round_after=round_after)


def _run(d, cu, Lmax, Q, state_in=None, state_dtype=None):
    return m3scan.prefill_varlen(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                                 cu, Lmax, Q, state_in=state_in, state_dtype=state_dtype)


# (lengths, H, G, P, N, R, Q, io)
CASES = [
    ([130, 0, 64, 17, 300, 1], 4, 1, 64, 128, 2, 32, "bf16"),     # matrix-core path
    ([200, 63, 1, 129], 2, 2, 64, 128, 4, 64, "bf16"),
    ([257, 0, 31, 96, 1000], 3, 1, 64, 128, 4, 32, "bf16"),         # 128-row chunks (4 waves)
    ([64, 190, 7], 2, 1, 64, 128, 2, 64, "bf16"),
    ([100, 0, 37, 64, 5], 4, 1, 16, 16, 1, 32, "fp32"),            # generic path
]


def _id(c):
    return "L{}-H{}G{}P{}N{}R{}Q{}-{}".format("_".join(map(str, c[0])), *c[1:])


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_varlen_each_sequence_matches_oracle(case):
    lengths, H, G, P, N, R, Q, io = case
    say("varlen", _id(case))
    d, cu, T = _pack(lengths, H, G, P, N, R, io, seed=sum(lengths))
    y, st = _run(d, cu, max(lengths), Q)
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    for s, n in enumerate(lengths):
        if n == 0:
            assert float(st.h[s].abs().max()) == 0.0          # nothing scanned: the zero state
            assert float(st.b_last[s].float().abs().max()) == 0.0
            continue
        yr, hr = _oracle_seq(d, c[s], c[s + 1])
        ey = slice_err(np64(y[c[s]:c[s + 1]])[None], yr, 2)
        eh = slice_err(np64(st.h[s:s + 1]), hr, 1)
        say(f"  seq {s} (len {n}): y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL[io] and eh <= TOL[io]
        assert torch.equal(st.b_last[s], d["B"][c[s + 1] - 1])
        assert torch.equal(st.x_last[s], d["x"][c[s + 1] - 1])


@pytest.mark.parametrize("Q,R", [(64, 4), (32, 1)])
def test_varlen_from_states(Q, R):
    lengths = [90, 0, 33, 200]
    H, G, P, N = 2, 1, 64, 128
    say("varlen from states", Q, R)
    d, cu, T = _pack(lengths, H, G, P, N, R, "bf16", seed=71 + Q)
    gen = torch.Generator(device="cpu").manual_seed(3)
    ns = len(lengths)
    h0 = torch.randn((ns, H, N, P), generator=gen).cuda()
    bl = torch.randn((ns, G, R, N), generator=gen).to(torch.bfloat16).cuda()
    xl = torch.randn((ns, H, R, P), generator=gen).to(torch.bfloat16).cuda()
    y, st = _run(d, cu, max(lengths), Q, state_in=m3scan.DecodeState(h0, bl, xl))
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    for s, n in enumerate(lengths):
        if n == 0:   # the state and the carry pass through unchanged
            assert torch.equal(st.h[s], h0[s])
            assert torch.equal(st.b_last[s], bl[s]) and torch.equal(st.x_last[s], xl[s])
            continue
        yr, hr = _oracle_seq(d, c[s], c[s + 1], state_in=(np64(h0[s:s + 1]), np64(bl[s:s + 1]),
                                                          np64(xl[s:s + 1])))
        ey = slice_err(np64(y[c[s]:c[s + 1]])[None], yr, 2)
        eh = slice_err(np64(st.h[s:s + 1]), hr, 1)
        say(f"  seq {s} (len {n}): y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_varlen_equal_lengths_is_the_uniform_prefill():
    """Equal lengths: the same kernels, the same chunking, one sweep per (b, h) in
    both (b * H = 512 workgroups, so the uniform path uses no segments either):
    bit-identical outputs and states."""
    b, L, H, G, P, N, R, Q = 8, 160, 64, 1, 64, 128, 2, 32
    d = draw(b, L, H, G, P, N, R, "bf16", 1.0, seed=91)
    y0, s0 = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"], Q)
    flat = {k: (v.reshape((b * L,) + tuple(v.shape[2:])).contiguous() if v.dim() > 1 else v)
            for k, v in d.items()}
    cu = torch.arange(0, b * L + 1, L, dtype=torch.int64, device="cuda")
    y1, s1 = _run(flat, cu, L, Q)
    torch.cuda.synchronize()
    assert torch.equal(y1.reshape(y0.shape), y0)
    assert torch.equal(s1.h, s0.h)
    assert torch.equal(s1.b_last, s0.b_last) and torch.equal(s1.x_last, s0.x_last)


def test_varlen_bf16_state():
    lengths = [70, 130, 1]
    H, G, P, N, R, Q = 2, 1, 64, 128, 2, 32
    d, cu, T = _pack(lengths, H, G, P, N, R, "bf16", seed=5)
    y, st = _run(d, cu, max(lengths), Q, state_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    for s, n in enumerate(lengths):
        flags = np.zeros(n, bool)
        flags[-1] = True
        yr, hr = _oracle_seq(d, c[s], c[s + 1], round_after=flags)
        assert slice_err(np64(y[c[s]:c[s + 1]])[None], yr, 2) <= TOL["bf16"]
        assert slice_err(np64(st.h[s:s + 1]), hr, 1) <= TOL["bf16"]


def test_varlen_inconsistent_offsets_are_clamped():
    """Offsets outside [0, T], decreasing ones and lengths above the bound are
    clamped on the device: the call completes and every sequence it can still
    make out is scanned within its clamped span."""
    lengths = [40, 40, 40]
    H, G, P, N, R, Q = 2, 1, 64, 128, 2, 32
    d, _, T = _pack(lengths, H, G, P, N, R, "bf16", seed=6)
    # seq 0: [-5, 40) -> [0, 40); seq 1: [40, 30) -> empty; seq 2: [30, 999) -> [30, 30 + 64)
    cu = torch.tensor([-5, 40, 30, 999], dtype=torch.int64, device="cuda")
    y, st = _run(d, cu, 64, Q)
    torch.cuda.synchronize()
    yr, hr = _oracle_seq(d, 0, 40)
    # tokens 30..39 are also in sequence 2's clamped span (its writes race there)
    assert slice_err(np64(y[0:30])[None], yr[:, :30], 2) <= TOL["bf16"]
    assert slice_err(np64(st.h[0:1]), hr, 1) <= TOL["bf16"]
    assert float(st.h[1].abs().max()) == 0.0
    yr, hr = _oracle_seq(d, 30, 94)
    assert slice_err(np64(st.h[2:3]), hr, 1) <= TOL["bf16"]
