"""GPU parity of the token-serial prefill (small states: N/2 a power of two, N/2 * P <= 256,
no fused norm, bias, gate or output norm), against the oracle: every rank up to 8 (the
kernel is instantiated per rank), io dtypes, groups, states and carries passed in,
sequences shorter than, equal to and longer than a staged block (ragged last blocks),
the smallest (N = 2) and widest (N = 128) state rows, a bf16 state, packed
variable-length batches with an empty sequence, a per-token decay rate and angles per
head (the two fused inputs this path takes), and a zero-length scan."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, draw, np64, oracle_args, oracle_state, rand_state, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")

# (b, L, H, G, P, N, R, io, with_state); block sizes these take: 64 tokens at N = P = 16,
# R = 1; 8 at N = 32, P = 16, R = 4; 1-4 at the widest rows
CASES = [
    (1, 256, 4, 1, 16, 16, 1, "fp32", False),    # the small fp32 workload's shape
    (2, 1, 4, 2, 16, 16, 1, "fp32", True),
    (2, 63, 4, 2, 16, 16, 2, "fp32", True),
    (1, 64, 2, 1, 16, 16, 3, "fp32", True),
    (1, 65, 2, 1, 16, 16, 4, "bf16", True),
    (3, 300, 6, 3, 8, 16, 5, "bf16", False),
    (1, 77, 2, 2, 16, 32, 4, "fp32", True),
    (1, 40, 2, 1, 4, 2, 6, "fp32", True),        # N = 2: one rotation pair
    (2, 50, 2, 1, 2, 128, 8, "fp32", True),      # N = 128, P = 2: a whole wave per column
    (1, 129, 4, 4, 32, 8, 7, "bf16", True),
]


def _id(c):
    return "b{}L{}H{}G{}P{}N{}R{}-{}{}".format(*c[:8], "-state" if c[8] else "")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_serial_prefill_matches_oracle(case):
    b, L, H, G, P, N, R, io, with_state = case
    say("serial prefill", _id(case))
    d = draw(b, L, H, G, P, N, R, io, 1.0, seed=L * 7 + R)
    st0 = rand_state(b, H, G, N, P, R, io, seed=L + 3) if with_state else None
    y, st = m3scan.prefill(*[d[k] for k in NAMES], 32, state_in=st0)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d), state_in=oracle_state(st0))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]
    # the carry written is the last token's B and X
    assert torch.equal(st.b_last, d["B"][:, -1]) and torch.equal(st.x_last, d["x"][:, -1])


def test_serial_prefill_bf16_state():
    """A bf16 state written after the last token (the oracle rounds there too)."""
    b, L, H, G, P, N, R = 2, 150, 4, 1, 16, 16, 2
    d = draw(b, L, H, G, P, N, R, "fp32", 1.0, seed=91)
    y, st = m3scan.prefill(*[d[k] for k in NAMES], 32, state_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    flags = np.zeros(L, bool)
    flags[-1] = True
    yr, hr = oracle.scan(*oracle_args(d), round_after=flags)
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"serial bf16 state: y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL["fp32"] and eh <= 2e-2


def test_serial_prefill_varlen():
    """Packed sequences (one of them empty), each against its own oracle run."""
    lengths, H, G, P, N, R = [70, 0, 1, 200, 33], 4, 2, 16, 16, 2
    T = sum(lengths)
    d = draw(1, T, H, G, P, N, R, "fp32", 1.0, seed=17)
    d = {k: (v[0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    y, st = m3scan.prefill_varlen(*[d[k] for k in NAMES], cu, max(lengths), 32)
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    for s, n in enumerate(lengths):
        if n == 0:
            assert float(st.h[s].abs().max()) == 0.0
            continue
        sl = lambda k: np64(d[k][c[s]:c[s + 1]])[None]
        yr, hr = oracle.scan(sl("x"), sl("dt"), np64(d["A"]), sl("lam"), sl("theta"), sl("B"), sl("C"),
                             np64(d["D"]))
        ey = slice_err(np64(y[c[s]:c[s + 1]])[None], yr, 2)
        eh = slice_err(np64(st.h[s])[None], hr, 1)
        say(f"  sequence {s} (L={n}): y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL["fp32"] and eh <= TOL["fp32"]


def test_serial_prefill_per_token_A_and_angle_groups():
    """The fused call with only a per-token decay rate and angles per head stays on this path."""
    b, L, H, G, Gt, P, N, R = 2, 90, 4, 1, 4, 16, 16, 2
    d = draw(b, L, H, G, P, N, R, "fp32", 1.0, seed=23)
    g = torch.Generator(device="cpu").manual_seed(5)
    d["theta"] = ((torch.rand((b, L, Gt, N // 2), generator=g) * 2 - 1) * np.pi).cuda()
    A_t = (-torch.rand((b, L, H), generator=g) * 2).cuda()
    y, st = m3scan.prefill_fused(*[d[k] for k in NAMES], 32, A_t=A_t)
    torch.cuda.synchronize()
    args = [np64(d[k]) for k in NAMES]
    args[2] = np64(A_t)
    yr, hr = oracle.scan_fused(*args)
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"serial per-token A, {Gt} angle groups: y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL["fp32"] and eh <= TOL["fp32"]


def test_serial_prefill_zero_length_passes_the_state_through():
    b, H, G, P, N, R = 2, 4, 1, 16, 16, 1
    d = draw(b, 1, H, G, P, N, R, "fp32", 1.0, seed=2)
    d0 = {k: (v[:, :0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    st0 = rand_state(b, H, G, N, P, R, "fp32", seed=9)
    y, st = m3scan.prefill(*[d0[k] for k in NAMES], 32, state_in=st0)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(st.h, st0.h)
