"""GPU parity over a seeded sweep of 32 shapes, against the oracle: batch, length (1 to 700,
so ragged last chunks and sequences shorter than a chunk), heads and groups, rank, chunk
size, io dtype and kernel family (matrix-core bf16 at N=128, P=64; the fp32 path at
smaller N and P), with and without an incoming state; each case runs a prefill, then
two decode steps continuing it, and the backward (the fast kernel at N=128, P=64, the
generic one at the fp32 shapes)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, draw, np64, oracle_args, oracle_state, rand_state, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")


def _cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mfma = i % 4 != 3
        H = int(rng.choice([2, 4, 6, 8]))
        G = int(rng.choice([g for g in (1, 2, H) if H % g == 0]))
        R = int(rng.choice([1, 2, 4]))
        b = int(rng.integers(1, 4))
        L = int(rng.integers(1, 701))
        if mfma:
            out.append((b, L, H, G, 64, 128, R, int(rng.choice([32, 64])), "bf16", bool(rng.integers(2))))
        else:
            NP = int(rng.choice([16, 32]))
            out.append((b, L, H, G, NP, NP, min(R, 2), int(rng.choice([16, 32])), "fp32", bool(rng.integers(2))))
    return out


CASES = _cases(32)


def _id(c):
    return "b{}L{}H{}G{}P{}N{}R{}Q{}-{}{}".format(*c[:9], "-state" if c[9] else "")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_random_shape_prefill_decode_backward(case):
    b, L, H, G, P, N, R, Q, io, with_state = case
    say("random shape", _id(case))
    steps = 2
    d = draw(b, L + steps, H, G, P, N, R, io, 1.0, seed=L * 13 + H)
    pre = {k: (v[:, :L].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    st0 = rand_state(b, H, G, N, P, R, io, seed=L + 1) if with_state else None
    y, st = m3scan.prefill(*[pre[k] for k in NAMES], Q, state_in=st0)
    ys = [y]
    for t in range(L, L + steps):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ys.append(m3scan.decode_step(st, *[tok[k] for k in NAMES])[:, None])
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d), state_in=oracle_state(st0))
    ey = slice_err(np64(torch.cat(ys, dim=1)), yr, 2)
    eh = slice_err(np64(st.h), hr, 1)
    say(f"  prefill + decode: y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]
    gen = torch.Generator(device="cpu").manual_seed(L)
    dy = torch.randn(tuple(pre["x"].shape), generator=gen).to(pre["x"].dtype).cuda()
    gr = m3scan.backward(*[pre[k] for k in NAMES], dy, state_in=st0)
    torch.cuda.synchronize()
    ref = oracle.scan_backward(*[np64(pre[k]) for k in NAMES], np64(dy), state_in=oracle_state(st0))
    worst = 0.0
    for k in ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0"):
        r = ref[k]
        e = float(np.max(np.abs(np64(gr[k]) - r)) / max(np.max(np.abs(r)), 1e-30)) if r.size else 0.0
        worst = max(worst, e)
    say(f"  backward: worst {worst:.2e}")
    assert worst <= 1e-3
