"""GPU parity at the edges of the input ranges, against the oracle.

The workloads draw dt = softplus(N(0,1) - 4), lambda in (0, 1) and angles within a few pi.
Here the same shapes see:
- strong decay: a fifth of the tokens with dt in [5, 15], so e^{dt A} underflows to zero
  inside a chunk and the state restarts from the input terms (every decay factor the
  matrix-core prefill forms is at most 1, so none overflows);
- dt = 0 on a run of tokens: alpha = 1 and beta = gamma = 0, so the state passes through
  them untouched and only the skip term and C h reach y;
- lambda exactly 0 or 1 per token (the two one-sided endpoint rules);
- theta = 0 (no rotation) and angles of up to 20 rad per token.
Each runs the matrix-core prefill (bf16, R = 2 and 4), the fp32 prefill, prefill
followed by decode steps, and the backward (bar 1e-3 as for the other backward tests)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, draw, gpu_prefill, np64, oracle_args, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")
EDGES = ("strong_decay", "dt_zero_run", "lambda_0_1", "theta_zero", "theta_large")


def _edit(d, edge, seed):
    """Replace dt, lambda or theta of a drawn case by the edge's values (in place)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = tuple(d["dt"].shape)
    if edge == "strong_decay":
        hit = torch.rand(shape, generator=g) < 0.2
        big = 5.0 + 10.0 * torch.rand(shape, generator=g)
        d["dt"] = torch.where(hit.cuda(), big.cuda(), d["dt"])
    elif edge == "dt_zero_run":
        dt = d["dt"].clone()
        L = shape[1]
        dt[:, L // 4:L // 4 + max(L // 3, 1)] = 0.0
        d["dt"] = dt
    elif edge == "lambda_0_1":
        d["lam"] = (torch.rand(shape, generator=g) < 0.5).float().cuda()
    elif edge == "theta_zero":
        d["theta"] = torch.zeros_like(d["theta"])
    elif edge == "theta_large":
        d["theta"] = (40.0 * torch.rand(tuple(d["theta"].shape), generator=g) - 20.0).cuda()
    return d


@pytest.mark.parametrize("edge", EDGES)
@pytest.mark.parametrize("R,Q", [(2, 64), (4, 32)])
def test_mfma_prefill_at_edges(edge, R, Q):
    b, L, H, G = 2, 300, 2, 1
    say("mfma prefill edge", edge, "R", R, "Q", Q)
    d = _edit(draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=31 + R), edge, seed=5)
    y, st = gpu_prefill(d, Q)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all()) and bool(torch.isfinite(st.h).all())
    yr, hr = oracle.scan(*oracle_args(d))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("edge", EDGES)
def test_fp32_prefill_at_edges(edge):
    b, L, H, G, R, N, P = 2, 200, 4, 2, 1, 16, 16
    say("fp32 prefill edge", edge)
    d = _edit(draw(b, L, H, G, P, N, R, "fp32", 1.0, seed=41), edge, seed=6)
    y, st = gpu_prefill(d, 32)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["fp32"] and eh <= TOL["fp32"]


@pytest.mark.parametrize("edge", EDGES)
def test_prefill_then_decode_at_edges(edge):
    """The first 96 tokens by prefill, the last 32 by decode steps: y of every token and
    the final state against one oracle scan over all 128."""
    b, L, L0, H, G, R = 2, 128, 96, 4, 1, 4
    say("prefill + decode edge", edge)
    d = _edit(draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=51), edge, seed=7)
    pre = {k: (v[:, :L0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    y0, st = gpu_prefill(pre, 64)
    ys = [y0]
    for t in range(L0, L):
        tok = {k: (d[k][:, t].contiguous() if d[k].dim() > 1 else d[k]) for k in NAMES}
        ys.append(m3scan.decode_step(st, tok["x"], tok["dt"], d["A"], tok["lam"], tok["theta"], tok["B"],
                                     tok["C"], d["D"]).unsqueeze(1))
    y = torch.cat(ys, dim=1)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def _rel(g, r):
    return float(np.max(np.abs(np.asarray(g) - r)) / max(np.max(np.abs(r)), 1e-30))


@pytest.mark.parametrize("edge", EDGES)
def test_backward_at_edges(edge):
    """Every gradient; L = 200 with 24 heads splits each sequence into pieces, so the
    pieces' decay and angle sums meet the edge values too."""
    b, L, H, G, R = 2, 200, 24, 1, 2
    say("backward edge", edge)
    d = _edit(draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=61), edge, seed=8)
    gen = torch.Generator(device="cpu").manual_seed(9)
    dy = torch.randn(tuple(d["x"].shape), generator=gen).to(torch.bfloat16).cuda()
    dh = torch.randn((b, H, 128, 64), generator=gen).cuda()
    gr = m3scan.backward(*[d[k] for k in NAMES], dy, dh_out=dh)
    torch.cuda.synchronize()
    ref = oracle.scan_backward(*oracle_args(d), np64(dy), dh_out=np64(dh))
    errs = {k: _rel(np64(gr[k]), ref[k]) for k in ("dx", "ddt", "dA", "dlam", "dtheta", "dB", "dC", "dD", "dh0")}
    say("  " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= 1e-3}
    assert not bad, bad
