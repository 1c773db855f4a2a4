"""The workloads at their full sizes, in the launch configuration the benchmark
times, checked on sampled (batch, head) slices that the oracle computes one by
one (a full-size oracle run would take hours)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, say
from state_space_sequence_scan_amd import CONFIGS, inputs, m3scan

pytestmark = pytest.mark.gpu

f64 = lambda t: t.detach().double().cpu().numpy()


def _slice(d, bi, h, G, H):
    g = h // (H // G)
    return [f64(d["x"][bi:bi + 1, :, h:h + 1]), f64(d["dt"][bi:bi + 1, :, h:h + 1]),
            f64(d["A"][h:h + 1]), f64(d["lam"][bi:bi + 1, :, h:h + 1]),
            f64(d["theta"][bi:bi + 1, :, g:g + 1]), f64(d["B"][bi:bi + 1, :, g:g + 1]),
            f64(d["C"][bi:bi + 1, :, g:g + 1]), f64(d["D"][h:h + 1])]


def _err(g, r):
    return float(np.max(np.abs(g - r)) / np.max(np.abs(r)))


@pytest.mark.parametrize("name", ["siso_l256_fp32", "nanomamba3", "siso_l8192", "mimo4_l16384"])
def test_prefill_workload_sampled(name):
    cfg = CONFIGS[name]
    say("workload", name, cfg.label)
    d = inputs.draw_config(cfg, device="cuda")
    y, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                           cfg.chunk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.seed)
    picks = [(0, 0), (cfg.batch - 1, cfg.nheads - 1)] + \
            [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.nheads))) for _ in range(2)]
    for bi, h in picks:
        yr, hr = oracle.scan(*_slice(d, bi, h, cfg.ngroups, cfg.nheads))
        ey = _err(f64(y[bi:bi + 1, :, h:h + 1]), yr)
        eh = _err(f64(st.h[bi:bi + 1, h:h + 1]), hr)
        say(f"  slice b={bi} h={h}: y {ey:.2e} state {eh:.2e}")
        assert ey <= TOL[cfg.io_dtype] and eh <= TOL[cfg.io_dtype]


def test_decode_workload_sampled():
    """1.5B MIMO R=4 layer, batch 256: 1024-token prefill, then 512 decode steps."""
    cfg = CONFIGS["mimo4_decode_b256"]
    say("workload mimo4_decode_b256", cfg.label)
    d = inputs.draw_config(cfg, device="cuda")
    dd = inputs.draw_decode(cfg, cfg.decode_steps, device="cuda")
    y, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                           cfg.chunk)
    ydec = torch.empty((cfg.decode_steps,) + tuple(d["x"][:, 0].shape), dtype=d["x"].dtype, device="cuda")
    for t in range(cfg.decode_steps):
        m3scan.decode_step(st, dd["x"][t], dd["dt"][t], d["A"], dd["lam"][t], dd["theta"][t],
                           dd["B"][t], dd["C"][t], d["D"], y_t=ydec[t])
    torch.cuda.synchronize()
    for bi, h in [(0, 0), (255, 63), (137, 21)]:
        g = h // (cfg.nheads // cfg.ngroups)
        pre = _slice(d, bi, h, cfg.ngroups, cfg.nheads)
        dec = [f64(dd["x"][:, bi:bi + 1, h:h + 1].transpose(0, 1)),
               f64(dd["dt"][:, bi:bi + 1, h:h + 1].transpose(0, 1)), pre[2],
               f64(dd["lam"][:, bi:bi + 1, h:h + 1].transpose(0, 1)),
               f64(dd["theta"][:, bi:bi + 1, g:g + 1].transpose(0, 1)),
               f64(dd["B"][:, bi:bi + 1, g:g + 1].transpose(0, 1)),
               f64(dd["C"][:, bi:bi + 1, g:g + 1].transpose(0, 1)), pre[7]]
        full = [np.concatenate([a, c], axis=1) if a.ndim > 1 else a for a, c in zip(pre, dec)]
        yr, hr = oracle.scan(*full)
        yg = np.concatenate([f64(y[bi:bi + 1, :, h:h + 1]),
                             f64(ydec[:, bi:bi + 1, h:h + 1].transpose(0, 1))], axis=1)
        ey, eh = _err(yg, yr), _err(f64(st.h[bi:bi + 1, h:h + 1]), hr)
        say(f"  slice b={bi} h={h}: y {ey:.2e} state {eh:.2e}")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("name", ["nanomamba3", "mimo4_l16384"])
def test_backward_workload_sampled(name):
    """The backward at the full size of a training-shaped workload (nanomamba3 is the benchmark's
    default for it): per-head gradients dx, ddt, dlambda of sampled (batch, head) slices
    against the oracle's adjoint run on that slice alone (group-shared and batch-summed
    gradients mix slices and are covered by the small-size tests)."""
    cfg = CONFIGS[name]
    say("backward workload", name)
    d = inputs.draw_config(cfg, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 11)
    dy = torch.randn(d["x"].shape, generator=g, device="cuda").to(d["x"].dtype)
    gr = m3scan.backward(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"], dy,
                         want_state_grads=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.seed + 1)
    for bi, h in [(0, 0), (cfg.batch - 1, cfg.nheads - 1), (int(rng.integers(cfg.batch)), int(rng.integers(cfg.nheads)))]:
        ref = oracle.scan_backward(*_slice(d, bi, h, cfg.ngroups, cfg.nheads), f64(dy[bi:bi + 1, :, h:h + 1]))
        for k in ("dx", "ddt", "dlam"):
            gv = f64(gr[k][bi:bi + 1, :, h:h + 1])
            e = _err(gv, ref[k])
            say(f"  ({bi},{h}) {k} {e:.2e}")
            assert e <= 1e-3, (bi, h, k, e)


def test_fused_prefill_workload_sampled():
    """The fused prologue/epilogue at the full size of the 1.5B-scale SISO layer."""
    cfg = CONFIGS["siso_l8192"]
    say("fused workload siso_l8192")
    d = inputs.draw_config(cfg, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 23)
    R, N = cfg.rank, cfg.dstate
    fz = {"A_t": -torch.exp(torch.rand(d["dt"].shape, generator=g, device="cuda") * np.log(16.0)),
          "b_norm_w": 1.0 + 0.3 * torch.randn((R, N), generator=g, device="cuda"),
          "c_norm_w": 1.0 + 0.3 * torch.randn((R, N), generator=g, device="cuda"),
          "b_bias": 0.02 + 0.05 * torch.randn((R, N), generator=g, device="cuda"),
          "c_bias": 0.02 + 0.05 * torch.randn((R, N), generator=g, device="cuda"),
          "z": torch.randn(d["x"].shape, generator=g, device="cuda").to(d["x"].dtype)}
    y, st = m3scan.prefill_fused(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                                 cfg.chunk, **fz)
    torch.cuda.synchronize()
    for bi, h in [(0, 0), (cfg.batch - 1, cfg.nheads - 1)]:
        args = _slice(d, bi, h, cfg.ngroups, cfg.nheads)
        args[2] = f64(fz["A_t"][bi:bi + 1, :, h:h + 1])
        yr, hr = oracle.scan_fused(*args, b_norm_w=f64(fz["b_norm_w"]), c_norm_w=f64(fz["c_norm_w"]),
                                   b_bias=f64(fz["b_bias"]), c_bias=f64(fz["c_bias"]),
                                   z=f64(fz["z"][bi:bi + 1, :, h:h + 1]))
        ey = _err(f64(y[bi:bi + 1, :, h:h + 1]), yr)
        eh = _err(f64(st.h[bi:bi + 1, h:h + 1]), hr)
        say(f"  ({bi},{h}) y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
