"""Seeded synthetic inputs for the scan (shared by the tests, the benchmark and
the oracle checks).  This module draws random numbers only; it holds none of
the scan's arithmetic.

Distributions (per tensor, i.i.d.):
  x      ~ N(0, 1)
  dt     = softplus(N(0, 1) - 4)
  A      = -exp(U[0, ln 16])            one value per head
  lambda = sigmoid(N(0, 1))
  theta  ~ U[-pi, pi] * theta_scale     one angle per (token, group, pair)
  B, C   ~ N(0, 1) / sqrt(N) + 0.02     (the +0.02 stands in for the B/C bias
                                         that replaces the short convolution;
                                         nanomamba3 initialised it at 0.02)
  D      ~ N(0, 1)                      one value per head
x, B and C are drawn in fp32 and rounded to the io dtype (bf16: round to
nearest even), so both the GPU path and the oracle see identical values.
"""
from __future__ import annotations

import math
from typing import Dict

import torch

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(io_dtype: str) -> torch.dtype:
    return _DT[io_dtype]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _uniform(shape, lo, hi, g, device):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def draw(batch: int, seqlen: int, nheads: int, ngroups: int, headdim: int, dstate: int,
         rank: int, io_dtype: str = "bf16", theta_scale: float = 1.0, seed: int = 0,
         device="cpu", per_head: bool = True) -> Dict[str, torch.Tensor]:
    """Inputs for a scan over `seqlen` tokens.

    Returns x (b,L,H,R,P), dt, lam (b,L,H), theta (b,L,G,N/2), B, C (b,L,G,R,N)
    and, when per_head, A and D (H,).  All on `device`; x/B/C in the io dtype,
    the rest fp32.
    """
    assert dstate % 2 == 0 and nheads % ngroups == 0
    g = _gen(seed, device)
    dt_ = torch_dtype(io_dtype)
    out = {}
    out["x"] = _normal((batch, seqlen, nheads, rank, headdim), g, device).to(dt_)
    out["dt"] = torch.nn.functional.softplus(_normal((batch, seqlen, nheads), g, device) - 4.0)
    out["lam"] = torch.sigmoid(_normal((batch, seqlen, nheads), g, device))
    out["theta"] = _uniform((batch, seqlen, ngroups, dstate // 2), -math.pi, math.pi, g,
                            device) * float(theta_scale)
    s = 1.0 / math.sqrt(dstate)
    out["B"] = (_normal((batch, seqlen, ngroups, rank, dstate), g, device) * s + 0.02).to(dt_)
    out["C"] = (_normal((batch, seqlen, ngroups, rank, dstate), g, device) * s + 0.02).to(dt_)
    if per_head:
        out["A"] = -torch.exp(_uniform((nheads,), 0.0, math.log(16.0), g, device))
        out["D"] = _normal((nheads,), g, device)
    return out


def draw_config(cfg, device="cpu", seqlen=None, batch=None, seed=None):
    """Prefill inputs for a ScanConfig (optionally with a shorter length or batch)."""
    return draw(batch or cfg.batch, seqlen or cfg.seqlen, cfg.nheads, cfg.ngroups, cfg.headdim,
                cfg.dstate, cfg.rank, cfg.io_dtype, cfg.theta_scale,
                cfg.seed if seed is None else seed, device)


def draw_decode(cfg, steps: int, device="cpu", seed=None, batch=None):
    """Per-token inputs for `steps` decode steps, stacked on a leading step axis:
    x (S,b,H,R,P), dt, lam (S,b,H), theta (S,b,G,N/2), B, C (S,b,G,R,N)."""
    b = batch or cfg.batch
    d = draw(b, steps, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank,
             cfg.io_dtype, cfg.theta_scale, (cfg.seed if seed is None else seed) + 7919,
             device, per_head=False)
    # (b, S, ...) -> (S, b, ...), contiguous per step
    return {k: v.transpose(0, 1).contiguous() for k, v in d.items()}
