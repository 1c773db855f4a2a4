"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare them.

Error metric: per (b, h) slice, max|gpu - ref| / max|ref| over that slice's
outputs, maximised over slices (elementwise relative error is undefined where
outputs cross zero).  Bars: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with
fp32 state.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from state_space_sequence_scan_amd import inputs, m3scan

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def slice_err(gpu, ref, head_axis):
    """max over (b, h) of max|gpu-ref| / max|ref| within the slice."""
    g = np.moveaxis(np.asarray(gpu, np.float64), head_axis, 1)
    r = np.moveaxis(np.asarray(ref, np.float64), head_axis, 1)
    b, H = g.shape[:2]
    g = g.reshape(b, H, -1)
    r = r.reshape(b, H, -1)
    if g.shape[2] == 0:
        return 0.0
    num = np.max(np.abs(g - r), axis=2)
    den = np.maximum(np.max(np.abs(r), axis=2), 1e-30)
    return float(np.max(num / den))


def slice_errs(gpu, ref, head_axis):
    """Per (b, h) slice: the metric of slice_err (max|gpu-ref| / max|ref|), as an array
    (b, H), and the elementwise diagnostic max |gpu-ref| / (|ref| + 1e-3 max|ref|)
    over the whole block: it exposes errors on small outputs (early or strongly decayed
    tokens) that the slice maximum would hide."""
    g = np.moveaxis(np.asarray(gpu, np.float64), head_axis, 1)
    r = np.moveaxis(np.asarray(ref, np.float64), head_axis, 1)
    b, H = g.shape[:2]
    g = g.reshape(b, H, -1)
    r = r.reshape(b, H, -1)
    if g.shape[2] == 0:
        return np.zeros((b, H)), 0.0
    d = np.abs(g - r)
    scale = np.maximum(np.max(np.abs(r), axis=2), 1e-30)
    per_slice = np.max(d, axis=2) / scale
    elem = float(np.max(d / (np.abs(r) + 1e-3 * scale[:, :, None])))
    return per_slice, elem


def onorm_slice_errs(gpu_n, ref_pre, w, eps):
    """Error of outputs after the output RMSNorm, on the scale of the rows before it.

    The norm divides every row (b, t, h, r, :) by its own root mean square, so it magnifies
    the absolute error of rows that are small next to the rest of their slice; the bar of
    the scan output (max|error| / max|ref| per slice) is therefore applied before that
    division: each normalised row's error is multiplied back by the oracle's row RMS and
    divided by the head's largest |weight|.  gpu_n (b, L, H, R, P) is the normalised GPU
    output, ref_pre the oracle's output before the norm, w (H, P) the weight.  Returns
    (per-slice errors (b, H), max of the plain per-slice error of the normalised outputs)."""
    pre = np.asarray(ref_pre, np.float64)
    w = np.asarray(w, np.float64)
    rms = np.sqrt(np.mean(pre * pre, axis=-1, keepdims=True) + eps)
    ref_n = pre / rms * w[None, None, :, None, :]
    d = np.abs(np.asarray(gpu_n, np.float64) - ref_n) * rms / np.max(np.abs(w), axis=1)[None, None, :, None, None]
    b, L, H = pre.shape[:3]
    num = np.moveaxis(d, 2, 1).reshape(b, H, -1).max(-1)
    den = np.maximum(np.moveaxis(np.abs(pre), 2, 1).reshape(b, H, -1).max(-1), 1e-30)
    plain, _ = slice_errs(gpu_n, ref_n, 2)
    return num / den, float(np.max(plain))


def oracle_args(d):
    return [np64(d[k]) for k in ("x", "dt", "A", "lam", "theta", "B", "C", "D")]


def gpu_prefill(d, chunk, state_in=None):
    return m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                          chunk, state_in=state_in)


def to_device(d, dev="cuda"):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def draw(b, L, H, G, P, N, R, io="fp32", theta_scale=1.0, seed=0, device="cuda"):
    return inputs.draw(b, L, H, G, P, N, R, io_dtype=io, theta_scale=theta_scale, seed=seed,
                       device=device)


def rand_state(b, H, G, N, P, R, io, seed=5, device="cuda"):
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt_ = inputs.torch_dtype(io)
    h = torch.randn((b, H, N, P), generator=g).to(device)
    bl = torch.randn((b, G, R, N), generator=g).to(dt_).to(device)
    xl = torch.randn((b, H, R, P), generator=g).to(dt_).to(device)
    return m3scan.DecodeState(h, bl, xl)


def oracle_state(st):
    if st is None:
        return None
    return (np64(st.h), np64(st.b_last), np64(st.x_last))
