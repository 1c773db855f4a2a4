"""Pins for the oracle's fused prologue/epilogue (oracle.scan_fused and its parts):
BCNorm against torch's own RMSNorm, the gate against torch's SiLU, per-token A
against a per-head A held constant over tokens (identical) and against a chain of
single-token scans with per-head A set to that token's A_t (an independent path
through the forward pin), and the normalised carry of a split scan."""
import numpy as np
import torch

import oracle
from pins import _args, rand_case, rand_state

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")


def test_bc_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    M = rng.standard_normal((2, 5, 3, 2, 16)) * 3.0
    w = rng.standard_normal((2, 16))
    bias = rng.standard_normal((2, 16))
    got = oracle.bc_norm(M, w, bias, eps=1e-6)
    t = torch.tensor(M)
    ref = torch.stack([torch.nn.functional.rms_norm(t[:, :, :, r], (16,), torch.tensor(w[r]), eps=1e-6)
                       for r in range(2)], dim=3) + torch.tensor(bias)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-13)
    # bias only, and nothing
    np.testing.assert_array_equal(oracle.bc_norm(M, None, bias), M + bias)
    np.testing.assert_array_equal(oracle.bc_norm(M), M)


def test_gate_matches_torch_silu():
    rng = np.random.default_rng(2)
    y = rng.standard_normal(1000)
    z = rng.standard_normal(1000) * 6
    ref = y * torch.nn.functional.silu(torch.tensor(z)).numpy()
    np.testing.assert_allclose(oracle.gate(y, z), ref, rtol=1e-14, atol=1e-14)


def test_per_token_A_constant_over_tokens_is_the_per_head_scan():
    d = rand_case(b=2, L=9, H=4, G=2, P=3, N=4, R=2, seed=21)
    A_t = np.broadcast_to(d["A"][None, None, :], d["dt"].shape).copy()
    y0, h0 = oracle.scan(*_args(d))
    args = list(_args(d))
    args[2] = A_t
    y1, h1 = oracle.scan(*args)
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)


def test_per_token_A_is_a_chain_of_single_token_scans():
    b, L, H, G, P, N, R = 2, 7, 4, 2, 3, 4, 2
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=22)
    rng = np.random.default_rng(3)
    A_t = -np.exp(rng.uniform(0, np.log(16), size=(b, L, H)))
    st = rand_state(d, seed=4)
    args = list(_args(d))
    args[2] = A_t
    y_all, h_all = oracle.scan(*args, state_in=st)
    h, bl, xl = st
    ys = []
    for t in range(L):
        cut = {k: (v[:, t:t + 1] if v.ndim > 1 else v) for k, v in d.items()}
        outs = []
        # one call per batch element: the per-head A of token t differs by batch element
        for bi in range(b):
            cb = {k: (v[bi:bi + 1] if v.ndim > 1 else v) for k, v in cut.items()}
            cb["A"] = A_t[bi, t]
            yb, hb = oracle.scan(*[cb[k] for k in NAMES], state_in=(h[bi:bi + 1], bl[bi:bi + 1], xl[bi:bi + 1]))
            outs.append((yb, hb))
        ys.append(np.concatenate([o[0] for o in outs], axis=0))
        h = np.concatenate([o[1] for o in outs], axis=0)
        bl, xl = d["B"][:, t], d["x"][:, t]
    np.testing.assert_allclose(np.concatenate(ys, axis=1), y_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(h, h_all, rtol=0, atol=1e-13)


def test_fused_split_scan_normalises_the_carry():
    """A fused prefill followed by fused single-token steps (raw B carried, normalised in
    each step) equals one fused scan: the carried B goes through the same BCNorm."""
    b, L, H, G, P, N, R = 1, 6, 2, 1, 3, 4, 2
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=23)
    rng = np.random.default_rng(5)
    kw = dict(b_norm_w=rng.standard_normal((R, N)), c_norm_w=rng.standard_normal((R, N)),
              b_bias=rng.standard_normal((R, N)), c_bias=rng.standard_normal((R, N)),
              z=rng.standard_normal(d["x"].shape))
    y_all, h_all = oracle.scan_fused(*_args(d), **kw)
    L1 = 4
    cut = lambda v, s: v[:, s] if v.ndim > 1 else v
    d1 = {k: cut(v, slice(0, L1)) for k, v in d.items()}
    kw1 = dict(kw, z=kw["z"][:, :L1])
    y1, h = oracle.scan_fused(*_args(d1), **kw1)
    ys = [y1]
    bl, xl = d["B"][:, L1 - 1], d["x"][:, L1 - 1]
    for t in range(L1, L):
        dt_ = {k: cut(v, slice(t, t + 1)) for k, v in d.items()}
        yt, h = oracle.scan_fused(*_args(dt_), **dict(kw, z=kw["z"][:, t:t + 1]), state_in=(h, bl, xl))
        ys.append(yt)
        bl, xl = d["B"][:, t], d["x"][:, t]
    np.testing.assert_allclose(np.concatenate(ys, axis=1), y_all, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h, h_all, rtol=0, atol=1e-12)


def test_out_norm_matches_torch_rms_norm():
    """The output RMSNorm against torch's rms_norm over the last axis, head by head with
    that head's weight."""
    rng = np.random.default_rng(6)
    b, L, H, R, P = 2, 3, 4, 2, 8
    y = rng.standard_normal((b, L, H, R, P)) * 2.0
    w = rng.standard_normal((H, P))
    got = oracle.out_norm(y, w, eps=1e-5)
    t = torch.tensor(y)
    ref = torch.stack([torch.nn.functional.rms_norm(t[:, :, h], (P,), torch.tensor(w[h]), eps=1e-5)
                       for h in range(H)], dim=2)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_out_norm_follows_the_gate():
    """scan_fused applies the gate, then the norm: equal to out_norm(gate(y, z))."""
    d = rand_case(b=1, L=5, H=2, G=1, P=4, N=4, R=2, seed=24)
    rng = np.random.default_rng(7)
    z = rng.standard_normal(d["x"].shape)
    w = rng.standard_normal((2, 4))
    y0, _ = oracle.scan(*_args(d))
    y1, _ = oracle.scan_fused(*_args(d), z=z, out_norm_w=w, eps=1e-6)
    np.testing.assert_allclose(y1, oracle.out_norm(oracle.gate(y0, z), w, 1e-6), rtol=1e-14, atol=1e-14)


def test_theta_groups_equal_within_a_group_is_the_grouped_scan():
    """Angles per head that are equal over the heads of each B/C group reproduce the
    grouped scan bit for bit (state carried in, with a carry, included)."""
    b, L, H, G, P, N, R = 2, 7, 6, 2, 3, 6, 2
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=25)
    st = rand_state(d, seed=8)
    y0, h0 = oracle.scan_fused(*_args(d), state_in=st)
    args = list(_args(d))
    args[4] = np.repeat(d["theta"], H // G, axis=2)      # (b, L, H, N/2): each head its group's angles
    y1, h1 = oracle.scan_fused(*args, state_in=st)
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)


def test_theta_per_head_is_each_head_alone():
    """Distinct angles per head over shared B and C: every head equals a one-head scan with
    its own angles and its group's B and C (the head-to-group maps of both groupings)."""
    b, L, H, G, Gt, P, N, R = 2, 6, 8, 2, 4, 3, 4, 2
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=26)
    rng = np.random.default_rng(9)
    theta_t = rng.uniform(-np.pi, np.pi, size=(b, L, Gt, N // 2))
    st = rand_state(d, seed=10)
    args = list(_args(d))
    args[4] = theta_t
    y, hh = oracle.scan_fused(*args, state_in=st)
    for h in range(H):
        g, j = h // (H // G), h // (H // Gt)
        yh, hs = oracle.scan(d["x"][:, :, h:h + 1], d["dt"][:, :, h:h + 1], d["A"][h:h + 1],
                             d["lam"][:, :, h:h + 1], theta_t[:, :, j:j + 1], d["B"][:, :, g:g + 1],
                             d["C"][:, :, g:g + 1], d["D"][h:h + 1],
                             state_in=(st[0][:, h:h + 1], st[1][:, g:g + 1], st[2][:, h:h + 1]))
        np.testing.assert_allclose(y[:, :, h:h + 1], yh, rtol=0, atol=1e-13)
        np.testing.assert_allclose(hh[:, h:h + 1], hs, rtol=0, atol=1e-13)
