"""Pins for the oracle's reduced-precision state (a state stored in bf16 between
steps): the rounding itself against torch's fp32 -> bf16 conversion (an
independent implementation of round-to-nearest-even), and the rounded scan
against the plain scan and against the splitting of a sequence into a prefill
and single-token steps."""
import numpy as np
import torch

import oracle
from pins import _args, rand_case, rand_state


def _torch_bf16(v):
    return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000)),
        # exact ties between two bf16 neighbours (the 9th significant bit set alone)
        (1.0 + (2 * rng.integers(0, 128, 200) + 1) / 256.0) * 2.0 ** rng.integers(-20, 20, 200),
        np.array([0.0, -0.0, 1e-40, -3e-39, 3.3e38, -1.5e-45, 2.0 ** -126, 1.0 - 2.0 ** -24]),
    ]).astype(np.float32).astype(np.float64)      # inputs exact in fp32, as the GPU's
    got = np.array([oracle.round_bf16(x) for x in v])
    np.testing.assert_array_equal(got, _torch_bf16(v))


def test_no_rounding_flags_is_the_plain_scan():
    d = rand_case(b=1, L=9, H=2, G=1, P=3, N=4, R=2, seed=11)
    y0, h0 = oracle.scan(*_args(d))
    y1, h1 = oracle.scan(*_args(d), round_after=np.zeros(9, bool))
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)


def test_rounded_state_is_bf16_and_outputs_read_the_unrounded_state():
    d = rand_case(b=2, L=1, H=2, G=1, P=3, N=4, R=2, seed=12)
    st = rand_state(d, seed=3)
    y0, h0 = oracle.scan(*_args(d), state_in=st)
    y1, h1 = oracle.scan(*_args(d), state_in=st, round_after=np.ones(1, bool))
    np.testing.assert_array_equal(y1, y0)                 # Y_t from the unrounded h_t
    np.testing.assert_array_equal(h1, _torch_bf16(h0))    # h_t stored rounded
    assert not np.array_equal(h1, h0)


def test_rounding_every_token_changes_later_outputs():
    d = rand_case(b=1, L=12, H=2, G=1, P=4, N=6, R=1, seed=13)
    y0, _ = oracle.scan(*_args(d))
    y1, h1 = oracle.scan(*_args(d), round_after=np.ones(12, bool))
    np.testing.assert_array_equal(y1[:, 0], y0[:, 0])     # token 0 reads an unrounded state
    assert not np.array_equal(y1[:, 1:], y0[:, 1:])
    rel = np.max(np.abs(y1 - y0)) / np.max(np.abs(y0))
    assert rel < 2e-2                                      # bf16-sized perturbations only
    np.testing.assert_array_equal(h1, _torch_bf16(h1))


def test_prefill_then_rounded_steps_is_one_rounded_scan():
    """A prefill that stores its final state in bf16 followed by decode steps that
    read and write a bf16 state, as separate calls, equals one scan whose flags
    mark the prefill's last token and every later token."""
    L1, L = 7, 12
    d = rand_case(b=2, L=L, H=4, G=2, P=3, N=4, R=2, seed=14)
    flags = np.zeros(L, bool)
    flags[L1 - 1:] = True
    y_all, h_all = oracle.scan(*_args(d), round_after=flags)

    cut = lambda a, s: a[:, s] if a.ndim > 1 else a
    d1 = {k: cut(v, slice(0, L1)) for k, v in d.items()}
    f1 = np.zeros(L1, bool)
    f1[-1] = True
    y_parts, (h, bl, xl) = [], (None, None, None)
    y1, h = oracle.scan(*_args(d1), round_after=f1)
    y_parts.append(y1)
    bl, xl = d["B"][:, L1 - 1], d["x"][:, L1 - 1]
    for t in range(L1, L):
        dt_ = {k: cut(v, slice(t, t + 1)) for k, v in d.items()}
        yt, h = oracle.scan(*_args(dt_), state_in=(h, bl, xl), round_after=np.ones(1, bool))
        y_parts.append(yt)
        bl, xl = d["B"][:, t], d["x"][:, t]
    np.testing.assert_allclose(np.concatenate(y_parts, axis=1), y_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(h, h_all, rtol=0, atol=1e-13)
