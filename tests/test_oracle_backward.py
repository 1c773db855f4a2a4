"""Pins for the oracle's backward pass (oracle.scan_backward): its gradients
against central finite differences of the forward oracle (oracle.scan, itself
pinned by tests/test_oracle_pins.py), input by input, along random directions
and element by element; the empty sequence; head sums over groups; and a set
of plausible mistakes planted in a copy of the C source, each of which the
finite-difference pin must catch."""
import functools
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
from pins import _args, rand_case, rand_state

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")


def _objective(scan, d, st, dy, dho):
    y, h = scan(*[d[k] for k in NAMES], state_in=st)
    return float(np.sum(dy * y) + np.sum(dho * h))


def fd_check(scan, scan_backward, seed=0, b=2, L=7, H=4, G=2, P=3, N=4, R=2, eps=1e-6, with_state=True,
             a_per_token=False):
    """Largest relative mismatch between <grad, v> and the central difference of the
    objective along v, over every input (and the state, when given) and 3 random v each.
    With a_per_token, A is a per-token decay rate (b, L, H) drawn like the per-head one."""
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=seed, theta_scale=2.0)
    rng = np.random.default_rng(seed + 100)
    if a_per_token:
        d["A"] = -np.exp(rng.uniform(0.0, np.log(16.0), (b, L, H)))
    st = rand_state(d, seed=seed + 1) if with_state else None
    dy = rng.standard_normal(d["x"].shape)
    dho = rng.standard_normal((b, H, N, P))
    gr = scan_backward(*[d[k] for k in NAMES], dy, dh_out=dho, state_in=st)
    worst = 0.0
    targets = list(NAMES) + (["h0", "b_last", "x_last"] if with_state else [])
    gkey = {"h0": "dh0", "b_last": "db_last", "x_last": "dx_last"}
    for name in targets:
        for _ in range(3):
            if name in NAMES:
                base = d[name]
            else:
                base = st[("h0", "b_last", "x_last").index(name)]
            v = rng.standard_normal(base.shape)

            def shifted(sgn):
                d2 = dict(d)
                st2 = st
                if name in NAMES:
                    d2[name] = base + sgn * eps * v
                else:
                    s = list(st)
                    s[("h0", "b_last", "x_last").index(name)] = base + sgn * eps * v
                    st2 = tuple(s)
                return _objective(scan, d2, st2, dy, dho)

            fd = (shifted(+1) - shifted(-1)) / (2 * eps)
            an = float(np.sum(gr[gkey.get(name, "d" + name)] * v))
            worst = max(worst, abs(fd - an) / max(abs(fd), abs(an), 1e-3))
    return worst


def test_gradients_match_finite_differences():
    e = fd_check(oracle.scan, oracle.scan_backward, seed=3)
    assert e < 1e-6, e


def test_gradients_without_state_and_siso():
    e = fd_check(oracle.scan, oracle.scan_backward, seed=4, R=1, G=1, H=2, with_state=False)
    assert e < 1e-6, e


def test_elementwise_gradients_of_a_few_entries():
    """Single entries (not only random directions): one per input."""
    d = rand_case(b=1, L=5, H=2, G=1, P=2, N=4, R=2, seed=9, theta_scale=2.0)
    rng = np.random.default_rng(5)
    dy = rng.standard_normal(d["x"].shape)
    dho = np.zeros((1, 2, 4, 2))
    gr = oracle.scan_backward(*_args(d), dy, dh_out=dho)
    eps = 1e-6
    for name in NAMES:
        idx = tuple(int(rng.integers(s)) for s in d[name].shape)
        def f(sgn):
            d2 = dict(d)
            a = d[name].copy()
            a[idx] += sgn * eps
            d2[name] = a
            return _objective(oracle.scan, d2, None, dy, dho)
        fd = (f(+1) - f(-1)) / (2 * eps)
        an = gr["d" + name][idx]
        assert abs(fd - an) <= 1e-6 * max(abs(fd), 1e-3), (name, idx, fd, an)


def test_empty_sequence_passes_the_state_gradient_through():
    d = rand_case(b=1, L=0, H=2, G=1, P=2, N=4, R=1, seed=2)
    st = rand_state(d, seed=3)
    dho = np.random.default_rng(1).standard_normal((1, 2, 4, 2))
    gr = oracle.scan_backward(*_args(d), np.zeros(d["x"].shape), dh_out=dho, state_in=st)
    np.testing.assert_array_equal(gr["dh0"], dho)
    assert np.all(gr["db_last"] == 0) and np.all(gr["dx_last"] == 0)
    assert np.all(gr["dA"] == 0) and np.all(gr["dD"] == 0)


def test_group_gradients_sum_over_heads():
    """With G groups, dB/dC/dtheta of a group are the sums of its heads' gradients:
    the same inputs with B, C, theta repeated per head (G = H) give per-head
    gradients whose group sums equal the grouped result."""
    b, L, H, G, P, N, R = 1, 6, 4, 2, 3, 4, 2
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=11)
    rng = np.random.default_rng(2)
    dy = rng.standard_normal(d["x"].shape)
    gr = oracle.scan_backward(*_args(d), dy)
    rep = {k: (np.repeat(d[k], H // G, axis=2) if k in ("B", "C", "theta") else d[k]) for k in NAMES}
    gh = oracle.scan_backward(*[rep[k] for k in NAMES], dy)
    for k in ("dB", "dC", "dtheta"):
        s = gh[k].reshape(gh[k].shape[:2] + (G, H // G) + gh[k].shape[3:]).sum(axis=3)
        np.testing.assert_allclose(gr[k], s, rtol=1e-12, atol=1e-12)
    for k in ("dx", "ddt", "dlam", "dA", "dD"):
        np.testing.assert_allclose(gr[k], gh[k], rtol=1e-12, atol=1e-12)


SRC = os.path.join(os.path.dirname(oracle.__file__), "m3_oracle.c")

# Plausible mistakes in the backward pass only (the forward is left intact).
BWD_MUTANTS = {
    "dU_drops_next_beta_term": [("dU[i] = gamma * g[i] + beta_next * qn[i];", "dU[i] = gamma * g[i];")],
    "adjoint_without_rotation": [("const double q0 = c * g0 + s * g1, q1 = -s * g0 + c * g1;",
                                  "const double q0 = g0, q1 = g1;")],
    "adjoint_rotated_forward": [("const double q0 = c * g0 + s * g1, q1 = -s * g0 + c * g1;",
                                 "const double q0 = c * g0 - s * g1, q1 = s * g0 + c * g1;")],
    "dtheta_sign": [("dth += q1 * v0 - q0 * v1;", "dth += q0 * v1 - q1 * v0;")],
    "dtheta_without_beta_input": [("const double v0 = alpha * h0v + beta * u0, v1 = alpha * h1v + beta * u1;",
                                   "const double v0 = alpha * h0v, v1 = alpha * h1v;")],
    "dC_from_previous_state": [("a += ht[n * P + p] * dy[", "a += hp[n * P + p] * dy[")],
    "ddt_missing_decay_chain": [("dbe * (1.0 - lv) * (alpha + dtv * a_th * alpha)", "dbe * (1.0 - lv) * alpha")],
    "dlam_sign": [("dlam[(b * L + t) * H + h] = -dbe * dtv * alpha + dgam * dtv;",
                   "dlam[(b * L + t) * H + h] = dbe * dtv * alpha + dgam * dtv;")],
    "dA_drops_beta_path": [("const double dA_t = dal * dtv * alpha + dbe * (1.0 - lv) * dtv * dtv * alpha;",
                            "const double dA_t = dal * dtv * alpha;")],
    "skip_gradient_dropped": [("dx[xi] = D[h] * dy[xi];", "dx[xi] = 0.0;")],
    "carry_gradient_without_beta": [("for (int64_t i = 0; i < NP; ++i) dU[i] = beta_next * qn[i];",
                                     "for (int64_t i = 0; i < NP; ++i) dU[i] = qn[i];")],
}


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="m3o_bmut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", list(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, tmpdir_mod):
    src = open(SRC).read()
    for old, new in BWD_MUTANTS[name]:
        assert src.count(old) == 1, f"mutation anchor missing or repeated for {name}: {old}"
        src = src.replace(old, new)
    path = os.path.join(tmpdir_mod, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.build(force=True, src=path, out=os.path.join(tmpdir_mod, f"lib{name}.so"))
    bwd = functools.partial(oracle.scan_backward, lib_path=lib)
    e = fd_check(oracle.scan, bwd, seed=3)
    assert e > 1e-4, f"mutant {name} passed the finite-difference pin ({e:.2e})"


def test_per_token_A_gradients_match_finite_differences():
    """A per-token decay rate A_t (the discretisation's A_t): every gradient, dA per token
    included, against central differences of the forward oracle run with the same A_t."""
    assert fd_check(oracle.scan, oracle.scan_backward, seed=6, a_per_token=True) < 1e-6
    assert fd_check(oracle.scan, oracle.scan_backward, seed=7, R=1, G=1, H=2, with_state=False,
                    a_per_token=True) < 1e-6


def test_per_token_A_constant_over_tokens_matches_per_head():
    """A_t equal to A[h] at every token: the same gradients, and dA_t summed over batch and
    tokens is the per-head dA."""
    b, L, H, G, P, N, R = 2, 6, 4, 2, 3, 4, 2
    d = rand_case(b=b, L=L, H=H, G=G, P=P, N=N, R=R, seed=12, theta_scale=2.0)
    st = rand_state(d, seed=13)
    rng = np.random.default_rng(3)
    dy = rng.standard_normal(d["x"].shape)
    dho = rng.standard_normal((b, H, N, P))
    g1 = oracle.scan_backward(*_args(d), dy, dh_out=dho, state_in=st)
    dt_ = dict(d)
    dt_["A"] = np.broadcast_to(d["A"], (b, L, H)).copy()
    g2 = oracle.scan_backward(*[dt_[k] for k in NAMES], dy, dh_out=dho, state_in=st)
    for k in ("dx", "ddt", "dlam", "dtheta", "dB", "dC", "dD", "dh0", "db_last", "dx_last"):
        np.testing.assert_allclose(g2[k], g1[k], rtol=1e-12, atol=1e-12)
    assert g2["dA"].shape == (b, L, H)
    np.testing.assert_allclose(g2["dA"].sum(axis=(0, 1)), g1["dA"], rtol=1e-12, atol=1e-12)


def test_per_token_A_mutant_is_caught(tmpdir_mod):
    """A reverse sweep that reads the per-head slot of A instead of the token's rate."""
    src = open(SRC).read()
    old = ("const double a_th = a_per_token ? A[(b * L + t) * H + h] : A[h];\n"
           "            const double alpha = exp(dtv * a_th), beta = (1.0 - lv) * dtv * alpha, gamma = lv * dtv;\n"
           "            const double* ht = hall + (t + 1) * NP;")
    assert src.count(old) == 1
    src = src.replace(old, old.replace("a_per_token ? A[(b * L + t) * H + h] : A[h]", "A[h]"))
    path = os.path.join(tmpdir_mod, "a_tok.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.build(force=True, src=path, out=os.path.join(tmpdir_mod, "liba_tok.so"))
    bwd = functools.partial(oracle.scan_backward, lib_path=lib)
    assert fd_check(oracle.scan, bwd, seed=6, a_per_token=True) > 1e-4
