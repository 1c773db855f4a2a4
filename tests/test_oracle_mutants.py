"""Each plausible mistake planted in a copy of the oracle's C source (a dropped
term, a wrong sign, a wrong index, a transposed operand) is caught by at least
one pin.  The mutants are built in a temporary directory; the committed oracle
is not touched."""
import functools
import os
import shutil
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "m3_oracle.c")

MUTANTS = {
    "drop_beta_term": [("h0r[p] = alpha * mh0 + beta * mu0 + gamma * u0[p];",
                        "h0r[p] = alpha * mh0 + gamma * u0[p];"),
                       ("h1r[p] = alpha * mh1 + beta * mu1 + gamma * u1[p];",
                        "h1r[p] = alpha * mh1 + gamma * u1[p];")],
    "beta_without_rotation": [("beta * mu0", "beta * u0p[p]"), ("beta * mu1", "beta * u1p[p]")],
    "beta_without_decay": [("const double beta = (1.0 - lv) * dtv * alpha;",
                            "const double beta = (1.0 - lv) * dtv;")],
    "gamma_without_lambda": [("const double gamma = lv * dtv;", "const double gamma = dtv;")],
    "lambda_swapped": [("const double beta = (1.0 - lv) * dtv * alpha;",
                        "const double beta = lv * dtv * alpha;"),
                       ("const double gamma = lv * dtv;", "const double gamma = (1.0 - lv) * dtv;")],
    "rotation_clockwise": [("const double mh0 = c * h0r[p] - s * h1r[p];",
                            "const double mh0 = c * h0r[p] + s * h1r[p];"),
                           ("const double mh1 = s * h0r[p] + c * h1r[p];",
                            "const double mh1 = -s * h0r[p] + c * h1r[p];"),
                           ("const double mu0 = c * u0p[p] - s * u1p[p];",
                            "const double mu0 = c * u0p[p] + s * u1p[p];"),
                           ("const double mu1 = s * u0p[p] + c * u1p[p];",
                            "const double mu1 = -s * u0p[p] + c * u1p[p];")],
    "pair_split_halves": [("double* h1r = hs + (2 * k + 1) * P;", "double* h1r = hs + (k + K) * P;"),
                          ("double* h0r = hs + (2 * k) * P;", "double* h0r = hs + (k) * P;")],
    "angle_of_wrong_group": [("const double th = theta[((b * L + t) * G + g) * K + k];",
                              "const double th = theta[((b * L + t) * G + (h % G)) * K + k];")],
    "decay_of_wrong_head": [("const double a_th = a_per_token ? A[(b * L + t) * H + h] : A[h];\n"
                             "        const double alpha = exp(dtv * a_th);",
                             "const double a_th = a_per_token ? A[(b * L + t) * H + h] : A[g];\n"
                             "        const double alpha = exp(dtv * a_th);")],
    "C_transposed_rank": [("acc += C[IDX5(b, t, g, r, n, L, G, R, N)] * hs[n * P + p];",
                           "acc += C[IDX5(b, t, g, (n % R), (r * (N / R) + n / R) % N, L, G, R, N)] * hs[n * P + p];")],
    "B_read_for_C": [("acc += C[IDX5(b, t, g, r, n, L, G, R, N)] * hs[n * P + p];",
                      "acc += B[IDX5(b, t, g, r, n, L, G, R, N)] * hs[n * P + p];")],
    "carry_ignored": [("if (b_last && x_last)", "if (0)")],
    "skip_term_dropped": [("y[xi] = acc + D[h] * x[xi];", "y[xi] = acc;")],
}


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="m3o_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor missing for {name}: {old}"
        src = src.replace(old, new)
    path = os.path.join(tmpdir_mod, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.build(force=True, src=path, out=os.path.join(tmpdir_mod, f"lib{name}.so"))
    scan = functools.partial(oracle.scan, lib_path=lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            ok, _ = pin(scan)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
