"""GPU parity of the fused prologue/epilogue (m3_prefill_fused, m3_decode_step_fused)
against the oracle's scan_fused: per-token A, RMSNorm of B and C with weights, their
biases, and the output gate -- together and one at a time, on the matrix-core and the
generic prefill paths, from a state with a (raw) carried B, and a fused prefill
continued by fused decode steps."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, draw, np64, onorm_slice_errs, rand_state, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")


def _fusion(b, L, H, R, N, P, io, seed, parts):
    g = torch.Generator(device="cpu").manual_seed(seed)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    f = {}
    if "A_t" in parts:
        f["A_t"] = (-torch.exp(torch.rand((b, L, H), generator=g) * np.log(16.0))).cuda()
    if "norm" in parts:
        f["b_norm_w"] = (1.0 + 0.3 * torch.randn((R, N), generator=g)).cuda()
        f["c_norm_w"] = (1.0 + 0.3 * torch.randn((R, N), generator=g)).cuda()
    if "bias" in parts:
        f["b_bias"] = (0.02 + 0.05 * torch.randn((R, N), generator=g)).cuda()
        f["c_bias"] = (0.02 + 0.05 * torch.randn((R, N), generator=g)).cuda()
    if "gate" in parts:
        f["z"] = torch.randn((b, L, H, R, P), generator=g).to(tdt).cuda()
    if "onorm" in parts:
        f["out_norm_w"] = (1.0 + 0.3 * torch.randn((H, P), generator=g)).cuda()
    return f


def _theta_per_group(d, Gt, seed, scale=1.0):
    """Replace the angles by Gt angle groups (b, L, Gt, N/2): angles per head over shared B, C."""
    b, L, _, KP = d["theta"].shape
    g = torch.Generator(device="cpu").manual_seed(seed)
    d = dict(d)
    d["theta"] = ((torch.rand((b, L, Gt, KP), generator=g) * 2 - 1) * np.pi * scale).cuda()
    return d


def _oracle(d, f, state_in=None):
    kw = {k: np64(v) for k, v in f.items() if k != "A_t"}
    args = [np64(d[k]) for k in NAMES]
    if "A_t" in f:
        args[2] = np64(f["A_t"])
    return oracle.scan_fused(*args, **kw, state_in=state_in)


CASES = [
    # b, L, H, G, P, N, R, Q, io, parts
    (2, 100, 4, 2, 64, 128, 2, 32, "bf16", ("A_t", "norm", "bias", "gate")),   # matrix cores
    (1, 70, 2, 1, 64, 128, 4, 64, "bf16", ("norm",)),
    (1, 70, 2, 1, 64, 128, 4, 64, "bf16", ("bias",)),
    (1, 70, 2, 1, 64, 128, 1, 64, "bf16", ("gate",)),
    (1, 70, 2, 1, 64, 128, 1, 64, "bf16", ("A_t",)),
    (1, 90, 2, 1, 64, 128, 4, 32, "bf16", ("A_t", "norm", "bias", "gate")),    # chunks of 128 rows
    (2, 150, 4, 2, 64, 128, 2, 64, "bf16", ("gate",)),
    (2, 45, 4, 2, 16, 16, 2, 16, "fp32", ("A_t", "norm", "bias", "gate")),      # generic path
]


def _id(c):
    return "b{}L{}H{}G{}P{}N{}R{}Q{}-{}-{}".format(*c[:9], "+".join(c[9]))


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_prefill_fused_matches_oracle(case):
    b, L, H, G, P, N, R, Q, io, parts = case
    say("prefill fused", _id(case))
    d = draw(b, L, H, G, P, N, R, io, 1.0, seed=L + R)
    f = _fusion(b, L, H, R, N, P, io, seed=7, parts=parts)
    st = rand_state(b, H, G, N, P, R, io, seed=3)
    y, so = m3scan.prefill_fused(*[d[k] for k in NAMES], Q, **f, state_in=st)
    torch.cuda.synchronize()
    yr, hr = _oracle(d, f, state_in=(np64(st.h), np64(st.b_last), np64(st.x_last)))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(so.h), hr, 1)
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]
    # the carry written is the raw last token
    assert torch.equal(so.b_last, d["B"][:, -1]) and torch.equal(so.x_last, d["x"][:, -1])


@pytest.mark.parametrize("R", [2, 4])
def test_fused_prefill_then_fused_decode(R):
    b, L, H, G, P, N, Q, steps = 2, 64, 4, 1, 64, 128, 32, 5
    say("fused prefill + decode", R)
    d = draw(b, L + steps, H, G, P, N, R, "bf16", 1.0, seed=40 + R)
    f = _fusion(b, L + steps, H, R, N, P, "bf16", seed=9, parts=("A_t", "norm", "bias", "gate"))
    cut = lambda t, s: t[:, s].contiguous() if t.dim() > 1 else t
    pre = {k: cut(v, slice(0, L)) for k, v in d.items()}
    fpre = {k: (cut(v, slice(0, L)) if k in ("A_t", "z") else v) for k, v in f.items()}
    y, st = m3scan.prefill_fused(*[pre[k] for k in NAMES], Q, **fpre)
    ys = [y]
    for t in range(L, L + steps):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ft = {k: (v[:, t].contiguous() if k in ("A_t", "z") else v) for k, v in f.items()}
        ys.append(m3scan.decode_step_fused(st, *[tok[k] for k in NAMES], **ft)[:, None])
    torch.cuda.synchronize()
    yr, hr = _oracle(d, f)
    ey = slice_err(np64(torch.cat(ys, dim=1)), yr, 2)
    eh = slice_err(np64(st.h), hr, 1)
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_fused_without_parts_is_the_plain_prefill():
    """An empty fusion gives bit-identical results to m3_prefill_chunked."""
    b, L, H, G, P, N, R, Q = 1, 80, 2, 1, 64, 128, 2, 32
    d = draw(b, L, H, G, P, N, R, "bf16", 1.0, seed=5)
    y0, s0 = m3scan.prefill(*[d[k] for k in NAMES], Q)
    y1, s1 = m3scan.prefill_fused(*[d[k] for k in NAMES], Q)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(s0.h, s1.h)


# (lengths, H, G, P, N, R, Q, io): packed batches with every fused piece
VARLEN_CASES = [
    ([130, 0, 64, 17, 300, 1], 4, 2, 64, 128, 2, 32, "bf16"),    # matrix cores
    ([100, 0, 37, 64, 5], 4, 2, 16, 16, 2, 16, "fp32"),           # generic path
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "L{}-R{}-{}".format("_".join(map(str, c[0])), c[5], c[7]))
def test_prefill_varlen_fused_each_sequence_matches_oracle(case):
    """m3_prefill_varlen_fused: each sequence of the pack against oracle.scan_fused run on it
    alone, from its own state slice with a raw carried B (normalised by the call)."""
    lengths, H, G, P, N, R, Q, io = case
    ns, T = len(lengths), int(sum(lengths))
    say("prefill varlen fused", lengths, io)
    d = draw(1, T, H, G, P, N, R, io, 1.0, seed=T + R)
    d = {k: (v[0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    f = _fusion(1, T, H, R, N, P, io, seed=11, parts=("A_t", "norm", "bias", "gate"))
    f = {k: (v[0].contiguous() if k in ("A_t", "z") else v) for k, v in f.items()}
    st = rand_state(ns, H, G, N, P, R, io, seed=13)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    y, so = m3scan.prefill_varlen_fused(*[d[k] for k in NAMES], cu, max(lengths), Q, **f, state_in=st)
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    for s, n in enumerate(lengths):
        if n == 0:   # nothing scanned: the state and the raw carry pass through
            assert torch.equal(so.h[s], st.h[s])
            assert torch.equal(so.b_last[s], st.b_last[s]) and torch.equal(so.x_last[s], st.x_last[s])
            continue
        ds = {k: (v[c[s]:c[s + 1]][None] if v.dim() > 1 else v) for k, v in d.items()}
        fs = {k: (v[c[s]:c[s + 1]][None] if k in ("A_t", "z") else v) for k, v in f.items()}
        yr, hr = _oracle(ds, fs, state_in=(np64(st.h[s:s + 1]), np64(st.b_last[s:s + 1]), np64(st.x_last[s:s + 1])))
        ey = slice_err(np64(y[c[s]:c[s + 1]])[None], yr, 2)
        eh = slice_err(np64(so.h[s:s + 1]), hr, 1)
        say(f"  seq {s} (len {n}): y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL[io] and eh <= TOL[io], (s, ey, eh)
        assert torch.equal(so.b_last[s], d["B"][c[s + 1] - 1]) and torch.equal(so.x_last[s], d["x"][c[s + 1] - 1])


@pytest.mark.parametrize("parts", [("gate",), ("A_t",), ("norm",), ("bias",), ("A_t", "norm", "bias", "gate")],
                         ids=lambda p: "+".join(p))
@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_fused_decode_steps_match_oracle(parts, state):
    """Three fused decode steps from a random state with a raw carried B, one fused piece at a
    time and all together (the decode kernel has a variant for norm, bias or gate, and reads
    a per-token A in both); fp32 and bf16 state (the latter against the oracle rounded
    after every token)."""
    b, H, G, P, N, R, steps = 2, 8, 2, 64, 128, 4, 3
    say("fused decode", "+".join(parts), state)
    d = draw(b, steps, H, G, P, N, R, "bf16", 1.0, seed=70 + len(parts))
    f = _fusion(b, steps, H, R, N, P, "bf16", seed=12, parts=parts)
    st = rand_state(b, H, G, N, P, R, "bf16", seed=14)
    if state == "bf16":
        st = m3scan.DecodeState(st.h.to(torch.bfloat16), st.b_last, st.x_last)
    st0 = (np64(st.h), np64(st.b_last), np64(st.x_last))
    ys = []
    for t in range(steps):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ft = {k: (v[:, t].contiguous() if k in ("A_t", "z") else v) for k, v in f.items()}
        ys.append(m3scan.decode_step_fused(st, *[tok[k] for k in NAMES], **ft)[:, None])
    torch.cuda.synchronize()
    kw = {k: np64(v) for k, v in f.items() if k != "A_t"}
    args = [np64(d[k]) for k in NAMES]
    if "A_t" in f:
        args[2] = np64(f["A_t"])
    yr, hr = oracle.scan_fused(*args, **kw, state_in=st0,
                               round_after=np.ones(steps, bool) if state == "bf16" else None)
    ey = slice_err(np64(torch.cat(ys, dim=1)), yr, 2)
    eh = slice_err(np64(st.h), hr, 1)
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("carry", [True, False], ids=["carried_B", "no_carry"])
def test_fused_decode_generic_shape_matches_oracle(carry):
    """The decode kernel for shapes other than N=128, P=64 (decode_generic) with every fused
    piece together: per-token A, BCNorm of B and C (its row sums of squares in one wave of
    64 lanes), biases and the gate, fp32 io, four steps from a random state, with and
    without a carried previous B."""
    b, H, G, P, N, R, steps = 2, 6, 3, 12, 24, 3, 4
    say("fused decode, generic shape", "carry" if carry else "no carry")
    d = draw(b, steps, H, G, P, N, R, "fp32", 1.0, seed=91)
    f = _fusion(b, steps, H, R, N, P, "fp32", seed=15, parts=("A_t", "norm", "bias", "gate"))
    st = rand_state(b, H, G, N, P, R, "fp32", seed=16)
    if not carry:
        st = m3scan.DecodeState(st.h, None, None)
    st0 = (np64(st.h), np64(st.b_last), np64(st.x_last)) if carry else (np64(st.h), None, None)
    ys = []
    for t in range(steps):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ft = {k: (v[:, t].contiguous() if k in ("A_t", "z") else v) for k, v in f.items()}
        ys.append(m3scan.decode_step_fused(st, *[tok[k] for k in NAMES], **ft)[:, None])
    torch.cuda.synchronize()
    kw = {k: np64(v) for k, v in f.items() if k != "A_t"}
    args = [np64(d[k]) for k in NAMES]
    args[2] = np64(f["A_t"])
    yr, hr = oracle.scan_fused(*args, **kw, state_in=st0)
    ey = slice_err(np64(torch.cat(ys, dim=1)), yr, 2)
    eh = slice_err(np64(st.h), hr, 1)
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL["fp32"] and eh <= TOL["fp32"]



# b, L, H, G, Gt, P, N, R, Q, io, parts: angles per head (Gt = H) or per finer group (G < Gt < H),
# and the output norm, alone and with every other piece
THETA_ONORM_CASES = [
    (2, 100, 4, 1, 4, 64, 128, 2, 32, "bf16", ("onorm",)),                          # matrix cores
    (2, 130, 8, 2, 4, 64, 128, 4, 64, "bf16", ("theta",)),
    (1, 200, 4, 1, 4, 64, 128, 1, 64, "bf16", ("theta", "onorm")),
    (2, 100, 8, 2, 8, 64, 128, 2, 32, "bf16", ("A_t", "norm", "bias", "gate", "theta", "onorm")),
    (2, 100, 4, 1, 4, 64, 128, 4, 32, "bf16", ("A_t", "norm", "bias", "gate", "theta", "onorm")),
    (1, 150, 4, 2, 4, 64, 128, 2, 64, "bf16", ("onorm",)),
    (2, 45, 4, 2, 4, 16, 16, 2, 16, "fp32", ("onorm",)),                             # generic path
    (2, 45, 6, 1, 6, 16, 16, 2, 16, "fp32", ("A_t", "norm", "bias", "gate", "theta", "onorm")),
]


def _tid(c):
    return "b{}L{}H{}G{}Gt{}P{}N{}R{}Q{}-{}-{}".format(*c[:10], "+".join(c[10]))


@pytest.mark.parametrize("case", THETA_ONORM_CASES, ids=_tid)
def test_prefill_theta_groups_and_out_norm_match_oracle(case):
    b, L, H, G, Gt, P, N, R, Q, io, parts = case
    say("prefill fused", _tid(case))
    d = draw(b, L, H, G, P, N, R, io, 1.0, seed=L + H)
    if "theta" in parts:
        d = _theta_per_group(d, Gt, seed=L)
    f = _fusion(b, L, H, R, N, P, io, seed=17, parts=parts)
    st = rand_state(b, H, G, N, P, R, io, seed=18)
    y, so = m3scan.prefill_fused(*[d[k] for k in NAMES], Q, **f, state_in=st)
    torch.cuda.synchronize()
    ey, eh = _fused_errs(y, so.h, d, f, state_in=(np64(st.h), np64(st.b_last), np64(st.x_last)))
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]
    assert torch.equal(so.b_last, d["B"][:, -1]) and torch.equal(so.x_last, d["x"][:, -1])


def _fused_errs(y, h, d, f, state_in=None, y_axis=2):
    """(y error, state error) against the oracle; with the output norm, y is held to the bar
    on the scale of the rows before the norm (gpu_util.onorm_slice_errs)."""
    if "out_norm_w" not in f:
        yr, hr = _oracle(d, f, state_in=state_in)
        return slice_err(np64(y), yr, y_axis), slice_err(np64(h), hr, 1)
    fpre = {k: v for k, v in f.items() if k != "out_norm_w"}
    ypre, hr = _oracle(d, fpre, state_in=state_in)
    per, _ = onorm_slice_errs(np64(y), ypre, np64(f["out_norm_w"]), 1e-6)
    return float(np.max(per)), slice_err(np64(h), hr, 1)


def test_theta_groups_equal_within_a_group_is_the_grouped_prefill():
    """Angle groups finer than the B/C groups (Gt = 4 over G = 2, two heads per angle group)
    that repeat each B/C group's angles give bit for bit the plain grouped prefill: the same
    operands are prepared once per angle group instead of once per B/C group."""
    b, L, H, G, Gt, P, N, R, Q = 2, 150, 8, 2, 4, 64, 128, 4, 64
    d = draw(b, L, H, G, P, N, R, "bf16", 1.0, seed=55)
    y0, s0 = m3scan.prefill(*[d[k] for k in NAMES], Q)
    d1 = dict(d)
    d1["theta"] = d["theta"].repeat_interleave(Gt // G, dim=2).contiguous()
    y1, s1 = m3scan.prefill_fused(*[d1[k] for k in NAMES], Q)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(s0.h, s1.h)


@pytest.mark.parametrize("shape", [(8, 2, 64, 128, 4), (6, 3, 12, 24, 3)], ids=["fast", "generic"])
def test_fused_prefill_then_decode_theta_per_head_out_norm(shape):
    """A fused prefill continued by fused decode steps, with angles per head and the output
    norm (and every other piece), equals one oracle scan: the decode kernels read the head's
    angle group and normalise each output row."""
    H, G, P, N, R = shape
    b, L, steps = 2, 70, 4
    io = "bf16" if N == 128 else "fp32"
    Q = 32 if io == "bf16" else 16
    say("fused prefill + decode, angles per head, output norm", shape)
    d = _theta_per_group(draw(b, L + steps, H, G, P, N, R, io, 1.0, seed=66), H, seed=67)
    f = _fusion(b, L + steps, H, R, N, P, io, seed=19, parts=("A_t", "norm", "bias", "gate", "onorm"))
    cut = lambda t, s: t[:, s].contiguous() if t.dim() > 1 else t
    per_tok = ("A_t", "z")
    y, st = m3scan.prefill_fused(*[cut(d[k], slice(0, L)) for k in NAMES], Q,
                                 **{k: (cut(v, slice(0, L)) if k in per_tok else v) for k, v in f.items()})
    ys = [y]
    for t in range(L, L + steps):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ft = {k: (v[:, t].contiguous() if k in per_tok else v) for k, v in f.items()}
        ys.append(m3scan.decode_step_fused(st, *[tok[k] for k in NAMES], **ft)[:, None])
    torch.cuda.synchronize()
    ey, eh = _fused_errs(torch.cat(ys, dim=1), st.h, d, f)
    say(f"  y {ey:.2e} h {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]


def test_prefill_varlen_fused_theta_per_head_out_norm():
    lengths, H, G, P, N, R, Q = [130, 0, 64, 17, 300, 1], 4, 1, 64, 128, 2, 32
    T = int(sum(lengths))
    say("prefill varlen fused, angles per head, output norm")
    d = _theta_per_group(draw(1, T, H, G, P, N, R, "bf16", 1.0, seed=T), H, seed=T + 1)
    d = {k: (v[0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    f = _fusion(1, T, H, R, N, P, "bf16", seed=21, parts=("A_t", "norm", "bias", "gate", "onorm"))
    f = {k: (v[0].contiguous() if k in ("A_t", "z") else v) for k, v in f.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    y, so = m3scan.prefill_varlen_fused(*[d[k] for k in NAMES], cu, max(lengths), Q, **f)
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lengths))
    for s_, n in enumerate(lengths):
        if n == 0:
            continue
        ds = {k: (v[c[s_]:c[s_ + 1]][None] if v.dim() > 1 else v) for k, v in d.items()}
        fs = {k: (v[c[s_]:c[s_ + 1]][None] if k in ("A_t", "z") else v) for k, v in f.items()}
        ey, eh = _fused_errs(y[c[s_]:c[s_ + 1]][None], so.h[s_:s_ + 1], ds, fs)
        say(f"  seq {s_} (len {n}): y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
