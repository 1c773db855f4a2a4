"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_util import (TOL, draw, gpu_prefill, np64, oracle_args, oracle_state, rand_state, say,
                      slice_err)
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

# (b, L, H, G, P, N, R, Q, io, theta_scale)
PREFILL_CASES = [
    (1, 256, 4, 1, 16, 16, 1, 32, "fp32", 1.0),     # the single-SISO-layer fp32 workload itself
    (2, 37, 4, 2, 8, 16, 3, 8, "fp32", 1.0),        # ragged last chunk, 2 groups, R=3
    (2, 50, 6, 3, 12, 10, 2, 7, "fp32", 4.0),       # odd chunk, N/2 odd, strong rotation
    (1, 5, 2, 2, 4, 4, 1, 16, "fp32", 1.0),         # L shorter than one chunk
    (1, 100, 2, 1, 64, 128, 2, 32, "bf16", 1.0),    # nanomamba3 head shape, ragged
    (2, 130, 2, 1, 64, 128, 1, 64, "bf16", 1.0),    # 1.5B SISO head shape, ragged
    (1, 96, 4, 4, 32, 64, 2, 16, "bf16", 4.0),      # G = H
]


def _ids(c):
    return "b{}L{}H{}G{}P{}N{}R{}Q{}-{}-th{}".format(*c)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=_ids)
def test_prefill_matches_oracle(case):
    b, L, H, G, P, N, R, Q, io, ts = case
    say("prefill case", _ids(case))
    d = draw(b, L, H, G, P, N, R, io, ts, seed=zlib.crc32(_ids(case).encode()) % 10000)
    y, st = gpu_prefill(d, Q)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d))
    ey = slice_err(np64(y), yr, 2)
    eh = slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]
    # the carry is the last token's B and X, bit for bit
    if L > 0:
        assert torch.equal(st.b_last, d["B"][:, -1]) and torch.equal(st.x_last, d["x"][:, -1])


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_prefill_from_state(io):
    b, L, H, G, P, N, R, Q = 2, 45, 4, 2, 16, 32, 2, 16
    say("prefill from state", io)
    d = draw(b, L, H, G, P, N, R, io, 2.0, seed=31)
    st0 = rand_state(b, H, G, N, P, R, io)
    y, st = gpu_prefill(d, Q, state_in=st0)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d), state_in=oracle_state(st0))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]


def test_prefill_empty_sequence_passes_state_through():
    b, H, G, P, N, R = 2, 4, 2, 8, 16, 2
    say("prefill L=0")
    d = draw(b, 0, H, G, P, N, R, "fp32")
    st0 = rand_state(b, H, G, N, P, R, "fp32")
    y, st = gpu_prefill(d, 16, state_in=st0)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(st.h, st0.h)
    assert torch.equal(st.b_last, st0.b_last) and torch.equal(st.x_last, st0.x_last)


# (b, H, G, P, N, R, io)
DECODE_CASES = [
    (3, 4, 2, 64, 128, 4, "bf16"),
    (2, 4, 1, 64, 128, 1, "fp32"),
    (2, 6, 3, 64, 128, 2, "bf16"),
    (2, 4, 4, 16, 16, 1, "fp32"),
    (2, 3, 1, 12, 24, 3, "fp32"),          # generic decode kernel
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "b{}H{}G{}P{}N{}R{}-{}".format(*c))
def test_decode_matches_oracle(case):
    b, H, G, P, N, R, io = case
    steps = 6
    say("decode case", case)
    st = rand_state(b, H, G, N, P, R, io, seed=7)
    ost = oracle_state(st)
    d = draw(b, steps, H, G, P, N, R, io, 1.0, seed=17)
    for t in range(steps):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        y = m3scan.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["lam"], tok["theta"],
                               tok["B"], tok["C"], tok["D"])
        torch.cuda.synchronize()
        one = {k: (v[:, t:t + 1] if v.dim() > 1 else v) for k, v in d.items()}
        yr, hr = oracle.scan(*oracle_args(one), state_in=ost)
        ost = (hr, np64(tok["B"]), np64(tok["x"]))
        ey = slice_err(np64(y)[:, None], yr, 2)
        eh = slice_err(np64(st.h), hr, 1)
        assert ey <= TOL[io] and eh <= TOL[io], (t, ey, eh)
    say(f"  last step y err {ey:.2e}  h err {eh:.2e}")


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_prefill_then_decode_equals_longer_prefill(io):
    """prefill(L1) followed by decode steps equals prefill(L1 + L2)."""
    b, H, G, P, N, R, Q = 2, 4, 1, 64, 128, 2, 32
    L1, L2 = 70, 6
    say("prefill+decode chain", io)
    d = draw(b, L1 + L2, H, G, P, N, R, io, 1.0, seed=41)
    yfull, stfull = gpu_prefill(d, Q)
    d1 = {k: (v[:, :L1].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    y1, st = gpu_prefill(d1, Q)
    ys = [y1]
    for t in range(L1, L1 + L2):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ys.append(m3scan.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["lam"], tok["theta"],
                                     tok["B"], tok["C"], tok["D"])[:, None])
    torch.cuda.synchronize()
    ycat = torch.cat(ys, dim=1)
    yr, hr = oracle.scan(*oracle_args(d))
    e1 = slice_err(np64(ycat), yr, 2)
    e2 = slice_err(np64(st.h), hr, 1)
    e3 = slice_err(np64(yfull), yr, 2)
    say(f"  chain y {e1:.2e} h {e2:.2e}  full y {e3:.2e}")
    assert max(e1, e2, e3) <= TOL[io]


def test_parity_example_through_gpu_decode():
    """The worked parity example (Mamba-3 paper note, "Solution 2"), run through the
    GPU decode kernel one bit per call: the state ends at (-1, 0) and the sign of
    its first component gives the parity the page prints."""
    g, bits = pins._parity_bits()
    say("parity example, GPU decode")
    dev = "cuda"
    st = m3scan.DecodeState(torch.tensor([[[[1.0], [0.0]]]], device=dev))
    z = lambda *s: torch.zeros(s, device=dev)
    A, D = z(1), z(1)
    C = torch.tensor([[[[1.0, 0.0]]]], device=dev)
    Bt, xt, lam, dt = z(1, 1, 1, 2), z(1, 1, 1, 1), torch.full((1, 1), 0.5, device=dev), torch.ones(1, 1, device=dev)
    for bit in bits:
        th = torch.full((1, 1, 1), math.pi * float(bit), device=dev)
        y = m3scan.decode_step(st, xt, dt, A, lam, th, Bt, C, D)
    torch.cuda.synchronize()
    final = st.h.flatten().tolist()
    assert abs(final[0] - g["rotating_state_final"][0]) < 1e-3 and abs(final[1]) < 1e-3
    assert (0 if float(y.flatten()[0]) > 0 else 1) == g["parity"]
    # decay: 0.5 per 1-bit and 0.9 per 0-bit over the first 20 bits
    st = m3scan.DecodeState(torch.tensor([[[[1.0], [0.0]]]], device=dev))
    Am = torch.full((1,), -1.0, device=dev)
    for bit in bits[:g["decay_steps"]]:
        dtv = math.log(2.0) if bit else -math.log(0.9)
        y = m3scan.decode_step(st, xt, torch.full((1, 1), dtv, device=dev), Am, lam, z(1, 1, 1), Bt, C, D)
    torch.cuda.synchronize()
    assert round(float(y.flatten()[0]), 6) == g["decay_final_rounded_6dp"]


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_causality_and_determinism(io):
    """Outputs before t are bit-identical when inputs after t change; two runs of
    the same call are bit-identical."""
    b, L, H, G, P, N, R, Q = 1, 90, 2, 1, 64, 128, 2, 32
    say("causality/determinism", io)
    d = draw(b, L, H, G, P, N, R, io, 1.0, seed=51)
    y1, s1 = gpu_prefill(d, Q)
    y2, s2 = gpu_prefill(d, Q)
    d2 = {k: v.clone() for k, v in d.items()}
    cut = 50
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        d2[k][:, cut:] = (d2[k][:, cut:].float() * 1.5 + 0.25).to(d2[k].dtype)
    y3, _ = gpu_prefill(d2, Q)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1.h, s2.h)
    assert torch.equal(y3[:, :cut], y1[:, :cut])
    assert not torch.equal(y3[:, cut:], y1[:, cut:])


@pytest.mark.parametrize("Q", [1, 2, 7, 32, 61])
def test_chunk_size_invariance(Q):
    """The chunked result does not depend on the chunk size (up to rounding)."""
    b, L, H, G, P, N, R = 1, 61, 2, 1, 16, 32, 2
    say("chunk size", Q)
    d = draw(b, L, H, G, P, N, R, "fp32", 3.0, seed=61)
    y, st = gpu_prefill(d, Q)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d))
    assert slice_err(np64(y), yr, 2) <= 1e-4 and slice_err(np64(st.h), hr, 1) <= 1e-4


@pytest.mark.parametrize("R,Q", [(4, 64), (2, 64)])
def test_fp32_at_the_mimo_head_shape(R, Q):
    """fp32 io at N=128, P=64 (the 1.5B head shape) with a chunk whose arrays exceed LDS: the
    vector kernel runs it in smaller blocks; held to the fp32 bar (1e-4), ragged end included."""
    b, L, H, G = 2, 150, 2, 1
    say("fp32 prefill at the MIMO head shape", R, Q)
    d = draw(b, L, H, G, 64, 128, R, "fp32", 1.0, seed=100 + R)
    st0 = rand_state(b, H, G, 128, 64, R, "fp32", seed=11)
    y, st = gpu_prefill(d, Q, state_in=st0)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d), state_in=oracle_state(st0))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["fp32"] and eh <= TOL["fp32"]
