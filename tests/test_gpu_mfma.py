"""GPU parity of the matrix-core prefill (bf16, N=128, P=64, R in {1,2,4},
chunk in {32,64}) against the fp64 oracle: ragged ends, several segments per
sequence, incoming state, shared and per-head groups."""
import zlib

import pytest
import torch

import oracle
from gpu_util import TOL, draw, gpu_prefill, np64, oracle_args, oracle_state, rand_state, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

# (b, L, H, G, R, Q, theta_scale)
CASES = [
    (2, 100, 3, 1, 1, 32, 1.0),
    (1, 300, 2, 1, 1, 64, 1.0),
    (1, 1000, 2, 1, 2, 32, 1.0),     # 32 chunks -> 8 segments
    (1, 777, 2, 2, 4, 64, 4.0),      # ragged, 3 segments, G = H
    (2, 130, 4, 2, 4, 32, 1.0),
    (1, 2048, 2, 1, 4, 64, 4.0),     # 8 segments, strong rotation
    (3, 64, 2, 1, 2, 64, 1.0),       # exactly one chunk
    (1, 17, 2, 1, 1, 32, 1.0),       # shorter than a chunk
    (2, 512, 4, 1, 2, 32, 1.0),
    # two segments whose summarised one is cut into two pieces for the state-only pass
    # (few (b, h) pairs): the output pass starts segment 1 from the second piece's end
    (2, 1100, 44, 1, 4, 64, 1.0),
    (4, 600, 48, 2, 2, 32, 1.0),
    # chunks of 128 rows (4 waves, two workgroups per CU, no s X tile): R = 4 at Q = 32 and
    # R = 2 at Q = 64, ragged, several segments (cut into pieces at few (b, h)), G = H
    (1, 1500, 2, 1, 4, 32, 4.0),
    (1, 400, 4, 4, 4, 32, 1.0),
    (2, 1100, 100, 1, 2, 64, 1.0),   # two segments, the summarised one in two pieces
    (2, 300, 4, 2, 2, 64, 1.0),
]


def _id(c):
    return "b{}L{}H{}G{}R{}Q{}-th{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_mfma_prefill_matches_oracle(case):
    b, L, H, G, R, Q, ts = case
    say("mfma prefill", _id(case))
    d = draw(b, L, H, G, 64, 128, R, "bf16", ts, seed=zlib.crc32(_id(case).encode()) % 10000)
    y, st = gpu_prefill(d, Q)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    assert torch.equal(st.b_last, d["B"][:, -1]) and torch.equal(st.x_last, d["x"][:, -1])


@pytest.mark.parametrize("L,R,Q", [(1000, 2, 32), (200, 4, 64), (64, 1, 64), (300, 4, 32), (500, 2, 64)])
def test_mfma_prefill_from_state(L, R, Q):
    b, H, G = 1, 2, 1
    say("mfma prefill from state", L, R, Q)
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=77)
    st0 = rand_state(b, H, G, 128, 64, R, "bf16", seed=9)
    y, st = gpu_prefill(d, Q, state_in=st0)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d), state_in=oracle_state(st0))
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_mfma_state_in_may_alias_state_out():
    b, L, H, G, R, Q = 1, 256, 2, 1, 2, 32
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=78)
    st0 = rand_state(b, H, G, 128, 64, R, "bf16", seed=10)
    ref_in = oracle_state(st0)
    out = m3scan.DecodeState(st0.h, st0.b_last, st0.x_last)   # same buffers for in and out
    dims = m3scan.make_dims(b, L, H, G, 64, 128, R, Q, m3scan.M3_BF16)
    ws = m3scan.workspace_size(dims)
    wbuf = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    s = m3scan.State(out.h.data_ptr(), out.b_last.data_ptr(), out.x_last.data_ptr())
    import ctypes
    rc = m3scan.lib().m3_prefill_chunked(ctypes.byref(dims), *[m3scan._p(d[k]) for k in
                                         ("x", "dt", "A", "lam", "theta", "B", "C", "D")],
                                         ctypes.byref(s), ctypes.byref(s), m3scan._p(y),
                                         m3scan._p(wbuf), ws, m3scan._stream(torch.device("cuda")))
    assert rc == 0
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d), state_in=ref_in)
    assert slice_err(np64(y), yr, 2) <= TOL["bf16"]
    assert slice_err(np64(out.h), hr, 1) <= TOL["bf16"]
    assert torch.equal(out.b_last, d["B"][:, -1]) and torch.equal(out.x_last, d["x"][:, -1])


def test_mfma_prefill_then_decode():
    b, H, G, R, Q = 2, 4, 1, 4, 64
    L1, L2 = 200, 8
    say("mfma prefill + decode chain")
    d = draw(b, L1 + L2, H, G, 64, 128, R, "bf16", 1.0, seed=81)
    d1 = {k: (v[:, :L1].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    y1, st = gpu_prefill(d1, Q)
    ys = [y1]
    for t in range(L1, L1 + L2):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ys.append(m3scan.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["lam"], tok["theta"],
                                     tok["B"], tok["C"], tok["D"])[:, None])
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*oracle_args(d))
    e1 = slice_err(np64(torch.cat(ys, 1)), yr, 2)
    e2 = slice_err(np64(st.h), hr, 1)
    say(f"  y err {e1:.2e}  h err {e2:.2e}")
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_mfma_causality_and_determinism():
    b, L, H, G, R, Q = 1, 1000, 2, 1, 2, 32    # several segments
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=91)
    y1, s1 = gpu_prefill(d, Q)
    y2, s2 = gpu_prefill(d, Q)
    d2 = {k: v.clone() for k, v in d.items()}
    cut = 613
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        d2[k][:, cut:] = (d2[k][:, cut:].float() * 1.5 + 0.25).to(d2[k].dtype)
    y3, _ = gpu_prefill(d2, Q)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1.h, s2.h)
    assert torch.equal(y3[:, :cut], y1[:, :cut])
    assert not torch.equal(y3[:, cut:], y1[:, cut:])


def test_mfma_one_hot_pairing():
    """A one-hot B at state row 2k, theta = pi/2 on pair k at the first token, and
    C reading row 2k+1 at the second: the rotation moves the input onto row 2k+1
    (counter-clockwise), so only that read-out sees it; reading row 2k sees zero."""
    b, L, H, G, R, Q = 1, 64, 1, 1, 1, 32
    dev = "cuda"
    z = lambda *s, dt=torch.float32: torch.zeros(s, device=dev, dtype=dt)
    x = z(b, L, H, R, 64, dt=torch.bfloat16)
    x[0, 0, 0, 0, :] = 1.0
    dt = torch.full((b, L, H), 0.5, device=dev)
    lam = torch.ones((b, L, H), device=dev)
    A = z(H)
    D = z(H)
    theta = z(b, L, G, 64)
    k = 5
    theta[0, 1, 0, k] = torch.pi / 2
    B = z(b, L, G, R, 128, dt=torch.bfloat16)
    B[0, 0, 0, 0, 2 * k] = 1.0
    C = z(b, L, G, R, 128, dt=torch.bfloat16)
    C[0, 1, 0, 0, 2 * k + 1] = 1.0
    C[0, 2, 0, 0, 2 * k] = 1.0
    y, st = m3scan.prefill(x, dt, A, lam, theta, B, C, D, Q)
    torch.cuda.synchronize()
    # token 0 writes 0.5 (dt * lambda) into row 2k; token 1 turns it onto row 2k+1
    assert torch.allclose(y[0, 1, 0, 0].float(), torch.full((64,), 0.5, device=dev), atol=1e-2)
    assert float(y[0, 2, 0, 0].abs().max()) < 1e-2
    assert torch.allclose(st.h[0, 0, 2 * k + 1], torch.full((64,), 0.5, device=dev), atol=1e-2)
