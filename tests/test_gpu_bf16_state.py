"""GPU parity of the reduced-precision (bf16) state: a prefill that writes its
final state in bf16 and decode steps that read and write a bf16 state, against
the oracle with the same rounding (the state replaced by its nearest bf16 value
after the prefill's last token and after every decode token; the outputs read
the unrounded state).  Bar: 2e-2 (max relative error per slice), for fp32 as
well as bf16 inputs, since one bf16 rounding of the state is ~4e-3 relative."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import draw, np64, oracle_args, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu
TOL_BF16_STATE = 2e-2

# (b, L_prefill, steps, H, G, P, N, R, Q, io) -- MFMA prefill + fast decode, generic
# prefill + fast decode (N = 16), and generic prefill + generic decode
CASES = [
    (2, 130, 12, 4, 1, 64, 128, 4, 64, "bf16"),
    (1, 1000, 6, 2, 1, 64, 128, 2, 32, "bf16"),      # several segments
    (2, 300, 8, 4, 1, 64, 128, 4, 32, "bf16"),       # 128-row chunks (4-wave prefill)
    (1, 96, 10, 4, 1, 16, 16, 1, 32, "fp32"),
    (2, 40, 8, 2, 2, 8, 12, 3, 16, "fp32"),
]


def _id(c):
    return "b{}L{}s{}H{}G{}P{}N{}R{}Q{}-{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_prefill_then_decode_bf16_state(case):
    b, L1, K, H, G, P, N, R, Q, io = case
    say("bf16 state", _id(case))
    d = draw(b, L1 + K, H, G, P, N, R, io, 1.0, seed=31 + L1)
    d1 = {k: (v[:, :L1].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    y1, st = m3scan.prefill(d1["x"], d1["dt"], d1["A"], d1["lam"], d1["theta"], d1["B"], d1["C"],
                            d1["D"], Q, state_dtype=torch.bfloat16)
    assert st.h.dtype == torch.bfloat16
    ys = [y1]
    for t in range(L1, L1 + K):
        tok = {k: (v[:, t].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
        ys.append(m3scan.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["lam"], tok["theta"],
                                     tok["B"], tok["C"], tok["D"])[:, None])
    torch.cuda.synchronize()
    flags = np.zeros(L1 + K, bool)
    flags[L1 - 1:] = True
    yr, hr = oracle.scan(*oracle_args(d), round_after=flags)
    ey = slice_err(np64(torch.cat(ys, 1)), yr, 2)
    eh = slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL_BF16_STATE and eh <= TOL_BF16_STATE


@pytest.mark.parametrize("L,R,Q", [(200, 4, 64), (1000, 2, 32), (50, 1, 32), (700, 4, 32)])
def test_prefill_from_bf16_state(L, R, Q):
    """state_in in bf16 (values exact in bf16), state_out in bf16."""
    b, H, G, P, N = 1, 2, 1, 64, 128
    say("prefill from bf16 state", L, R, Q)
    d = draw(b, L, H, G, P, N, R, "bf16", 1.0, seed=41 + L)
    gen = torch.Generator(device="cpu").manual_seed(7)
    h0 = torch.randn((b, H, N, P), generator=gen).to(torch.bfloat16).cuda()
    bl = torch.randn((b, G, R, N), generator=gen).to(torch.bfloat16).cuda()
    xl = torch.randn((b, H, R, P), generator=gen).to(torch.bfloat16).cuda()
    st0 = m3scan.DecodeState(h0, bl, xl)
    y, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                           Q, state_in=st0)
    torch.cuda.synchronize()
    assert st.h.dtype == torch.bfloat16
    flags = np.zeros(L, bool)
    flags[-1] = True
    yr, hr = oracle.scan(*oracle_args(d), state_in=(np64(h0), np64(bl), np64(xl)), round_after=flags)
    ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(st.h), hr, 1)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL_BF16_STATE and eh <= TOL_BF16_STATE


def test_bf16_state_decode_matches_fp32_state_decode_to_bf16_rounding():
    """From the same (bf16-exact) state, one decode step with a bf16 state gives
    y within one bf16 ulp of the step with an fp32 state (both fp32 arithmetic;
    the kernels sum the read-out in different orders), and its new state is the
    fp32 one rounded to nearest: within half a bf16 ulp."""
    b, H, G, P, N, R = 4, 8, 2, 64, 128, 4
    d = draw(b, 1, H, G, P, N, R, "bf16", 1.0, seed=55)
    tok = {k: (v[:, 0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    gen = torch.Generator(device="cpu").manual_seed(8)
    h0 = torch.randn((b, H, N, P), generator=gen).to(torch.bfloat16)
    st32 = m3scan.DecodeState(h0.float().cuda())
    st16 = m3scan.DecodeState(h0.cuda())
    args = (tok["x"], tok["dt"], tok["A"], tok["lam"], tok["theta"], tok["B"], tok["C"], tok["D"])
    y32 = m3scan.decode_step(st32, *args)
    y16 = m3scan.decode_step(st16, *args)
    torch.cuda.synchronize()
    assert torch.allclose(y16.float(), y32.float(), rtol=2.0 ** -7, atol=1e-6)
    h16, h32 = st16.h.float(), st32.h
    assert torch.all((h16 - h32).abs() <= h32.abs() * 2.0 ** -8 + 1e-30)
    assert (h16 == h32.to(torch.bfloat16).float()).float().mean() > 0.99
