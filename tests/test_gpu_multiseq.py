"""GPU parity of the matrix-core prefill when one workgroup sweeps several short
sequences one after another (batches of many equal-length sequences of one to four
whole chunks; m3_prefill_sequences_per_workgroup > 1).

Each case runs the whole batch through that sweep, then the same inputs again in
slices of the batch small enough that every workgroup takes one sequence; the
outputs, final states and carries must be the same bits (the sweep changes which
workgroup computes a sequence, not its arithmetic).  The sequences on both sides
of the sweep's boundaries (the last of one workgroup, the first of the next, the
ragged last group) are also checked against the fp64 oracle at the bf16 bar."""
import ctypes
import zlib

import pytest
import torch

import oracle
from gpu_util import TOL, draw, np64, oracle_args, oracle_state, rand_state, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

P, N = 64, 128

# (b, L, H, G, R, Q, state: None | "fp32" | "bf16", theta_scale); every case leaves a
# ragged last group of sequences
CASES = [
    (37, 64, 64, 1, 4, 64, None, 1.0),       # one chunk per sequence, two per workgroup
    (600, 64, 64, 1, 4, 64, None, 4.0),      # sixteen per workgroup
    (301, 256, 64, 1, 1, 64, "fp32", 1.0),   # four chunks each, from a state with carries
    (201, 128, 64, 8, 2, 32, "bf16", 1.0),   # groups of heads, bf16 state, four chunks each
    (265, 64, 64, 2, 1, 32, None, 1.0),      # 32-row chunks, two chunks each
    (100, 96, 64, 1, 2, 32, "fp32", 1.0),    # three chunks each
]


def _id(c):
    return "b{}L{}H{}G{}R{}Q{}-{}-th{}".format(*c)


def _run(d, Q, sin, sdt, lo, hi):
    cut = lambda t: None if t is None else t[lo:hi].contiguous()
    st = None if sin is None else m3scan.DecodeState(cut(sin.h), cut(sin.b_last), cut(sin.x_last))
    return m3scan.prefill(*(cut(d[k]) if k not in ("A", "D") else d[k]
                            for k in ("x", "dt", "A", "lam", "theta", "B", "C", "D")),
                          Q, state_in=st, state_dtype=sdt)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_multi_sequence_sweep(case):
    b, L, H, G, R, Q, sk, ts = case
    say("multi-sequence prefill", _id(case))
    sdt = torch.bfloat16 if sk == "bf16" else torch.float32
    sflag = m3scan.M3_BF16 if sk == "bf16" else m3scan.M3_F32
    seqs = m3scan.prefill_sequences_per_workgroup(m3scan.make_dims(b, L, H, G, P, N, R, Q, m3scan.M3_BF16, sflag))
    say(f"  sequences per workgroup: {seqs}")
    assert seqs > 1 and b % seqs != 0
    d = draw(b, L, H, G, P, N, R, "bf16", ts, seed=zlib.crc32(_id(case).encode()) % 10000)
    sin = None
    if sk is not None:
        sin = rand_state(b, H, G, N, P, R, "bf16", seed=11)
        sin = m3scan.DecodeState(sin.h.to(sdt), sin.b_last, sin.x_last)
    y, st = _run(d, Q, sin, sdt, 0, b)
    # the same sequences in slices that run one sequence per workgroup
    step = 1
    while m3scan.prefill_sequences_per_workgroup(
            m3scan.make_dims(2 * step, L, H, G, P, N, R, Q, m3scan.M3_BF16, sflag)) == 1 and 2 * step <= b:
        step *= 2
    assert m3scan.prefill_sequences_per_workgroup(m3scan.make_dims(step, L, H, G, P, N, R, Q, m3scan.M3_BF16,
                                                                   sflag)) == 1
    for lo in range(0, b, step):
        hi = min(b, lo + step)
        yr, sr = _run(d, Q, sin, sdt, lo, hi)
        assert torch.equal(y[lo:hi], yr), f"y differs in batch slice {lo}:{hi}"
        assert torch.equal(st.h[lo:hi], sr.h), f"state differs in batch slice {lo}:{hi}"
        assert torch.equal(st.b_last[lo:hi], sr.b_last) and torch.equal(st.x_last[lo:hi], sr.x_last)
    torch.cuda.synchronize()
    say(f"  bit-identical to one sequence per workgroup (slices of {step})")
    # the oracle on the sequences around the sweep's boundaries
    picks = sorted({0, seqs - 1, seqs, 2 * seqs - 1, (b // seqs) * seqs - 1, (b // seqs) * seqs, b - 1})
    sub = {k: (d[k][picks] if k not in ("A", "D") else d[k]) for k in d}
    sref = None if sin is None else oracle_state(m3scan.DecodeState(sin.h[picks], sin.b_last[picks],
                                                                   sin.x_last[picks]))
    # a bf16 state is rounded once, after the last token (the outputs read it unrounded)
    flags = [False] * (L - 1) + [True] if sk == "bf16" else None
    yr, hr = oracle.scan(*oracle_args(sub), state_in=sref, round_after=flags)
    ey, eh = slice_err(np64(y[picks]), yr, 2), slice_err(np64(st.h[picks]), hr, 1)
    say(f"  oracle on batch entries {picks}: y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_multi_sequence_sweep_in_place():
    """state_in may alias state_out in the sweep too: each sequence's incoming state is read
    before its own final state is written, and the carries are copied after the scan.  The
    in-place call gives the same bits as separate buffers."""
    b, L, H, G, R, Q = 70, 64, 64, 1, 4, 64
    seqs = m3scan.prefill_sequences_per_workgroup(m3scan.make_dims(b, L, H, G, P, N, R, Q, m3scan.M3_BF16))
    assert seqs > 1
    d = draw(b, L, H, G, P, N, R, "bf16", 1.0, seed=4242)
    sin = rand_state(b, H, G, N, P, R, "bf16", seed=13)
    args = [d[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C", "D")]
    y_ref, st_ref = m3scan.prefill(*args, Q, state_in=sin)
    buf = m3scan.DecodeState(sin.h.clone(), sin.b_last.clone(), sin.x_last.clone())
    dims = m3scan.make_dims(b, L, H, G, P, N, R, Q, m3scan.M3_BF16)
    ws = torch.empty(max(m3scan.workspace_size(dims), 1), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    s = m3scan.State(buf.h.data_ptr(), buf.b_last.data_ptr(), buf.x_last.data_ptr())
    rc = m3scan.lib().m3_prefill_chunked(ctypes.byref(dims), *[m3scan._p(t) for t in args],
                                         ctypes.byref(s), ctypes.byref(s), m3scan._p(y), m3scan._p(ws),
                                         ws.numel(), m3scan._stream(torch.device("cuda")))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(buf.h, st_ref.h)
    assert torch.equal(buf.b_last, st_ref.b_last) and torch.equal(buf.x_last, st_ref.x_last)
