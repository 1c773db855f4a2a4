"""HIP graph capture of the scan (torch.cuda.graph, which captures the stream the binding
launches on): a prefill through the allocation-free entry point followed by decode steps
continuing it, on each prefill kernel family, captured once after an eager warm-up call and
replayed several times with new inputs copied into the captured buffers between replays,
with eager work and synchronisations in between.  Every replay must give the bits of an
eager run of the same calls on the same inputs: after a first call the path records kernel
launches only (no allocation, memset, host synchronisation or attribute change)."""
import pytest
import torch

from gpu_util import draw, say
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "D")


def _split(d, L, steps):
    pre = {k: (v[:, :L].contiguous() if v.dim() > 1 else v.clone()) for k, v in d.items()}
    toks = [{k: (v[:, t].contiguous() if v.dim() > 1 else v.clone()) for k, v in d.items()}
            for t in range(L, L + steps)]
    return pre, toks


def _run(pre, toks, Q, y, st, ydec):
    """The captured sequence: prefill into y / st, then the decode steps into ydec."""
    m3scan.prefill_noalloc(*[pre[k] for k in NAMES], Q, y=y, state_out=st)
    for t, tok in enumerate(toks):
        m3scan.decode_step(st, *[tok[k] for k in NAMES], y_t=ydec[t])


def _buffers(pre, toks, state_dtype):
    b, L, H, R, P = pre["x"].shape
    G, N = pre["B"].shape[2], pre["B"].shape[4]
    dev, io = pre["x"].device, pre["x"].dtype
    y = torch.empty_like(pre["x"])
    st = m3scan.DecodeState(torch.empty((b, H, N, P), dtype=state_dtype, device=dev),
                            torch.empty((b, G, R, N), dtype=io, device=dev),
                            torch.empty((b, H, R, P), dtype=io, device=dev))
    ydec = [torch.empty_like(t["x"]) for t in toks]
    return y, st, ydec


# (b, L, H, G, P, N, R, Q, io, state dtype): the matrix-core prefill with an fp32 and a bf16
# state, the token-serial fp32 prefill (66.5 KB of LDS: its limit is raised by the warm-up
# call, before the capture) and the chunked fp32 prefill
CASES = [
    (2, 200, 4, 1, 64, 128, 2, 32, "bf16", torch.float32),
    (2, 200, 4, 1, 64, 128, 2, 32, "bf16", torch.bfloat16),
    (1, 256, 4, 1, 16, 16, 1, 32, "fp32", torch.float32),
    (2, 100, 4, 2, 32, 32, 2, 16, "fp32", torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "P{}N{}R{}-{}-{}".format(c[4], c[5], c[6], c[8], str(c[9])[6:]))
def test_graph_replays_match_eager(case):
    b, L, H, G, P, N, R, Q, io, state_dtype = case
    steps = 3
    say("graph capture", case)
    pre, toks = _split(draw(b, L + steps, H, G, P, N, R, io, 1.0, seed=77), L, steps)
    y, st, ydec = _buffers(pre, toks, state_dtype)

    # warm-up on a side stream (the binding and kernels loaded before capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(pre, toks, Q, y, m3scan.DecodeState(st.h, st.b_last, st.x_last), ydec)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    cap = m3scan.DecodeState(st.h, st.b_last, st.x_last)
    with torch.cuda.graph(graph):
        _run(pre, toks, Q, y, cap, ydec)
    torch.cuda.synchronize()

    for rep in range(3):
        new_pre, new_toks = _split(draw(b, L + steps, H, G, P, N, R, io, 1.0, seed=100 + rep), L, steps)
        for k in NAMES:   # new inputs into the captured buffers (eager copies)
            pre[k].copy_(new_pre[k])
            for t in range(steps):
                toks[t][k].copy_(new_toks[t][k])
        graph.replay()
        torch.cuda.synchronize()
        ye, ste, ydece = _buffers(new_pre, new_toks, state_dtype)
        _run(new_pre, new_toks, Q, ye, ste, ydece)   # eager, on fresh buffers
        torch.cuda.synchronize()
        assert torch.equal(y, ye), rep
        assert torch.equal(cap.h, ste.h), rep
        for t in range(steps):
            assert torch.equal(ydec[t], ydece[t]), (rep, t)
        say(f"  replay {rep}: y, decode outputs and state equal to the eager run")
