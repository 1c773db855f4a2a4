"""The allocation-free prefill (m3_prefill_chunked_noalloc, whose workspace is the
library's static scratch array) against the prefill with a caller-provided workspace
(m3_prefill_chunked) and against the oracle: two calls in a row on one GPU, the second
with a smaller input, so the second reads a scratch array that still holds the first
call's contents."""
import pytest
import torch

import oracle
from gpu_util import TOL, draw, np64, oracle_args, oracle_state, rand_state, say, slice_err
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu

# (b, L, H, G, R, Q, with state_in): the first is segmented (its summarised segment is cut
# into pieces: the scratch holds prepared operands, segment summaries and entering states)
CALLS = [(2, 1100, 44, 1, 4, 64, False), (1, 300, 4, 2, 2, 32, True)]


def test_noalloc_matches_workspace_prefill_twice():
    dims0 = m3scan.make_dims(*[CALLS[0][i] for i in (0, 1, 2, 3)], 64, 128, CALLS[0][4], CALLS[0][5],
                             m3scan.M3_BF16)
    assert m3scan.workspace_size(dims0) <= m3scan.NOALLOC_SCRATCH_BYTES
    for n, (b, L, H, G, R, Q, with_state) in enumerate(CALLS):
        say(f"noalloc call {n}: b{b} L{L} H{H} G{G} R{R} Q{Q} state_in={with_state}")
        d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=400 + n)
        st0 = rand_state(b, H, G, 128, 64, R, "bf16", seed=40 + n) if with_state else None
        args = [d[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C", "D")]
        y_ref, s_ref = m3scan.prefill(*args, Q, state_in=st0)
        y, s = m3scan.prefill_noalloc(*args, Q, state_in=st0)
        torch.cuda.synchronize()
        # same kernels and the same plan: identical bits
        assert torch.equal(y, y_ref)
        assert torch.equal(s.h, s_ref.h)
        assert torch.equal(s.b_last, s_ref.b_last) and torch.equal(s.x_last, s_ref.x_last)
        yr, hr = oracle.scan(*oracle_args(d), state_in=oracle_state(st0))
        ey, eh = slice_err(np64(y), yr, 2), slice_err(np64(s.h), hr, 1)
        say(f"  identical to the workspace call; vs oracle: y {ey:.2e} h {eh:.2e}")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
