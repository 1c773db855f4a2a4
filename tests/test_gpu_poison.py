"""Workspace canaries: every call that takes a workspace is run twice, once with the
workspace filled with NaN bytes (0xFF: NaN as fp32 and as bf16) and once with zeros.
A kernel that reads a workspace word it did not write first (in this call) would
carry a NaN into its outputs, so the two runs must agree bit for bit and hold no NaN.
Covered: the segmented prefill (segment summaries, entering states), the segmented
prefill whose summarised segment is cut into pieces, the packed variable-length
prefill (chunk slots past a short sequence's end are never written), the fused
prefill with a carried B (its normalised copy lives in the workspace), and the
backward with split sequences and per-head partial gradients."""
import numpy as np
import pytest
import torch

from gpu_util import draw, rand_state, say
from state_space_sequence_scan_amd import m3scan

pytestmark = pytest.mark.gpu


def _ws(nbytes, fill):
    return torch.full((max(nbytes, 1),), fill, dtype=torch.uint8, device="cuda")


def _same(a, b, what):
    assert not torch.isnan(a.float()).any(), f"{what}: NaN from the poisoned workspace"
    assert torch.equal(a, b), f"{what}: results depend on the workspace contents"


def _args(d):
    return [d[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C", "D")]


# (b, L, H, G, R, Q): several segments; one summarised segment cut into two pieces; G = H groups;
# segments of 128-row chunks (4-wave workgroups)
PREFILL = [(1, 1000, 2, 1, 2, 32), (2, 1100, 44, 1, 4, 64), (1, 777, 2, 2, 4, 64), (1, 1500, 2, 1, 4, 32)]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "b{}L{}H{}G{}R{}Q{}".format(*c))
def test_prefill_ignores_workspace_contents(case):
    b, L, H, G, R, Q = case
    say("poison prefill", case)
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=601)
    st0 = rand_state(b, H, G, 128, 64, R, "bf16", seed=61)
    n = m3scan.workspace_size(m3scan.make_dims(b, L, H, G, 64, 128, R, Q, m3scan.M3_BF16))
    outs = []
    for fill in (0xFF, 0x00):
        y, st = m3scan.prefill(*_args(d), Q, state_in=st0, workspace=_ws(n, fill))
        outs.append((y, st))
    torch.cuda.synchronize()
    _same(outs[0][0], outs[1][0], "y")
    _same(outs[0][1].h, outs[1][1].h, "state")


def test_packed_prefill_ignores_workspace_contents():
    lengths = [130, 0, 64, 17, 300, 1, 700]
    H, G, R, Q = 4, 1, 2, 32
    T = sum(lengths)
    d = draw(1, T, H, G, 64, 128, R, "bf16", 1.0, seed=602)
    d = {k: (v[0].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    n = m3scan.workspace_size(m3scan.make_dims(len(lengths), max(lengths), H, G, 64, 128, R, Q, m3scan.M3_BF16))
    outs = [m3scan.prefill_varlen(*_args(d), cu, max(lengths), Q, workspace=_ws(n, f)) for f in (0xFF, 0x00)]
    torch.cuda.synchronize()
    _same(outs[0][0], outs[1][0], "y")
    _same(outs[0][1].h, outs[1][1].h, "state")


def test_fused_prefill_ignores_workspace_contents():
    b, L, H, G, R, Q = 2, 900, 4, 1, 4, 64
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=603)
    st0 = rand_state(b, H, G, 128, 64, R, "bf16", seed=63)
    g = torch.Generator(device="cuda").manual_seed(9)
    fz = {"b_norm_w": 1.0 + 0.3 * torch.randn((R, 128), generator=g, device="cuda"),
          "c_norm_w": 1.0 + 0.3 * torch.randn((R, 128), generator=g, device="cuda"),
          "b_bias": 0.05 * torch.randn((R, 128), generator=g, device="cuda"),
          "c_bias": 0.05 * torch.randn((R, 128), generator=g, device="cuda")}
    n = m3scan.workspace_size(m3scan.make_dims(b, L, H, G, 64, 128, R, Q, m3scan.M3_BF16))
    outs = [m3scan.prefill_fused(*_args(d), Q, **fz, state_in=st0, workspace=_ws(n, f)) for f in (0xFF, 0x00)]
    torch.cuda.synchronize()
    _same(outs[0][0], outs[1][0], "y")
    _same(outs[0][1].h, outs[1][1].h, "state")


# (b, L, H, G, R): few (b, h) pairs (the sequence is split into pieces); H > G (per-head partials)
BACKWARD = [(1, 700, 2, 1, 2), (2, 300, 4, 2, 4)]


@pytest.mark.parametrize("case", BACKWARD, ids=lambda c: "b{}L{}H{}G{}R{}".format(*c))
def test_backward_ignores_workspace_contents(case):
    b, L, H, G, R = case
    d = draw(b, L, H, G, 64, 128, R, "bf16", 1.0, seed=604)
    st0 = rand_state(b, H, G, 128, 64, R, "bf16", seed=64)
    gen = torch.Generator(device="cuda").manual_seed(10)
    dy = torch.randn(d["x"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    dh = torch.randn((b, H, 128, 64), generator=gen, device="cuda")
    dims = m3scan.make_dims(b, L, H, G, 64, 128, R, 1, m3scan.M3_BF16)
    parts, _ = m3scan.backward_parts(dims)
    say("poison backward", case, "parts", parts)
    n = m3scan.backward_workspace_size(dims)
    outs = [m3scan.backward(*_args(d), dy, dh_out=dh, state_in=st0, workspace=_ws(n, f)) for f in (0xFF, 0x00)]
    torch.cuda.synchronize()
    for k in outs[0]:
        _same(outs[0][k], outs[1][k], k)
