"""The workloads at their full sizes, in the launch configuration the benchmark
times, checked against the oracle on every (batch, head) slice.

The GPU runs each workload whole (one prefill over all sequences, then the decode
steps); the oracle then runs block by block (a few batch elements and heads at a
time, OpenMP over the slices of a block), so host memory stays bounded.  Each
slice is held to the tolerance of its io dtype with the metric max|gpu - ref| /
max|ref| over the slice; the elementwise diagnostic max |gpu - ref| / (|ref| +
1e-3 max|ref|) is printed next to it for every workload."""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, onorm_slice_errs, say, slice_errs
from state_space_sequence_scan_amd import CONFIGS, inputs, m3scan

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

f64 = lambda t: t.detach().double().cpu().numpy()


def _blocks(cfg, heads_per_block):
    """(batch range, head range) blocks covering every slice; head ranges hold whole groups."""
    per_group = cfg.nheads // cfg.ngroups
    if cfg.ngroups == 1:   # one group: any head range sees it whole
        hb = min(heads_per_block, cfg.nheads)
    else:
        hb = max(per_group, (heads_per_block // per_group) * per_group)
    for b0 in range(cfg.batch):
        for h0 in range(0, cfg.nheads, hb):
            yield b0, b0 + 1, h0, min(cfg.nheads, h0 + hb)


def _block_args(d, cfg, b0, b1, h0, h1, At=None):
    per_group = cfg.nheads // cfg.ngroups
    g0, g1 = h0 // per_group, (h1 - 1) // per_group + 1
    return [f64(d["x"][b0:b1, :, h0:h1]), f64(d["dt"][b0:b1, :, h0:h1]),
            f64(d["A"][h0:h1]) if At is None else f64(At[b0:b1, :, h0:h1]),
            f64(d["lam"][b0:b1, :, h0:h1]), f64(d["theta"][b0:b1, :, g0:g1]),
            f64(d["B"][b0:b1, :, g0:g1]), f64(d["C"][b0:b1, :, g0:g1]), f64(d["D"][h0:h1])]


class Tally:
    def __init__(self, name, tol):
        self.name, self.tol = name, tol
        self.worst = {}
        self.elem = 0.0
        self.slices = 0

    def add(self, what, per_slice, elem, where):
        w = float(np.max(per_slice)) if per_slice.size else 0.0
        if w > self.worst.get(what, (-1.0, None))[0]:
            i = np.unravel_index(int(np.argmax(per_slice)), per_slice.shape) if per_slice.size else ()
            self.worst[what] = (w, (where, tuple(int(v) for v in i)))
        self.elem = max(self.elem, elem)
        assert w <= self.tol, f"{self.name} {what} {where}: slice error {w:.3e} > {self.tol}"

    def report(self):
        say(f"  {self.name}: {self.slices} slices; worst per-slice error "
            + ", ".join(f"{k} {v[0]:.2e} at {v[1]}" for k, v in self.worst.items())
            + f"; elementwise diagnostic max {self.elem:.2e}")


@pytest.mark.parametrize("name", ["siso_l256_fp32", "nanomamba3", "siso_l8192", "mimo4_l16384"])
def test_prefill_workload_every_slice(name):
    cfg = CONFIGS[name]
    say("workload", name, cfg.label)
    d = inputs.draw_config(cfg, device="cuda")
    y, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                           cfg.chunk)
    torch.cuda.synchronize()
    tally = Tally(name, TOL[cfg.io_dtype])
    for b0, b1, h0, h1 in _blocks(cfg, 16):
        yr, hr = oracle.scan(*_block_args(d, cfg, b0, b1, h0, h1))
        tally.add("y", *slice_errs(f64(y[b0:b1, :, h0:h1]), yr, 2), (b0, h0))
        tally.add("h", *slice_errs(f64(st.h[b0:b1, h0:h1]), hr, 1), (b0, h0))
        tally.slices += (b1 - b0) * (h1 - h0)
        say(f"  block b{b0} h{h0}..{h1 - 1} done")
    assert tally.slices == cfg.batch * cfg.nheads
    # the carry is a copy of the last token's B and X: bit-exact
    assert torch.equal(st.b_last, d["B"][:, -1]) and torch.equal(st.x_last, d["x"][:, -1])
    tally.report()


def test_decode_workload_every_slice():
    """1.5B MIMO R=4 layer, batch 256: 1024-token prefill, then 512 decode steps; every
    (batch, head) slice's 1536 outputs and final state against one oracle scan of the
    1536 tokens."""
    cfg = CONFIGS["mimo4_decode_b256"]
    say("workload mimo4_decode_b256", cfg.label)
    d = inputs.draw_config(cfg, device="cuda")
    dd = inputs.draw_decode(cfg, cfg.decode_steps, device="cuda")
    y, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                           cfg.chunk)
    ydec = torch.empty((cfg.decode_steps,) + tuple(d["x"][:, 0].shape), dtype=d["x"].dtype, device="cuda")
    for t in range(cfg.decode_steps):
        m3scan.decode_step(st, dd["x"][t], dd["dt"][t], d["A"], dd["lam"][t], dd["theta"][t],
                           dd["B"][t], dd["C"][t], d["D"], y_t=ydec[t])
    torch.cuda.synchronize()
    tally = Tally("mimo4_decode_b256", TOL["bf16"])
    nb = 8
    for b0 in range(0, cfg.batch, nb):
        b1 = b0 + nb
        cat = lambda k: np.concatenate([f64(d[k][b0:b1]), f64(dd[k][:, b0:b1].transpose(0, 1))], axis=1)
        yr, hr = oracle.scan(cat("x"), cat("dt"), f64(d["A"]), cat("lam"), cat("theta"), cat("B"), cat("C"),
                             f64(d["D"]))
        yg = np.concatenate([f64(y[b0:b1]), f64(ydec[:, b0:b1].transpose(0, 1))], axis=1)
        tally.add("y", *slice_errs(yg, yr, 2), (b0, 0))
        tally.add("h", *slice_errs(f64(st.h[b0:b1]), hr, 1), (b0, 0))
        tally.slices += nb * cfg.nheads
        say(f"  batches {b0}..{b1 - 1} done")
    assert tally.slices == cfg.batch * cfg.nheads
    tally.report()


@pytest.mark.parametrize("name", ["nanomamba3", "mimo4_l16384"])
def test_backward_workload_every_slice(name):
    """The backward at the full size of a training-shaped workload: every gradient.  The
    per-head ones (dx, ddt, dlambda) slice by slice; the group-shared ones (dB, dC, dtheta,
    summed over a group's heads) per batch element, after the head blocks of that element
    are summed; dA and dD (summed over batch and tokens) over the whole tensor."""
    cfg = CONFIGS[name]
    assert cfg.ngroups == 1   # the group-shared sums below run over every head
    say("backward workload", name)
    d = inputs.draw_config(cfg, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 11)
    dy = torch.randn(d["x"].shape, generator=g, device="cuda").to(d["x"].dtype)
    gr = m3scan.backward(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"], dy,
                         want_state_grads=False)
    torch.cuda.synchronize()
    tally = Tally(f"{name} backward", 1e-3)
    dA = np.zeros(cfg.nheads)
    dD = np.zeros(cfg.nheads)
    # The oracle's backward runs its batch elements in parallel; here every call is one
    # (batch, head) slice, and the slices of a batch element run side by side on host threads
    # (the C oracle runs outside the interpreter lock).
    workers = min(16, os.cpu_count() or 1)
    for b0 in range(cfg.batch):
        ins = [(_block_args(d, cfg, b0, b0 + 1, h, h + 1), f64(dy[b0:b0 + 1, :, h:h + 1])) for h in range(cfg.nheads)]
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            refs = list(ex.map(lambda a: oracle.scan_backward(*a[0], a[1], nthreads=1), ins))
        shared = {k: sum(r[k] for r in refs) for k in ("dB", "dC", "dtheta")}   # G = 1: over every head
        for h, ref in enumerate(refs):
            for k, ax in (("dx", 2), ("ddt", 2), ("dlam", 2)):
                tally.add(k, *slice_errs(f64(gr[k][b0:b0 + 1, :, h:h + 1]), ref[k], ax), (b0, h))
            dA[h] += ref["dA"][0]
            dD[h] += ref["dD"][0]
        for k, ax in (("dB", 2), ("dC", 2), ("dtheta", 2)):
            tally.add(k, *slice_errs(f64(gr[k][b0:b0 + 1]), shared[k], ax), (b0, "groups"))
        tally.slices += cfg.nheads
        say(f"  batch element {b0} done")
    for k, ref in (("dA", dA), ("dD", dD)):
        e = float(np.max(np.abs(f64(gr[k]) - ref)) / np.max(np.abs(ref)))
        say(f"  {k}: {e:.2e}")
        assert e <= 1e-3, (k, e)
    tally.report()


def test_fused_prefill_workload_every_slice():
    """The fused prologue/epilogue (per-token A, BCNorm and bias of B and C, gate) at the
    full size of the 1.5B-scale SISO layer, every slice."""
    cfg = CONFIGS["siso_l8192"]
    say("fused workload siso_l8192")
    d = inputs.draw_config(cfg, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 23)
    R, N = cfg.rank, cfg.dstate
    fz = {"A_t": -torch.exp(torch.rand(d["dt"].shape, generator=g, device="cuda") * np.log(16.0)),
          "b_norm_w": 1.0 + 0.3 * torch.randn((R, N), generator=g, device="cuda"),
          "c_norm_w": 1.0 + 0.3 * torch.randn((R, N), generator=g, device="cuda"),
          "b_bias": 0.02 + 0.05 * torch.randn((R, N), generator=g, device="cuda"),
          "c_bias": 0.02 + 0.05 * torch.randn((R, N), generator=g, device="cuda"),
          "z": torch.randn(d["x"].shape, generator=g, device="cuda").to(d["x"].dtype)}
    y, st = m3scan.prefill_fused(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                                 cfg.chunk, **fz)
    torch.cuda.synchronize()
    tally = Tally("siso_l8192 fused", TOL["bf16"])
    for b0, b1, h0, h1 in _blocks(cfg, 64):
        args = _block_args(d, cfg, b0, b1, h0, h1, At=fz["A_t"])
        yr, hr = oracle.scan_fused(*args, b_norm_w=f64(fz["b_norm_w"]), c_norm_w=f64(fz["c_norm_w"]),
                                   b_bias=f64(fz["b_bias"]), c_bias=f64(fz["c_bias"]),
                                   z=f64(fz["z"][b0:b1, :, h0:h1]))
        tally.add("y", *slice_errs(f64(y[b0:b1, :, h0:h1]), yr, 2), (b0, h0))
        tally.add("h", *slice_errs(f64(st.h[b0:b1, h0:h1]), hr, 1), (b0, h0))
        tally.slices += (b1 - b0) * (h1 - h0)
        say(f"  block b{b0} done")
    tally.report()


def test_theta_per_head_out_norm_workload_every_slice():
    """The 1.5B-scale SISO layer with angles per head over the shared B and C (64 angle
    groups: the rotated operands are prepared per head) and the output RMSNorm, at full
    size, every slice.  The normalised outputs are held to the bar on the scale of the rows
    before the norm (onorm_slice_errs); the printed elementwise figure is then the plain
    per-slice error of the normalised outputs, which the norm inflates on small rows."""
    cfg = CONFIGS["siso_l8192"]
    say("angles per head + output norm, workload siso_l8192")
    d = inputs.draw_config(cfg, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 29)
    theta_h = (torch.rand((cfg.batch, cfg.seqlen, cfg.nheads, cfg.dstate // 2), generator=g, device="cuda") * 2 - 1) \
        * np.pi
    onw = 1.0 + 0.3 * torch.randn((cfg.nheads, cfg.headdim), generator=g, device="cuda")
    y, st = m3scan.prefill_fused(d["x"], d["dt"], d["A"], d["lam"], theta_h, d["B"], d["C"], d["D"], cfg.chunk,
                                 out_norm_w=onw)
    torch.cuda.synchronize()
    tally = Tally("siso_l8192 angles per head + output norm", TOL["bf16"])
    worst_plain = 0.0
    for b0, b1, h0, h1 in _blocks(cfg, 16):
        args = _block_args(d, cfg, b0, b1, h0, h1)
        args[4] = f64(theta_h[b0:b1, :, h0:h1])
        ypre, hr = oracle.scan_fused(*args)
        per, plain = onorm_slice_errs(f64(y[b0:b1, :, h0:h1]), ypre, f64(onw[h0:h1]), 1e-6)
        tally.add("y (normalised, pre-norm scale)", per, 0.0, (b0, h0))
        worst_plain = max(worst_plain, plain)
        tally.add("h", *slice_errs(f64(st.h[b0:b1, h0:h1]), hr, 1), (b0, h0))
        tally.slices += (b1 - b0) * (h1 - h0)
        say(f"  block b{b0} h{h0}..{h1 - 1} done")
    assert tally.slices == cfg.batch * cfg.nheads
    tally.report()
    say(f"  plain per-slice error of the normalised outputs (inflated on near-zero rows): {worst_plain:.2e}")


@pytest.mark.parametrize("name", ["mimo4_chunk64_b4096", "siso_chunk64_b4096"])
def test_intra_chunk_workload(name):
    """Single-chunk sequences (L = chunk = 64, batch 4096) at the 1.5B head shapes: one launch
    as the benchmark times it (16 sequences of a head per workgroup, swept one after
    another); every (batch, head) slice against the oracle (each sequence is one intra-chunk
    block plus its chunk state), 128 batch elements at a time."""
    from state_space_sequence_scan_amd.configs import INTRA_CHUNK
    cfg = INTRA_CHUNK[name]
    say("intra-chunk workload", name, cfg.label)
    dims = m3scan.make_dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank,
                            cfg.chunk, m3scan.M3_BF16)
    assert m3scan.prefill_sequences_per_workgroup(dims) == 16
    d = inputs.draw_config(cfg, device="cuda")
    y, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"], cfg.chunk)
    torch.cuda.synchronize()
    tally = Tally(name, TOL[cfg.io_dtype])
    for b0 in range(0, cfg.batch, 128):
        b1 = b0 + 128
        yr, hr = oracle.scan(*[f64(d[k][b0:b1] if d[k].dim() > 1 else d[k]) for k in
                               ("x", "dt", "A", "lam", "theta", "B", "C", "D")])
        tally.add("y", *slice_errs(f64(y[b0:b1]), yr, 2), (b0, 0))
        tally.add("h", *slice_errs(f64(st.h[b0:b1]), hr, 1), (b0, 0))
        tally.slices += (b1 - b0) * cfg.nheads
        say(f"  batches {b0}..{b1 - 1} done")
    assert tally.slices == cfg.batch * cfg.nheads
    assert torch.equal(st.b_last, d["B"][:, -1]) and torch.equal(st.x_last, d["x"][:, -1])
    tally.report()
