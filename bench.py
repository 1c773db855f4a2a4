#!/usr/bin/env python3
"""Benchmark of the Mamba-3 scan on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the chunked prefill of every sequence, then the single-token decode steps that
continue from its state (default workload: the 1.5B-scale MIMO R=4 layer at
batch 256, 1024-token prefill + 512 decode steps).  Inputs are generated on the
GPU and resident in HBM before timing starts.

Prints one JSON line.  `value` is whole-step token throughput (prefill tokens +
decode tokens, all sequences) per second; the line also carries the prefill
tokens/s, the decode state bandwidth, the roofline of the dominant kernel and
the CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import math
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill scan tokens/s + decode state GB/s (% roofline), 1.5B-shape layer, 1 GPU"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6        # dense bf16 MFMA: 4096 flop/clk/CU x 256 CU x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 157.3    # fp32 vector: 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz
BWD_METRIC = "backward scan tokens/s (training step of the scan), 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None,
                    help="siso_l256_fp32, nanomamba3, siso_l8192, mimo4_l16384 (prefill only) or "
                         "mimo4_decode_b256 (prefill + decode); default mimo4_decode_b256, or nanomamba3 "
                         "with --backward")
    ap.add_argument("--decode-steps", type=int, default=None, help="override the decode steps per step")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (m3_backward) of the workload's prefill instead "
                         "(default workload for it: nanomamba3, the training shape)")
    ap.add_argument("--fused", action="store_true",
                    help="run the fused layer prologue/epilogue (m3_prefill_fused, m3_decode_step_fused): "
                         "per-token A, RMSNorm and bias of B and C, output gate; with --backward, the "
                         "backward with a per-token decay rate A_t (m3_backward_per_token_A)")
    ap.add_argument("--varlen", action="store_true",
                    help="pack the batch's sequences with seeded lengths uniform in [L/4, L] "
                         "(m3_prefill_varlen; with --backward, m3_backward_varlen) instead of equal lengths L")
    ap.add_argument("--state-dtype", default="fp32", choices=("fp32", "bf16"),
                    help="dtype of the state in HBM (bf16: reduced-precision state, fp32 math)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--check-slices", type=int, default=2,
                    help="(b,h) slices of the run checked against the oracle in the CPU-baseline leg "
                         "(none with --no-cpu-baseline)")
    ap.add_argument("--probe-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (known bytes) to calibrate HBM counters")
    ap.add_argument("--groups", type=int, default=None,
                    help="override the workload's B/C/theta group count G (e.g. 64 = G = H: per-head B, C, theta)")
    ap.add_argument("--no-intra-chunk", action="store_true",
                    help="skip the single-chunk (L = chunk) measurement of the intra-chunk contractions")
    return ap.parse_args()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size timed with HIP events: bytes read plus bytes
    written per second (the secondary denominator next to the 8 TB/s HBM peak)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9


def intra_chunk_flops(cfg, tokens):
    """Useful MFMA-shaped flops of single-chunk sequences: the masked block C~B~^T (once per
    group) and its product with X, and the chunk-state contraction; the inter-chunk term reads
    a zero state here and is not counted."""
    G, H, P, N, R, Q = cfg.ngroups, cfg.nheads, cfg.headdim, cfg.dstate, cfg.rank, cfg.chunk
    return 2 * (tokens * G * R * R * N * (Q + 1) / 2 + tokens * H * (R * R * P * (Q + 1) / 2 + R * N * P))


def intra_chunk_counters(name):
    """Matrix-core figures of the single-chunk workload's scan kernel from the committed rocprofv3
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "intra_chunk_mfma_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_sha") != source_sha(*rec["source_files"]):
            return None
        k = next(iter(rec["workloads"][name]["kernels"].values()))
        return {"mfma_busy_rocprof": round(k["mfma_util_percent"] / 100.0, 4),
                "executed_frac_of_peak": round(k["executed_frac_of_peak"], 4),
                "executed_over_useful": round(k["executed_over_useful"], 3),
                "source": "profiles/intra_chunk_mfma_counters.json"}
    except Exception:
        return None


def measure_intra_chunk(torch, dev, name="mimo4_chunk64_b4096", reps=3):
    """Prefill of the single-chunk workload (every sequence one chunk): time, useful
    intra-chunk flops against the bf16 peak, algorithmic bytes against HBM."""
    from state_space_sequence_scan_amd import inputs, m3scan
    from state_space_sequence_scan_amd.configs import INTRA_CHUNK
    cfg = INTRA_CHUNK[name]
    d = inputs.draw_config(cfg, device=dev)
    args = [d[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C", "D")]
    y = torch.empty_like(d["x"])
    _, st = m3scan.prefill(*args, cfg.chunk, y=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        m3scan.prefill(*args, cfg.chunk, y=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tok = cfg.batch * cfg.seqlen
    flops = intra_chunk_flops(cfg, tok)
    pre_bytes, _ = algorithmic_bytes(cfg, cfg.seqlen, 0)
    tflops = flops / (ms / 1e3) / 1e12
    out = {"workload": cfg.label, "name": name, "ms": round(ms, 4), "tokens_per_s": round(tok / (ms / 1e3), 1),
           "useful_mfma_tflops": round(tflops, 2), "useful_mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
           "alg_GB_per_s": round(pre_bytes / (ms / 1e3) / 1e9, 1),
           "hbm_frac": round(pre_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "mfma_frac_at_hbm_roofline": round(flops / (pre_bytes / (HBM_PEAK_GBS * 1e9)) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "counters": intra_chunk_counters(name)}
    del d, args, y, st
    return out


def fused_extra_bytes(cfg, L, steps, tokens=None):
    """Extra bytes of the fused prologue/epilogue: the gate input z (laid out as y) and the
    per-token A, per (token, head), for the prefill and for one decode step."""
    s = 2 if cfg.io_dtype == "bf16" else 4
    tok = cfg.batch * L if tokens is None else tokens
    per = cfg.nheads * (cfg.rank * cfg.headdim * s + 4)
    return tok * per, (cfg.batch * per if steps else 0)


def algorithmic_bytes(cfg, L, steps, state_bytes=4, tokens=None):
    """Bytes the method must move: every input read once and every output written once
    (the terms below); state_bytes is 4 for an fp32 state, 2 for a bf16 state; tokens is the number of
    prefill tokens over all sequences (batch * L unless the lengths vary)."""
    s = 2 if cfg.io_dtype == "bf16" else 4
    b, H, G, P, N, R = cfg.batch, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank
    tok = b * L if tokens is None else tokens
    pre = 0
    if tok > 0:
        pre += tok * H * (2 * R * P * s + 8)                # x read, y write, dt, lambda
        pre += tok * G * (2 * N * R * s + 4 * (N // 2))     # B, C, theta
        pre += b * H * N * P * state_bytes                  # state out
        pre += b * (G * R * N + H * R * P) * s              # carry out
        pre += 8 * H
    dec = 0
    if steps > 0:
        dec += 2 * b * H * N * P * state_bytes              # state read + write
        dec += b * H * (3 * R * P * s + 8)                  # x_t, x_last read, y_t write, dt, lambda
        dec += b * G * (3 * R * N * s + 4 * (N // 2))       # B_t, C_t, b_last, theta
        dec += 8 * H
    return pre, dec


def prefill_flops(cfg, L, tokens=None):
    """Useful MFMA-shaped flops of the chunked prefill (causal half of each chunk block)."""
    b, H, G, P, N, R, Q = cfg.batch, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank, cfg.chunk
    tok = b * L if tokens is None else tokens
    return 2 * (tok * G * R * R * N * (Q + 1) / 2 + tok * H * (R * R * P * (Q + 1) / 2 + 2 * R * N * P))


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "state_space_sequence_scan_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_file, src_names, per_launch_alg):
    """HBM bytes per launch from a committed counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_sha") != source_sha(*src_names):
            return None
        return float(rec["hbm_bytes_per_dispatch"])
    except Exception:
        return None


def mfma_util_rocprof(workload):
    """MFMA busy fraction (rocprofv3 MfmaUtil) of the workload's output-pass scan kernel from
    the committed counter summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "prefill_mfma_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_sha") != source_sha(*rec["source_files"]):
            return None
        kernels = rec["workloads"][workload]["kernels"]
        # output pass, no gate or norm, one sequence per workgroup
        full = next(v for k, v in kernels.items() if k.endswith("true, false, false, false>"))
        return round(full["mfma_util_percent"] / 100.0, 4)
    except Exception:
        return None


def main():
    args = parse()
    if args.workload is None:
        args.workload = "nanomamba3" if args.backward else "mimo4_decode_b256"
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan runs on a single MI355X "
              "(multi-GPU sharding is a design note, not implemented); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dataclasses

    from state_space_sequence_scan_amd import CONFIGS, inputs, m3scan
    from state_space_sequence_scan_amd.configs import INTRA_CHUNK

    cfg = CONFIGS[args.workload] if args.workload in CONFIGS else INTRA_CHUNK[args.workload]
    if args.groups is not None:
        if cfg.nheads % args.groups != 0:
            sys.exit(f"--groups {args.groups} does not divide the {cfg.nheads} heads")
        cfg = dataclasses.replace(cfg, ngroups=args.groups,
                                  label=cfg.label + f"; {args.groups} B/C/theta groups"
                                        + (" (per head)" if args.groups == cfg.nheads else ""))
    if args.backward:
        return run_backward(args, cfg)
    state_dtype = torch.bfloat16 if args.state_dtype == "bf16" else torch.float32
    state_bytes = 2 if args.state_dtype == "bf16" else 4
    steps_dec = cfg.decode_steps if args.decode_steps is None else args.decode_steps
    L = cfg.seqlen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m3scan.lib()
    stream = torch.cuda.current_stream(dev)

    if args.probe_copy:
        src = torch.empty(2**28, dtype=torch.float32, device=dev)   # 1 GiB read + 1 GiB written
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy_gbs = copy_bandwidth(torch, dev)

    t_gen = time.time()
    d = inputs.draw_config(cfg, device=dev)
    dd = inputs.draw_decode(cfg, steps_dec, device=dev) if steps_dec > 0 else None
    lens = np.full(cfg.batch, L, dtype=np.int64)
    if args.varlen:   # seeded length mix; the packed arrays hold each sequence's first lens[i] tokens
        lens = np.random.default_rng(cfg.seed + 7).integers(max(L // 4, 1), L + 1, cfg.batch)
        starts = np.concatenate([[0], np.cumsum(lens)])
        cu = torch.tensor(starts, dtype=torch.int64, device=dev)
        dp = {k: torch.cat([d[k][i, :int(lens[i])] for i in range(cfg.batch)]).contiguous()
              for k in ("x", "dt", "lam", "theta", "B", "C")}
        y = torch.empty_like(dp["x"])
    else:
        y = torch.empty_like(d["x"])
    ydec = torch.empty((max(steps_dec, 1),) + tuple(d["x"][:, 0].shape), dtype=d["x"].dtype, device=dev)
    fz = fzd = None
    if args.fused:   # seeded fusion inputs: per-token A, norm weights and biases (R, N), gate z
        gf = torch.Generator(device=dev).manual_seed(cfg.seed + 23)
        Rr, Nn = cfg.rank, cfg.dstate
        fz = {"A_t": -torch.exp(torch.rand(d["dt"].shape, generator=gf, device=dev) * math.log(16.0)),
              "b_norm_w": 1.0 + 0.3 * torch.randn((Rr, Nn), generator=gf, device=dev),
              "c_norm_w": 1.0 + 0.3 * torch.randn((Rr, Nn), generator=gf, device=dev),
              "b_bias": 0.02 + 0.05 * torch.randn((Rr, Nn), generator=gf, device=dev),
              "c_bias": 0.02 + 0.05 * torch.randn((Rr, Nn), generator=gf, device=dev),
              "z": torch.randn(d["x"].shape, generator=gf, device=dev).to(d["x"].dtype)}
        if steps_dec:
            fzd = {"A_t": -torch.exp(torch.rand((steps_dec,) + tuple(d["dt"][:, 0].shape), generator=gf, device=dev)
                                     * math.log(16.0)),
                   "z": torch.randn((steps_dec,) + tuple(d["x"][:, 0].shape), generator=gf, device=dev).to(d["x"].dtype)}
        if args.varlen:   # the per-token pieces packed like the other inputs
            dpf = {k: torch.cat([fz[k][i, :int(lens[i])] for i in range(cfg.batch)]).contiguous()
                   for k in ("A_t", "z")}
            dpf.update({k: fz[k] for k in ("b_norm_w", "c_norm_w", "b_bias", "c_bias")})
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def one_step(record=None):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        if args.varlen and args.fused:
            _, st = m3scan.prefill_varlen_fused(dp["x"], dp["dt"], d["A"], dp["lam"], dp["theta"], dp["B"],
                                                dp["C"], d["D"], cu, L, cfg.chunk, **dpf, y=y,
                                                state_dtype=state_dtype)
        elif args.varlen:
            _, st = m3scan.prefill_varlen(dp["x"], dp["dt"], d["A"], dp["lam"], dp["theta"], dp["B"],
                                          dp["C"], d["D"], cu, L, cfg.chunk, y=y, state_dtype=state_dtype)
        elif args.fused:
            _, st = m3scan.prefill_fused(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                                         cfg.chunk, **fz, y=y, state_dtype=state_dtype)
        else:
            _, st = m3scan.prefill(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], d["D"],
                                   cfg.chunk, y=y, state_dtype=state_dtype)
        e1.record(stream)
        for t in range(steps_dec):
            if args.fused:
                m3scan.decode_step_fused(st, dd["x"][t], dd["dt"][t], d["A"], dd["lam"][t], dd["theta"][t],
                                         dd["B"][t], dd["C"][t], d["D"], A_t=fzd["A_t"][t],
                                         b_norm_w=fz["b_norm_w"], c_norm_w=fz["c_norm_w"], b_bias=fz["b_bias"],
                                         c_bias=fz["c_bias"], z=fzd["z"][t], y_t=ydec[t])
            else:
                m3scan.decode_step(st, dd["x"][t], dd["dt"][t], d["A"], dd["lam"][t], dd["theta"][t],
                                   dd["B"][t], dd["C"][t], d["D"], y_t=ydec[t])
        e2.record(stream)
        if record is not None:
            record.append((e0, e1, e2))
        return st

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st = one_step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [a.elapsed_time(b) for a, b, _ in recs]
    dec_ms = [b.elapsed_time(c) for _, b, c in recs]
    step_ms = wall * 1e3 / args.steps
    pre_avg, dec_avg = float(np.mean(pre_ms)), float(np.mean(dec_ms))

    tokens_pre = int(lens.sum())
    tokens_dec = cfg.batch * steps_dec
    value = (tokens_pre + tokens_dec) / (step_ms / 1e3)
    pre_bytes, dec_bytes = algorithmic_bytes(cfg, L, steps_dec, state_bytes, tokens=tokens_pre)
    if args.fused:
        xp, xd = fused_extra_bytes(cfg, L, steps_dec, tokens=tokens_pre)
        pre_bytes += xp
        dec_bytes += xd
    pre_tps = tokens_pre / (pre_avg / 1e3)
    pre_gbs = pre_bytes / (pre_avg / 1e3) / 1e9
    dec_launch_ms = dec_avg / max(steps_dec, 1)
    dec_gbs = dec_bytes / (dec_launch_ms / 1e3) / 1e9 if steps_dec else 0.0
    state_gbs = (2 * cfg.batch * cfg.nheads * cfg.dstate * cfg.headdim * state_bytes) / (dec_launch_ms / 1e3) / 1e9 \
        if steps_dec else 0.0
    flops = prefill_flops(cfg, L, tokens=tokens_pre)

    # Dominant kernel: the one with the larger share of the step.
    if steps_dec and dec_avg >= pre_avg:
        sfx = ("" if args.state_dtype == "fp32" else "_bf16state") + ("_fused" if args.fused else "")
        traffic = pmc_traffic(f"decode_{args.workload}{sfx}_hbm_counters.json",
                              ["m3_decode.hip", "m3_common.h"], dec_bytes)
        roof = {"kernel": f"decode_fast<io bf16, state {args.state_dtype}, N128, P64, R4>", "bound": "hbm",
                "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": dec_bytes, "avg_launch_us": round(dec_launch_ms * 1e3, 2),
                "measured_copy_GB_per_s": round(copy_gbs, 1), "frac_of_measured_copy": round(dec_gbs / copy_gbs, 4)}
    else:
        traffic = pmc_traffic(f"prefill_{args.workload}{'_varlen' if args.varlen else ''}"
                              f"{'_fused' if args.fused else ''}_hbm_counters.json",
                              ["m3_prefill_mfma.hip", "m3_mfma_common.h", "m3_common.h"], pre_bytes)
        roof = {"kernel": "prefill (all kernels of one call)", "bound": "hbm",
                "achieved": round(pre_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(pre_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": pre_bytes, "avg_launch_us": round(pre_avg * 1e3, 2),
                "measured_copy_GB_per_s": round(copy_gbs, 1), "frac_of_measured_copy": round(pre_gbs / copy_gbs, 4)}

    # The CPU-baseline leg, the one place here that runs the oracle: the oracle timed on a
    # bounded sample of the workload and, in the same leg, sampled slices of this very run
    # checked against it.
    check = None
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        def slice_inputs(bi, h, with_decode=True, n=None):
            """(bi, h) slice: its first n prefill tokens (all L by default), then the decode tokens."""
            g = h // (cfg.nheads // cfg.ngroups)
            f = lambda t: t.detach().double().cpu().numpy()
            n = L if n is None else n
            parts = {
                "x": [f(d["x"][bi:bi + 1, :n, h:h + 1])], "dt": [f(d["dt"][bi:bi + 1, :n, h:h + 1])],
                "lam": [f(d["lam"][bi:bi + 1, :n, h:h + 1])],
                "theta": [f(d["theta"][bi:bi + 1, :n, g:g + 1])],
                "B": [f(d["B"][bi:bi + 1, :n, g:g + 1])], "C": [f(d["C"][bi:bi + 1, :n, g:g + 1])]}
            if with_decode and steps_dec:
                parts["x"].append(f(dd["x"][:, bi:bi + 1, h:h + 1].transpose(0, 1)))
                parts["dt"].append(f(dd["dt"][:, bi:bi + 1, h:h + 1].transpose(0, 1)))
                parts["lam"].append(f(dd["lam"][:, bi:bi + 1, h:h + 1].transpose(0, 1)))
                parts["theta"].append(f(dd["theta"][:, bi:bi + 1, g:g + 1].transpose(0, 1)))
                parts["B"].append(f(dd["B"][:, bi:bi + 1, g:g + 1].transpose(0, 1)))
                parts["C"].append(f(dd["C"][:, bi:bi + 1, g:g + 1].transpose(0, 1)))
            if args.fused:
                parts["A_t"] = [f(fz["A_t"][bi:bi + 1, :n, h:h + 1])]
                parts["z"] = [f(fz["z"][bi:bi + 1, :n, h:h + 1])]
                if with_decode and steps_dec:
                    parts["A_t"].append(f(fzd["A_t"][:, bi:bi + 1, h:h + 1].transpose(0, 1)))
                    parts["z"].append(f(fzd["z"][:, bi:bi + 1, h:h + 1].transpose(0, 1)))
            out = {k: np.concatenate(v, axis=1) for k, v in parts.items()}
            out["A"] = f(d["A"][h:h + 1])
            out["D"] = f(d["D"][h:h + 1])
            return out

        order = ("x", "dt", "A", "lam", "theta", "B", "C", "D")
        if args.check_slices > 0:
            rng = np.random.default_rng(cfg.seed)
            errs = []
            for _ in range(args.check_slices):
                bi, h = int(rng.integers(cfg.batch)), int(rng.integers(cfg.nheads))
                n = int(lens[bi])
                si = slice_inputs(bi, h, n=n)
                flags = None
                if args.state_dtype == "bf16":   # state rounded after the prefill and every decode token
                    flags = np.zeros(n + steps_dec, bool)
                    flags[n - 1:] = True
                if args.fused:
                    args_o = [si[k] for k in order]
                    args_o[2] = si["A_t"]
                    yr, hr = oracle.scan_fused(*args_o, b_norm_w=fz["b_norm_w"].double().cpu().numpy(),
                                               c_norm_w=fz["c_norm_w"].double().cpu().numpy(),
                                               b_bias=fz["b_bias"].double().cpu().numpy(),
                                               c_bias=fz["c_bias"].double().cpu().numpy(), z=si["z"],
                                               round_after=flags)
                else:
                    yr, hr = oracle.scan(*[si[k] for k in order], round_after=flags)
                if args.varlen:
                    yg = [y[int(starts[bi]):int(starts[bi + 1]), h:h + 1][None].double().cpu().numpy()]
                else:
                    yg = [y[bi:bi + 1, :, h:h + 1].double().cpu().numpy()]
                if steps_dec:
                    yg.append(ydec[:steps_dec, bi:bi + 1, h:h + 1].transpose(0, 1).double().cpu().numpy())
                yg = np.concatenate(yg, axis=1)
                e = float(np.max(np.abs(yg - yr)) / np.max(np.abs(yr)))
                eh = float(np.max(np.abs(st.h[bi, h].double().cpu().numpy() - hr[0, 0])) / np.max(np.abs(hr)))
                errs.append(max(e, eh))
            check = {"slices": args.check_slices, "max_rel_err": float(max(errs)),
                     "tolerance": 2e-2 if cfg.io_dtype == "bf16" else 1e-4}
        # the timed oracle sample
        threads = oracle.max_threads()
        si = slice_inputs(0, 0)
        t1 = time.perf_counter()
        oracle.scan(*[si[k] for k in order], nthreads=1)
        one = time.perf_counter() - t1
        n = int(max(threads, min(cfg.batch * cfg.nheads, args.cpu_seconds * threads / max(one, 1e-6))))
        n = max(threads, (n // threads) * threads)
        hs = list(range(n))
        batch_in = [slice_inputs(i // cfg.nheads % cfg.batch, i % cfg.nheads) for i in hs]
        # each sampled slice becomes its own head (and group) of one oracle call
        stack = {k: np.concatenate([s[k] for s in batch_in], axis=2)
                 for k in ("x", "dt", "lam", "theta", "B", "C")}
        stack["A"] = np.concatenate([s["A"] for s in batch_in])
        stack["D"] = np.concatenate([s["D"] for s in batch_in])
        t1 = time.perf_counter()
        oracle.scan(*[stack[k] for k in order], nthreads=threads)
        sec = time.perf_counter() - t1
        tok_per_slice = L + steps_dec
        # tokens of the full workload carry all H heads: (slice-tokens / H) per second
        cpu = {"value": round(n * tok_per_slice / cfg.nheads / sec, 2), "unit": "tokens/s",
               "cores": threads, "kind": "oracle",
               "sample": f"{n} (batch, head) slices of the workload, {tok_per_slice} tokens each "
                         f"({L} prefill + {steps_dec} decode), fp64 sequential loop, "
                         f"{sec:.1f} s; scaled to whole-workload tokens (1/{cfg.nheads} per slice-token)",
               "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
               "single_thread": oracle_single_thread(oracle, np)}

    intra = None
    if not args.no_intra_chunk and args.workload == "mimo4_decode_b256":
        del d, dd, y, ydec, st
        torch.cuda.empty_cache()
        intra = measure_intra_chunk(torch, dev)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.io_dtype == "bf16" else "fp32",
        "data": "synthetic (seeded torch generators on the GPU; distributions of the workload)",
        "config": {"workload": cfg.label + (f"; packed lengths uniform in [{max(L // 4, 1)}, {L}], "
                                            f"{tokens_pre} tokens" if args.varlen else "")
                               + ("; fused per-token A, BCNorm and bias of B and C, output gate" if args.fused else ""),
                   "name": cfg.name, "batch": cfg.batch, "prefill_len": L,
                   "decode_steps": steps_dec, "heads": cfg.nheads, "groups": cfg.ngroups,
                   "headdim": cfg.headdim, "dstate": cfg.dstate, "rank": cfg.rank, "chunk": cfg.chunk,
                   "io_dtype": cfg.io_dtype, "state_dtype": args.state_dtype},
        "prefill": {"ms": round(pre_avg, 4), "tokens_per_s": round(pre_tps, 1),
                    "alg_GB_per_s": round(pre_gbs, 1), "hbm_frac": round(pre_gbs / HBM_PEAK_GBS, 4),
                    "mfma_tflops": round(flops / (pre_avg / 1e3) / 1e12, 2),
                    "mfma_frac": round(flops / (pre_avg / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                    "mfma_busy_rocprof": (None if (args.fused or args.varlen or args.state_dtype != "fp32")
                                          else mfma_util_rocprof(args.workload))},
        "decode": ({"ms_total": round(dec_avg, 4), "us_per_step": round(dec_launch_ms * 1e3, 2),
                    "steps_per_s": round(1e3 / dec_launch_ms, 1), "state_GB_per_s": round(state_gbs, 1),
                    "alg_GB_per_s": round(dec_gbs, 1), "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4)}
                   if steps_dec else None),
        "roofline": roof,
        "intra_chunk": intra,
        "cpu_baseline": cpu,
        "parity_check": check,
        "input_gen_s": round(t_gen, 2),
    }
    print(json.dumps(out), flush=True)


def oracle_single_thread(oracle, np):
    """The oracle on one host thread: the whole single SISO layer workload (b1, L256, H4, fp32),
    and a sample of nanomamba3 (batch, head) slices (2048 tokens each), as whole-workload
    tokens per second."""
    from state_space_sequence_scan_amd import CONFIGS, inputs
    order = ("x", "dt", "A", "lam", "theta", "B", "C", "D")
    out = {}
    c0 = CONFIGS["siso_l256_fp32"]
    d = {k: v.double().numpy() for k, v in inputs.draw_config(c0, device="cpu").items()}
    oracle.scan(*[d[k] for k in order], nthreads=1)   # library loaded, pages touched
    reps, t = 0, time.perf_counter()
    while reps < 5 or time.perf_counter() - t < 0.5:   # about a millisecond per run: repeat
        oracle.scan(*[d[k] for k in order], nthreads=1)
        reps += 1
    out["siso_l256_fp32"] = {"tokens_per_s": round(reps * c0.tokens / (time.perf_counter() - t), 1),
                             "sample": f"the whole workload (1 x 256 tokens x 4 heads), {reps} runs"}
    c1 = CONFIGS["nanomamba3"]
    ns = 4   # heads 0..3 of batch element 0 (B, C and theta are shared by all heads: G = 1)
    d = {k: v.double().numpy() for k, v in inputs.draw_config(c1, device="cpu", batch=1).items()}
    for k in ("x", "dt", "lam"):
        d[k] = d[k][:, :, :ns]
    for k in ("A", "D"):
        d[k] = d[k][:ns]
    t = time.perf_counter()
    oracle.scan(*[d[k] for k in order], nthreads=1)
    sec = time.perf_counter() - t
    out["nanomamba3"] = {"tokens_per_s": round(ns * c1.seqlen / c1.nheads / sec, 1),
                         "sample": f"{ns} (batch, head) slices of 2048 tokens, scaled to whole-workload tokens "
                                   f"(1/{c1.nheads} per slice-token)"}
    return out


def backward_flops(cfg, L):
    """fp32 arithmetic of the adjoint method per workload: one forward step and one
    reverse step of the recurrence per (token, head) over the N x P state, counted as
    14 R + 33 flops per state element: 2 R + 8 for the forward step that recomputes the
    state and 12 R + 25 for the adjoint step and the gradient contractions."""
    return cfg.batch * L * cfg.nheads * cfg.dstate * cfg.headdim * (14 * cfg.rank + 33)


def backward_bytes(cfg, L):
    """Bytes the backward must move: its inputs once (x, dy, dt, lambda per head; B, C,
    theta per group) and its gradients once (fp32)."""
    s = 2 if cfg.io_dtype == "bf16" else 4
    b, H, G, P, N, R = cfg.batch, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank
    tok = b * L
    rd = tok * H * (2 * R * P * s + 8) + tok * G * (2 * N * R * s + 4 * (N // 2))
    wr = tok * H * (R * P * 4 + 8) + tok * G * (2 * N * R * 4 + 4 * (N // 2))
    return rd + wr


def run_backward(args, cfg):
    import numpy as np
    import torch

    from state_space_sequence_scan_amd import inputs, m3scan

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m3scan.lib()
    stream = torch.cuda.current_stream(dev)
    if args.probe_copy:
        src = torch.empty(2**28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    L = cfg.seqlen
    names = ("x", "dt", "A", "lam", "theta", "B", "C", "D")
    d = inputs.draw_config(cfg, device=dev)
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 11)
    dy = torch.randn(d["x"].shape, generator=gen, device=dev).to(d["x"].dtype)
    if args.fused:   # per-token decay rate A_t, drawn like the per-head rates: -exp(U(0, ln 16))
        d["At"] = -torch.exp(torch.rand(d["dt"].shape, generator=gen, device=dev) * math.log(16.0))
    dims = m3scan.make_dims(cfg.batch, L, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank,
                            1, m3scan.M3_BF16 if cfg.io_dtype == "bf16" else m3scan.M3_F32)
    ws = torch.empty(m3scan.backward_workspace_size(dims), dtype=torch.uint8, device=dev)
    lens = np.full(cfg.batch, L, dtype=np.int64)
    if args.varlen:   # the prefill's seeded length mix; each sequence keeps its first lens[i] tokens
        lens = np.random.default_rng(cfg.seed + 7).integers(max(L // 4, 1), L + 1, cfg.batch)
        starts = np.concatenate([[0], np.cumsum(lens)])
        cu = torch.tensor(starts, dtype=torch.int64, device=dev)
        dp = {k: torch.cat([v[i, :int(lens[i])] for i in range(cfg.batch)]).contiguous()
              for k, v in list(d.items()) + [("dy", dy)] if v.dim() > 1}

        def bwd(g=None):
            if args.fused:
                return m3scan.backward_per_token_A(*[dp["At"] if k == "A" else dp[k] if k in dp else d[k]
                                                     for k in names], dp["dy"], cu_seqlens=cu, max_seqlen=L,
                                                   workspace=ws, grads=g, want_state_grads=False)
            return m3scan.backward_varlen(*[dp[k] if k in dp else d[k] for k in names], dp["dy"], cu, L,
                                          workspace=ws, grads=g, want_state_grads=False)
    else:
        def bwd(g=None):
            if args.fused:
                return m3scan.backward_per_token_A(*[d["At"] if k == "A" else d[k] for k in names], dy,
                                                   workspace=ws, grads=g, want_state_grads=False)
            return m3scan.backward(*[d[k] for k in names], dy, workspace=ws, grads=g, want_state_grads=False)
    grads = bwd()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        bwd(grads)
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1 = ev(), ev()
        e0.record(stream)
        bwd(grads)
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in times]))
    step_ms = wall * 1e3 / args.steps
    tokens = int(lens.sum())
    flops = backward_flops(cfg, L) * tokens / (cfg.batch * L)
    nbytes = backward_bytes(cfg, L) * tokens / (cfg.batch * L)
    tflops = flops / (ms / 1e3) / 1e12
    traffic = pmc_traffic(f"backward_{args.workload}{'_varlen' if args.varlen else ''}"
                          f"{'_per_token_A' if args.fused else ''}_hbm_counters.json",
                          ["m3_backward.hip", "m3_common.h"], nbytes)
    parts, tpp = m3scan.backward_parts(dims)
    passes = "local + combine + " if parts > 1 else ""
    roof = {"kernel": f"{passes}bwd_scan<io {cfg.io_dtype}, R{cfg.rank}{', per-token A' if args.fused else ''}> + group sums "
                      f"({parts} pieces of {tpp} tokens per (b, h))", "bound": "alu",
            "achieved": round(tflops, 3), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / FP32_VALU_PEAK_TFLOPS, 4), "traffic": traffic,
            "alg_flops_per_launch": flops, "alg_bytes_per_launch": nbytes,
            "alg_GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1), "avg_launch_us": round(ms * 1e3, 1)}

    # The CPU-baseline leg (the oracle timed on a bounded sample, and sampled slices of this
    # run checked against it), the one place here that runs the oracle.
    check = cpu = None
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: t.detach().double().cpu().numpy()

        def grad_slice(k, bi, h):   # the per-head gradient k of sequence bi, head h, as (1, len, 1, ...)
            if args.varlen:
                return grads[k][int(starts[bi]):int(starts[bi + 1]), h:h + 1][None].double().cpu().numpy()
            return grads[k][bi:bi + 1, :, h:h + 1].double().cpu().numpy()

        def slice_inputs(bi, h, packed=args.varlen):
            g = h // (cfg.nheads // cfg.ngroups)
            if packed:
                s0, s1 = int(starts[bi]), int(starts[bi + 1])
                return {"x": f(dp["x"][s0:s1, h:h + 1][None]), "dt": f(dp["dt"][s0:s1, h:h + 1][None]),
                        "lam": f(dp["lam"][s0:s1, h:h + 1][None]), "theta": f(dp["theta"][s0:s1, g:g + 1][None]),
                        "B": f(dp["B"][s0:s1, g:g + 1][None]), "C": f(dp["C"][s0:s1, g:g + 1][None]),
                        "A": f(dp["At"][s0:s1, h:h + 1][None]) if args.fused else f(d["A"][h:h + 1]),
                        "D": f(d["D"][h:h + 1]), "dy": f(dp["dy"][s0:s1, h:h + 1][None])}
            return {"x": f(d["x"][bi:bi + 1, :, h:h + 1]), "dt": f(d["dt"][bi:bi + 1, :, h:h + 1]),
                    "lam": f(d["lam"][bi:bi + 1, :, h:h + 1]), "theta": f(d["theta"][bi:bi + 1, :, g:g + 1]),
                    "B": f(d["B"][bi:bi + 1, :, g:g + 1]), "C": f(d["C"][bi:bi + 1, :, g:g + 1]),
                    "A": f(d["At"][bi:bi + 1, :, h:h + 1]) if args.fused else f(d["A"][h:h + 1]),
                    "D": f(d["D"][h:h + 1]), "dy": f(dy[bi:bi + 1, :, h:h + 1])}

        if args.check_slices > 0:
            rng = np.random.default_rng(cfg.seed)
            errs = []
            for _ in range(args.check_slices):
                bi, h = int(rng.integers(cfg.batch)), int(rng.integers(cfg.nheads))
                si = slice_inputs(bi, h)
                ref = oracle.scan_backward(*[si[k] for k in names], si["dy"])
                # per-head gradients (group-shared and batch-summed ones mix other slices)
                for k in ("dx", "ddt", "dlam"):
                    gv = grad_slice(k, bi, h)
                    errs.append(float(np.max(np.abs(gv - ref[k])) / max(np.max(np.abs(ref[k])), 1e-30)))
            check = {"slices": args.check_slices, "max_rel_err": max(errs), "tolerance": 1e-3,
                     "compared": "dx, ddt, dlambda of sampled (b, h) slices"}
        # the timed oracle sample
        threads = oracle.max_threads()
        si = slice_inputs(0, 0, packed=False)   # the oracle's rate on whole-length slices
        t1 = time.perf_counter()
        oracle.scan_backward(*[si[k] for k in names], si["dy"], nthreads=1)
        one = time.perf_counter() - t1
        # the oracle parallelises over batch elements: each sampled slice is its own batch element
        n = int(max(threads, min(cfg.batch * cfg.nheads, args.cpu_seconds * threads / max(one, 1e-6))))
        n = max(threads, (n // threads) * threads)
        sl = [slice_inputs(i // cfg.nheads % cfg.batch, i % cfg.nheads, packed=False) for i in range(n)]
        st = {k: np.concatenate([s[k] for s in sl], axis=0) for k in ("x", "dt", "lam", "theta", "B", "C", "dy")}
        t1 = time.perf_counter()
        # A (per head), D differ per slice's head; the sample uses head 0's values for all (same
        # cost).  A per-token A_t is each slice's own.
        a_cpu = np.concatenate([s["A"] for s in sl], axis=0) if args.fused else sl[0]["A"]
        oracle.scan_backward(st["x"], st["dt"], a_cpu, st["lam"], st["theta"], st["B"], st["C"],
                             sl[0]["D"], st["dy"], nthreads=threads)
        sec = time.perf_counter() - t1
        cpu = {"value": round(n * L / cfg.nheads / sec, 2), "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{n} (batch, head) slices of the workload, {L} tokens each, backward "
                         f"(fp64 adjoint loop), {sec:.1f} s; scaled to whole-workload tokens "
                         f"(1/{cfg.nheads} per slice-token)"}

    out = {
        "metric": BWD_METRIC, "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded torch generators on the GPU; distributions of the workload; "
                "dy ~ N(0,1))",
        "config": {"workload": cfg.label + "; backward pass (gradients of every input)"
                               + ("; per-token decay rate A_t" if args.fused else "")
                               + (f"; packed lengths uniform in [{max(L // 4, 1)}, {L}], {tokens} tokens"
                                  if args.varlen else ""), "name": cfg.name,
                   "batch": cfg.batch, "seqlen": L, "heads": cfg.nheads, "groups": cfg.ngroups,
                   "headdim": cfg.headdim, "dstate": cfg.dstate, "rank": cfg.rank, "io_dtype": cfg.io_dtype},
        "backward": {"ms": round(ms, 4), "tokens_per_s": round(tokens / (ms / 1e3), 1),
                     "tflops": round(tflops, 3), "alg_GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "workspace_GB": round(ws.numel() / 1e9, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_check": check,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
