#!/usr/bin/env python3
"""Throughput of the Mamba-2 chunked SSD forward pass (libssd) on one MI355X.

One step = one ssd_fwd through the C ABI: the whole hot path over one batch of
synthetic input with the default tile choices: chunk_state (with the
within-chunk running sums) -> state_pass -> stage 3 (the resident-tile kernel
where it is built).  Inputs are resident
in HBM before timing starts.  The headline is the median of the timed steps
with the 256 MB last-level cache flushed before each by reading a 512 MiB
buffer (outside the events: the cache then holds clean, unrelated lines);
p10/p90, the mean, the median after a 512 MiB write instead (whose dirty lines
the timed step then has to write back) and the warm back-to-back rate are
reported beside it.  Prints one JSON line.

Default workload: the Mamba-2 2.7B-shaped layer, batch 2 x seqlen 8192,
80 heads, headdim 64, dstate 128, 1 group, chunk 256, bf16 x/B/C, fp32
dt/A/D and a nonzero fp32 initial state.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --raw-dt           (dt given raw: bias + softplus applied in stage 1)
  python bench.py --mode decode      (token-sequential mode: one ssd_step per step)
  python bench.py --tune [--workload NAME]   (time every tile choice with ssd_tune; one
                                      JSON line with each choice's mean ms and the fastest)
  python bench.py --copy-probe       (plain copy kernel, for counter scaling)
  python bench.py --graph            (each step replays one captured HIP graph of the pass;
                                      matters for the launch-bound small workloads)
  python bench.py --peaks            (achievable peaks on this GPU, for reference: a large
                                      bf16 GEMM through torch/hipBLASLt and a 1 GiB device copy)

  python bench.py --mode bwd         (backward pass: one ssd_bwd per step, upstream gradients
                                      dy and dfinal resident like the inputs)

Decode mode: the same 2.7B-shaped layer (80 heads, headdim 64, dstate 128,
1 group, bf16 x/B/C) at batch 128, one token per step, advancing a resident
fp32 state in place; the kernel streams the state (read + write) and is
measured against the HBM roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_MFMA = 2.5e15     # dense bf16 MFMA, MI355X published
PEAK_FP32_MFMA = 157.3e12   # dense fp32 MFMA
PEAK_HBM = 8.0e12           # HBM3E bytes/s
METRIC = "SSD fwd tokens/sec (batch·seqlen) at 1 MI355X; % of bf16 MFMA roofline"
DECODE_METRIC = "SSD decode tokens/sec (batch, one token per step) at 1 MI355X; % of HBM roofline"
BWD_METRIC = "SSD bwd tokens/sec (batch·seqlen) at 1 MI355X; % of MFMA roofline"
COPY_PROBE_BYTES = 1 << 30
DEFAULT_WORKLOAD = "mamba2_2p7b"
# committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries of the dominant kernel,
# valid while the sources they were taken from are unchanged
TRAFFIC = {
    "fused_fwd_kernel": ("fused_fwd_{workload}_traffic.txt", ["fused_fwd.hip", "ssd_device.hpp"]),
    "compute_out": ("compute_out_{workload}_traffic.txt", ["compute_out.hip", "ssd_device.hpp"]),
    "out_resident_kernel": ("out_resident_{workload}_traffic.txt", ["out_resident.hip", "ssd_device.hpp"]),
}


def counts(p):
    """Algorithmic flops and bytes (see the measurement section of the design doc)."""
    Bz, L, H, P, N, G, Q = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups, p.chunk_size
    T = -(-L // Q)
    Lp = T * Q
    e = 2 if p.io_dtype == "bf16" else 4
    per_chunk_head_intra = Q * (Q + 1) * (N + P)        # causal C B^T and S x
    per_chunk_head_state = 2 * Q * P * N                # one of: chunk state, C H^T
    f_path = Bz * H * T * (per_chunk_head_intra + 2 * per_chunk_head_state)
    f_out = Bz * H * T * (per_chunk_head_intra + per_chunk_head_state)
    init = 1 if p.init_std is not None else 0
    b_min = (2 * Bz * L * H * P * e + 2 * Bz * L * G * N * e + 4 * Bz * L * H + 8 * H
             + 4 * Bz * H * P * N * (1 + init))
    b_out = (2 * Bz * L * H * P * e            # x read, y written
             + Bz * H * T * P * N * e          # chunk-start states read
             + 2 * 4 * Bz * H * Lp             # G and dt in [b, h, token] order
             + 2 * Bz * L * G * N * e          # B and C rows
             + 4 * H)                          # D
    return dict(f_path=f_path, f_out=f_out, b_min=b_min, b_out=b_out,
                units_out=Bz * H * T, tokens=Bz * L)


def source_digest(kernel):
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "state_space_sequence_03_amd", "csrc", f) for f in TRAFFIC[kernel][1]]
    files.append(os.path.join(ROOT, "state_space_sequence_03_amd", "build.py"))   # compile flags
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counters, or
    None when the file is missing or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", TRAFFIC[kernel][0].format(workload=workload))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inputs, prob, target_seconds=15.0, gpu_out=None, raw_dt=False):
    """Time the fp64 oracle (the token recurrence, OpenMP over (batch, head)) on
    the host, on a bounded sample of the workload: the first `nh` heads of every
    batch over the whole sequence, sized from a short probe to take about
    `target_seconds`, or the whole workload when that fits.  Tokens/s is scaled
    to the full head count.  With gpu_out = (y, final_state) from the GPU
    run, the oracle's outputs of the sampled heads are also compared with it
    (rel-L2 over the sampled part, max-abs / max|ref|)."""
    import numpy as np
    import oracle

    nthreads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    arrs = {k: (None if v is None else oracle.as_f32(v)) for k, v in inputs.items()}
    H, hpg = prob.nheads, prob.nheads // prob.ngroups

    def run(nh):
        g = max(1, nh // hpg)
        sel = lambda a: a[:, :, :nh]
        init = arrs["init_state"]
        t0 = time.perf_counter()
        out = oracle.recurrence(sel(arrs["x"]), sel(arrs["dt"]), arrs["A"][:nh], arrs["B"][:, :, :g],
                                arrs["C"][:, :, :g], arrs["D"][:nh],
                                None if init is None else init[:, :nh], nthreads=nthreads)
        return time.perf_counter() - t0, out

    def legal(nh):   # head counts whose group mapping matches the full problem
        nh = max(1, min(H, nh))
        return nh if nh <= hpg else nh // hpg * hpg

    probe_heads = legal(min(H, max(1, nthreads // max(1, prob.batch))))
    probe, _ = run(probe_heads)
    nh = legal(int(target_seconds / max(probe, 1e-6) * probe_heads))
    dt, out = run(nh)
    reps = 1
    if nh == H and dt < target_seconds:
        # the whole workload takes less than the target: repeat it, so the
        # figure averages over about target_seconds of host work
        reps = max(1, min(200, int(round(target_seconds / max(dt, 1e-6)))))
        dt = dt + sum(run(nh)[0] for _ in range(reps - 1))
    tok_s = reps * prob.batch * prob.seqlen * (nh / H) / dt
    if nh == H:
        sample = ("full workload: %d (batch, head) pairs x %d tokens, run %d times"
                  % (prob.batch * H, prob.seqlen, reps))
    else:
        sample = ("heads 0..%d of %d in each of %d batches, %d tokens each; tokens/s scaled by %d/%d"
                  % (nh - 1, H, prob.batch, prob.seqlen, nh, H))
    res = {"value": tok_s, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
           "sample": sample, "seconds": round(dt, 3)}
    if gpu_out is not None and not raw_dt:
        y_ref, fin_ref, _ = out

        def err(got, ref):
            g = got.float().cpu().double().numpy()
            dlt = g - ref
            return (float(np.linalg.norm(dlt) / max(np.linalg.norm(ref), 1e-300)),
                    float(np.max(np.abs(dlt)) / max(np.max(np.abs(ref)), 1e-300)))
        yr, ya = err(gpu_out[0][:, :, :nh], y_ref)
        fr, fa = err(gpu_out[1][:, :nh], fin_ref)
        res["parity"] = {"heads_compared": "%d of %d (every batch, whole sequence)" % (nh, H),
                         "y_rel_l2": yr, "y_max_abs_frac": ya,
                         "final_rel_l2": fr, "final_max_abs_frac": fa,
                         "tolerance": {"rel_l2": 5e-3, "max_abs_frac": 2e-2}
                         if prob.io_dtype == "bf16" else {"rel_l2": 1e-5, "max_abs_frac": 1e-4}}
    return res


def bwd_counts(p):
    """Algorithmic flops of the backward pass, per (batch, chunk, head) and in
    all: the causal chunk x chunk products C B^T and dy x^T (once each), the
    three products with them (dx, dB, dC inside the chunk), and five chunk x
    state products (the recomputed chunk state, the reversed one for the
    state gradients, and the carried terms of dx, dB and dC)."""
    Bz, L, H, P, N, Q = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.chunk_size
    T = -(-L // Q)
    pairs = Q * (Q + 1) // 2
    chunk = 2 * pairs * (3 * N + 2 * P)     # the chunk x chunk products
    state = 2 * 5 * Q * P * N               # the chunk x state products
    per_unit = chunk + state
    units = Bz * H * T
    # peak for this mix: every flop at the rate of the MFMA that runs it -- the
    # chunk x chunk products on bf16 MFMA for bf16 io (fp32 MFMA for fp32 io),
    # the state products on the exact fp32 MFMA
    chunk_peak = PEAK_BF16_MFMA if p.io_dtype == "bf16" else PEAK_FP32_MFMA
    peak = per_unit / (chunk / chunk_peak + state / PEAK_FP32_MFMA)
    return dict(per_unit=per_unit, chunk_per_unit=chunk, state_per_unit=state, units=units,
                flops=per_unit * units, tokens=Bz * L, peak=peak)


def bench_bwd(args):
    import torch
    import oracle
    import ssd_synth
    import state_space_sequence_03_amd as ssd

    if args.workload not in ssd_synth.CONFIGS:
        print("unknown workload %r (choose from %s)" % (args.workload, ", ".join(ssd_synth.CONFIGS)),
              file=sys.stderr)
        sys.exit(2)
    prob = ssd_synth.CONFIGS[args.workload]
    seed = ssd_synth.CONFIG_ORDER.index(args.workload)
    inputs = ssd_synth.make_inputs(prob, seed)
    grads = ssd_synth.make_grads(prob, seed)
    dev = torch.device("cuda:0")
    d = {k: (None if v is None else v.to(dev)) for k, v in inputs.items()}
    dy, dfinal = grads["dy"].to(dev), grads["dfinal"].to(dev)
    io = ssd.SSD_BF16 if prob.io_dtype == "bf16" else ssd.SSD_F32
    cprob = ssd.make_problem(prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate,
                             prob.ngroups, prob.chunk_size, io)
    # the default workspace unless --bwd-workspace-bytes asks for another size
    # (ssd_bwd batches the heads to fit it; the results do not change)
    ws_bytes = args.bwd_workspace_bytes or ssd.ssd_bwd_workspace_size(cprob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        return ssd.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], prob.chunk_size,
                           d["init_state"], dy, dfinal, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record()
        step()
        ev[k][1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    ms_pass = sum(a.elapsed_time(b) for a, b in ev) / K
    c = bwd_counts(prob)
    achieved = c["flops"] / (ms_pass * 1e-3)
    line = {
        "metric": BWD_METRIC,
        "value": c["tokens"] / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.io_dtype,
        "data": "synthetic",
        "config": {"workload": prob.name, "pass": "backward", "batch": prob.batch,
                   "seqlen": prob.seqlen, "nheads": prob.nheads, "headdim": prob.headdim,
                   "dstate": prob.dstate, "ngroups": prob.ngroups, "chunk_size": prob.chunk_size,
                   "init_state": prob.init_std is not None, "dfinal": True,
                   "workspace_bytes": ws_bytes},
        # the whole backward call (every kernel of ssd_bwd) bracketed by events on
        # the stream it is enqueued on; the per-kernel split is in the kernel trace
        "roofline": {"kernel": "ssd_bwd (all kernels)", "bound": "mfma",
                     "achieved": achieved / 1e12, "peak": c["peak"] / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / c["peak"], "traffic": None,
                     "flops_per_unit": c["per_unit"], "units_per_launch": c["units"],
                     "peak_mix": "chunk x chunk products at %.1f TFLOP/s, state products at "
                                 "%.1f (fp32 MFMA)" % ((PEAK_BF16_MFMA if prob.io_dtype == "bf16"
                                                        else PEAK_FP32_MFMA) / 1e12,
                                                       PEAK_FP32_MFMA / 1e12),
                     "frac_of_fp32_peak": achieved / PEAK_FP32_MFMA,
                     # every flop priced at the bf16 dense rate, as the forward pass is
                     "frac_of_bf16_peak": achieved / PEAK_BF16_MFMA, "pass_ms": ms_pass},
    }
    if not args.no_cpu_baseline:
        arrs = {k: (None if v is None else oracle.as_f32(v)) for k, v in inputs.items()}
        gy, gf = oracle.as_f32(grads["dy"]), oracle.as_f32(grads["dfinal"])
        heads, t = 0, 0.0
        while t < 10.0 and heads < prob.batch * prob.nheads:
            b, h = heads % prob.batch, heads // prob.batch
            t0 = time.perf_counter()
            oracle.recurrence_bwd(arrs["x"], arrs["dt"], arrs["A"], arrs["B"], arrs["C"],
                                  arrs["D"], arrs["init_state"], gy, gf, heads=[(b, h)])
            t += time.perf_counter() - t0
            heads += 1
        line["cpu_baseline"] = {"value": heads / (prob.batch * prob.nheads) * c["tokens"] / t,
                                "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                "sample": "%d of the %d (batch, head) sequences, whole length, "
                                          "scaled to all heads" % (heads, prob.batch * prob.nheads),
                                "seconds": round(t, 3)}
    print(json.dumps(line), flush=True)


def decode_counts(p):
    """Algorithmic bytes of one decode step: the fp32 state read and written,
    x read and y written, the B and C rows, dt, A and D."""
    Bz, L, H, P, N, G = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups
    e = 2 if p.io_dtype == "bf16" else 4
    return (2 * 4 * Bz * H * P * N + 2 * Bz * L * H * P * e + 2 * Bz * L * G * N * e
            + 4 * Bz * L * H + 8 * H)


DECODE_WORKLOADS = {
    "decode_2p7b_b128": dict(batch=128, seqlen=1, nheads=80, headdim=64, dstate=128, ngroups=1,
                             chunk_size=256, init_std=0.1, name="decode_2p7b_b128"),
}


def bench_decode(args):
    import torch
    import oracle
    import ssd_synth
    import state_space_sequence_03_amd as ssd

    if args.workload in DECODE_WORKLOADS:
        name = args.workload
    elif args.workload == DEFAULT_WORKLOAD:
        name = "decode_2p7b_b128"
    else:
        print("unknown decode workload %r (choose from %s)" % (args.workload, ", ".join(DECODE_WORKLOADS)),
              file=sys.stderr)
        sys.exit(2)
    prob = ssd_synth.Problem(**DECODE_WORKLOADS[name])
    inputs = ssd_synth.make_inputs(prob, 0)
    dev = torch.device("cuda:0")
    d = {k: (None if v is None else v.to(dev)) for k, v in inputs.items()}
    state = d["init_state"].clone()
    y = torch.empty_like(d["x"])

    def step():
        ssd.ssd_step(state, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], out=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record()
        step()
        ev[k][1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    ms_kernel = sum(a.elapsed_time(b) for a, b in ev) / K
    nbytes = decode_counts(prob)
    achieved = nbytes / (ms_kernel * 1e-3)
    line = {
        "metric": DECODE_METRIC,
        "value": prob.batch / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.io_dtype,
        "data": "synthetic",
        "config": {"workload": name, "batch": prob.batch, "tokens_per_step": prob.seqlen,
                   "nheads": prob.nheads, "headdim": prob.headdim, "dstate": prob.dstate,
                   "ngroups": prob.ngroups, "state": "fp32, in place"},
        "roofline": {"kernel": "step", "bound": "hbm", "achieved": achieved / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": achieved / PEAK_HBM,
                     "traffic": None, "bytes_per_launch": nbytes,
                     "kernel_ms": ms_kernel},
    }
    if not args.no_cpu_baseline:
        arrs = {k: (None if v is None else oracle.as_f32(v)) for k, v in inputs.items()}
        nthreads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        reps, t = 0, 0.0
        while t < 10.0 and reps < 2000:
            t0 = time.perf_counter()
            oracle.recurrence(arrs["x"], arrs["dt"], arrs["A"], arrs["B"], arrs["C"], arrs["D"],
                              arrs["init_state"], nthreads=nthreads)
            t += time.perf_counter() - t0
            reps += 1
        line["cpu_baseline"] = {"value": reps * prob.batch / t, "unit": "tokens/s",
                                "cores": nthreads, "kind": "oracle",
                                "sample": "whole decode step (%d sequences x 1 token), run %d times"
                                          % (prob.batch, reps),
                                "seconds": round(t, 3)}
    print(json.dumps(line), flush=True)


def measure_peaks():
    """Achievable MFMA and HBM rates on this GPU, as references beside the
    published peaks: a large bf16 GEMM (torch.matmul, i.e. the vendor GEMM
    library) and a 1 GiB device-to-device copy, each event-timed."""
    import torch
    dev = torch.device("cuda:0")
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    x = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * COPY_PROBE_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    print(json.dumps({"measured_peaks": {
        "bf16_gemm_tflops": gemm_tflops, "gemm": "torch.matmul %dx%dx%d bf16" % (n, n, n),
        "copy_gbs_read_plus_write": copy_gbs, "copy": "1 GiB device copy",
        "published": {"bf16_mfma_tflops": PEAK_BF16_MFMA / 1e12, "hbm_gbs": PEAK_HBM / 1e9}}}),
        flush=True)


def copy_probe():
    import torch
    n = COPY_PROBE_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": COPY_PROBE_BYTES, "launches": 5}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--peaks", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one captured HIP graph of the whole pass")
    ap.add_argument("--mode", choices=("prefill", "decode", "bwd"), default="prefill")
    ap.add_argument("--cumsum-heads", type=int, choices=(0, 4, 16), default=None,
                    help="ssd_config.cumsum_heads (0: running sums inside chunk_state; "
                         "default: the library's choice)")
    ap.add_argument("--bwd-workspace-bytes", type=int, default=0,
                    help="--mode bwd: workspace size to give ssd_bwd (0: its default)")
    ap.add_argument("--tune", action="store_true",
                    help="time every valid tile choice of the forward pass (ssd_tune)")
    ap.add_argument("--kernels", choices=("default", "fused", "staged"), default="default",
                    help="the forward kernels to time: the library's default choice for the "
                         "shape, the single-pass fused kernel, or the four staged kernels")
    ap.add_argument("--evict", choices=("both", "read", "write"), default="both",
                    help="cache eviction before each timed step: read 512 MiB (the headline), "
                         "write 512 MiB (reported beside it), or both (default; a profiler run "
                         "can restrict the timed steps to one kind)")
    ap.add_argument("--raw-dt", action="store_true",
                    help="pass the raw step size and let stage 1 apply bias + softplus")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import ssd_synth
    import state_space_sequence_03_amd as ssd

    if args.copy_probe:
        copy_probe()
        return
    if args.peaks:
        measure_peaks()
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "decode":
        bench_decode(args)
        return
    if args.mode == "bwd":
        bench_bwd(args)
        return
    if args.workload not in ssd_synth.CONFIGS:
        print("unknown workload %r (choose from %s)" % (args.workload, ", ".join(ssd_synth.CONFIGS)),
              file=sys.stderr)
        sys.exit(2)
    prob = ssd_synth.CONFIGS[args.workload]
    seed = ssd_synth.CONFIG_ORDER.index(args.workload)
    inputs = ssd_synth.make_inputs(prob, seed)
    dev = torch.device("cuda:0")
    d = {k: (None if v is None else v.to(dev)) for k, v in inputs.items()}
    Q = prob.chunk_size
    if args.tune:
        default = ssd.ssd_default_config(ssd.make_problem(
            prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate, prob.ngroups, Q,
            ssd.SSD_BF16 if prob.io_dtype == "bf16" else ssd.SSD_F32))
        best, best_ms, rows = ssd.ssd_tune(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], Q,
                                           d["init_state"], reps=max(1, args.steps))
        default_ms = [ms for c, ms in rows if c == default][0]
        print(json.dumps({"metric": "SSD fwd mean ms per pass for each tile choice (ssd_tune)",
                          "workload": args.workload, "reps": max(1, args.steps),
                          "default": default, "default_ms": default_ms,
                          "best": best, "best_ms": best_ms,
                          "speedup_vs_default": default_ms / best_ms,
                          "choices": [dict(c, ms=ms) for c, ms in rows]}), flush=True)
        return
    pr = ssd.make_problem(prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate,
                          prob.ngroups, Q, ssd.SSD_BF16 if prob.io_dtype == "bf16" else ssd.SSD_F32)
    cfg = ssd.ssd_default_config(pr)
    if args.kernels != "default":
        cfg["fused"] = int(args.kernels == "fused")
    if args.cumsum_heads is not None:
        cfg["cumsum_heads"] = args.cumsum_heads
    fused = bool(cfg["fused"])
    ws = torch.empty(ssd.ssd_fwd_workspace_size(pr), dtype=torch.uint8, device=dev)
    y = torch.empty_like(d["x"])
    fin = torch.empty((prob.batch, prob.nheads, prob.headdim, prob.dstate), dtype=torch.float32,
                      device=dev)
    dt_kw = dict(dt_bias=d["dt_bias"], dt_softplus=True) if args.raw_dt else {}
    dt_in = d["dt_raw"] if args.raw_dt else d["dt"]

    def fwd():
        ssd.ssd_fwd(d["x"], dt_in, d["A"], d["B"], d["C"], d["D"], Q, d["init_state"], out=y,
                    final_out=fin, workspace=ws, config=cfg, **dt_kw)

    if args.graph:
        graph_line(args, prob, fwd)
        return

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()

    # timed region: K steps, each after a read of a 512 MiB buffer that
    # evicts the 256 MB last-level cache (outside the events), each bracketed
    # by HIP events on the stream the kernels run on (torch's current stream)
    K = args.steps
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)

    def cold_steps(evict):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(K):
            evict(k)
            evs[k][0].record()
            fwd()
            evs[k][1].record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs), time.perf_counter() - t_start

    def median(v):
        return v[K // 2] if K % 2 else 0.5 * (v[K // 2 - 1] + v[K // 2])

    if args.evict == "write":
        cold, wall = cold_steps(lambda k: flush.fill_(k & 0xFF))
    else:
        cold, wall = cold_steps(lambda k: evict_by_reading(flush))
    cold_mean = sum(cold) / K
    ms_step = median(cold)
    p10, p90 = cold[int(0.1 * (K - 1))], cold[int(round(0.9 * (K - 1)))]
    # secondary: the same after a 512 MiB write, which leaves the cache full of
    # dirty lines that the timed step's own traffic then writes back
    dirty = None
    if args.evict == "both":
        dirty, _ = cold_steps(lambda k: flush.fill_(k & 0xFF))
    del flush

    # secondary: the warm back-to-back rate (inputs partly in the last-level cache)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / K
    timed_out = ssd.ssd_fwd_status(ws)

    cnt = counts(prob)
    peak_mfma = PEAK_BF16_MFMA if prob.io_dtype == "bf16" else PEAK_FP32_MFMA
    if fused:
        # the fused kernel is the whole step: its launch is what the events bracket
        kname, k_ms, k_flops, k_bytes = "fused_fwd_kernel", cold_mean, cnt["f_path"], cnt["b_min"]
        units = cnt["units_out"]
        per_unit = {"flops": cnt["f_path"] / units, "bytes": cnt["b_min"] / units}
    else:
        # stage 3 alone (ssd_compute_out takes the default stage-3 kernel)
        kname = "out_resident_kernel" if cfg.get("out_resident") else "compute_out"
        k_ms = staged_compute_out_ms(args, ssd, prob, d, ws, y, dt_in, dt_kw)
        k_flops, k_bytes = cnt["f_out"], cnt["b_out"]
        units = cnt["units_out"]
        per_unit = {"flops": cnt["f_out"] / units, "bytes": cnt["b_out"] / units}
    t_k = k_ms * 1e-3
    if k_bytes / PEAK_HBM >= k_flops / peak_mfma:
        bound, achieved, peak, unit = "hbm", k_bytes / t_k / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", k_flops / t_k / 1e12, peak_mfma / 1e12, "TFLOP/s"

    line = {
        "metric": METRIC,
        "value": cnt["tokens"] / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.io_dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": prob.batch, "seqlen": prob.seqlen,
                   "nheads": prob.nheads, "headdim": prob.headdim, "dstate": prob.dstate,
                   "ngroups": prob.ngroups, "chunk_size": Q,
                   "init_state": prob.init_std is not None, "accumulate": "fp32",
                   "kernels": "fused single pass" if fused else
                              "staged (%d kernels; %s; stage 3 %s)" % (
                                  3 if cfg["cumsum_heads"] == 0 else 4,
                                  "running sums inside chunk_state" if cfg["cumsum_heads"] == 0
                                  else "running sums by chunk_cumsum",
                                  "with the interaction tile resident across heads"
                                  if cfg.get("out_resident") else "per head pair"),
                   "dt": "raw, bias + softplus in the first stage" if args.raw_dt else "prepared"},
        "timing": {"ms_per_step": "median of the timed steps, last-level cache evicted before "
                                  "each by %s 512 MiB" % ("writing" if args.evict == "write"
                                                           else "reading"),
                   "p10_ms": p10, "p90_ms": p90, "mean_ms": cold_mean,
                   "after_write_fill_ms": median(dirty) if dirty else None,
                   "after_write_fill_p10_p90_ms": [dirty[int(0.1 * (K - 1))],
                                                   dirty[int(round(0.9 * (K - 1)))]] if dirty else None,
                   "warm_ms_per_step": warm_ms, "warm_tokens_per_s": cnt["tokens"] / (warm_ms * 1e-3),
                   "wall_s": wall},
        "path_mfma_frac": cnt["f_path"] / (ms_step * 1e-3) / peak_mfma,
        "path_hbm_frac": cnt["b_min"] / (ms_step * 1e-3) / PEAK_HBM,
        "path_tflops": cnt["f_path"] / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": kname, "bound": bound, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak, "traffic": read_traffic(kname, args.workload),
                     "kernel_ms": k_ms, "units_per_launch": units, "per_unit": per_unit,
                     "mfma_frac": k_flops / t_k / peak_mfma, "hbm_frac": k_bytes / t_k / PEAK_HBM},
        "inputs_sha256": {k: ssd_synth.tensor_digest(v) for k, v in inputs.items()
                          if k in ("x", "dt", "dt_raw", "dt_bias", "A", "B", "C", "D", "init_state")},
        "status_timed_out": timed_out,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inputs, prob, gpu_out=(y, fin),
                                            raw_dt=args.raw_dt)
    print(json.dumps(line), flush=True)


def evict_by_reading(buf):
    """Evict the last-level cache by reading `buf` (512 MiB, twice the cache):
    the cache is then full of clean lines of an unrelated buffer, so the next
    kernels neither hit their inputs nor write back someone else's data."""
    import torch
    buf.view(dtype=torch.float32).sum()   # fp32 in, fp32 out: one reduction, no temporary


def staged_compute_out_ms(args, ssd, prob, d, ws, y, dt_in, dt_kw):
    """Mean event-timed compute_out launch on the staged path (stages 1-2 and
    stage 3 enqueued separately, cache evicted by reading before each step)."""
    import torch
    Q = prob.chunk_size
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=d["x"].device)
    fin = torch.empty((prob.batch, prob.nheads, prob.headdim, prob.dstate), dtype=torch.float32,
                      device=d["x"].device)
    tot = 0.0
    n = max(1, args.steps)
    for k in range(n):
        evict_by_reading(flush)
        ssd.ssd_fwd_states(d["x"], dt_in, d["A"], d["B"], Q, d["init_state"],
                           want_chunk_states=False, workspace=ws, final_out=fin, **dt_kw)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ssd.ssd_compute_out(d["x"], d["B"], d["C"], d["D"], Q, ws, out=y)
        b.record()
        torch.cuda.synchronize()
        tot += a.elapsed_time(b)
    return tot / n


def graph_line(args, prob, fwd):
    """Each step replays one captured HIP graph of the whole pass."""
    import torch
    fwd()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    cnt = counts(prob)
    print(json.dumps({"metric": METRIC + " (HIP graph replay, warm)",
                      "value": cnt["tokens"] / (ms_step * 1e-3), "unit": "tokens/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": ms_step, "higher_is_better": True,
                      "dtype": prob.io_dtype, "data": "synthetic",
                      "config": {"workload": args.workload, "graph": True}}), flush=True)


if __name__ == "__main__":
    main()
