#!/usr/bin/env python3
"""Throughput of one rank's share of batch-sharded sampling on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  1. lmhead_logits_local: bf16 hidden [rows, H] x lm_head [V, H] -> fp32 logits,
     written as n_slices vocabulary slices side by side (the slices the ranks
     of a tensor-parallel group each compute);
  2. sampler_assemble_vocab_slices: the received slices stitched into the
     batch buffer [rows, V] (receive side of the all-to-all);
  3. sampler_sample: temperature / top-k / top-p / log-probabilities /
     Gumbel-max sampling of every row.
After the timed steps, sampler_sample_slices (the sampler reading the slices
in place, with no stitching copy) is timed on its own over the same number of
steps and reported beside the per-kernel times.
Default workload: speculative decode, 128 requests x (4 draft + 1) = 640 rows,
H = 4096, V = 151,936 (4 slices of 37,984).

Prints one JSON line.  Per-kernel times come from HIP events recorded on the
stream the kernels are launched on, over the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/s + sampler HBM GB/s + lm_head TFLOP/s at 640 rows x V=151,936"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="spec_decode",
                    choices=["decode", "spec_decode", "rank_share", "large", "draft",
                             "draft_share"])
    ap.add_argument("--slices", type=int, default=4, help="vocabulary slices (TP ranks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=640,
                    help="rows of the workload the CPU oracle is timed on")
    return ap.parse_args()


def cpu_baseline(x, wt, logits_sample, params, max_logprobs, rows: int):
    """The CPU oracle as it stands, timed on a bounded sample of the workload:
    the float64 projection of `rows` rows against the whole lm_head, then the
    full-sort sampler on those rows.  Scaled to rows/s."""
    import numpy as np
    import threadpoolctl

    import oracle

    torch = __import__("torch")
    xb = x[:rows].view(torch.int16).cpu().numpy().view(np.uint16) if x is not None else None
    wb = wt.view(torch.int16).cpu().numpy().view(np.uint16) if wt is not None else None
    threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) \
        if threadpoolctl.threadpool_info() else 1
    t0 = time.perf_counter()
    if wb is not None:
        oracle.lmhead_logits(xb, wb)
    t1 = time.perf_counter()
    oracle.sample(logits_sample[:rows], params[:rows], 0, max_logprobs)
    t2 = time.perf_counter()
    proj = (f"float64 projection against the full lm_head ({t1 - t0:.1f}s, BLAS threads "
            f"{threads}) + " if wb is not None else "")
    return {
        "value": rows / (t2 - t0),
        "unit": "rows/s",
        "cores": int(threads) if wb is not None else 1,
        "kind": "oracle",
        "sample": f"{rows} rows: {proj}full-sort sampler ({t2 - t1:.1f}s, 1 thread)",
    }


def recorded_traffic(workload: str):
    """HBM bytes per projection launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when
    the summary is for another workload or the kernel source has changed
    since the counters were taken."""
    import hashlib

    if workload != "spec_decode":
        return None
    path = os.path.join(ROOT, "profiles", "spec_decode_step_hbm_traffic.txt")
    src = os.path.join(ROOT, "top_sampling_amd", "csrc", "lmhead_gemm.hip")
    try:
        text = open(path).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    for ln in text.splitlines():
        f = ln.split()
        if len(f) == 3 and f[0] == "lmhead_gemm" and f[1].startswith("traffic_bytes_per_launch="):
            if f[2] == f"source_sha256_16={digest}":
                return int(f[1].split("=", 1)[1])
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import top_sampling_amd as ts
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.get(args.workload)
    rows, vocab = w.rows, w.vocab
    stream = torch.cuda.current_stream()

    params_np = workloads.make_params(w)
    params = ts.params_to_device(params_np, dev)
    n_sl = w.n_slices if w.hidden is None else args.slices
    base, rem = divmod(vocab, n_sl)
    widths = [base + (1 if s < rem else 0) for s in range(n_sl)]
    cuts = np.concatenate([[0], np.cumsum(widths)])

    if w.hidden is not None:
        x, wt = workloads.make_projection_device(w, dev)
        local = torch.empty(rows, vocab, dtype=torch.float32, device=dev)
        slices = [local[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    else:
        x = wt = None
        full = torch.from_numpy(workloads.make_logits(w)).to(dev)
        slices = [full[:, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])]
        del full
    batch = torch.empty(rows, vocab, dtype=torch.float32, device=dev)
    out = ts.allocate_sample_output(rows, w.max_logprobs, dev)
    ws = ts.allocate_workspace(rows, vocab, w.max_logprobs, dev)

    def step(ev=None):
        if x is not None:
            ts.lmhead_logits_local(x, wt, out=local, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        ts.sampler_assemble_vocab_slices(slices, out=batch, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        ts.sampler_sample(batch, params, w.row_offset, w.max_logprobs, out=out, workspace=ws,
                          stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][3].record(stream)
        step(evs[i])
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    gemm_ms = sum(e[3].elapsed_time(e[0]) for e in evs) / args.steps
    asm_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    smp_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    # The same slices sampled in place (no stitching copy), timed on its own.
    ws_sl = torch.empty(max(256, ts.sampler_workspace_bytes_slices(rows, widths, w.max_logprobs)),
                        dtype=torch.uint8, device=dev)
    out_sl = ts.allocate_sample_output(rows, w.max_logprobs, dev)

    def sample_slices():
        ts.sampler_sample_slices(slices, params, w.row_offset, w.max_logprobs, out=out_sl,
                                 workspace=ws_sl,
                                 stream=stream)

    for _ in range(max(1, args.warmup)):
        sample_slices()
    ev_sl = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a, b in ev_sl:
        a.record(stream)
        sample_slices()
        b.record(stream)
    torch.cuda.synchronize()
    sl_ms = sum(a.elapsed_time(b) for a, b in ev_sl) / args.steps
    n_diff = int((out_sl.token_ids != out.token_ids).sum())

    flops = 2.0 * rows * vocab * w.hidden if w.hidden else 0.0
    sampler_bytes = 4.0 * rows * vocab + rows * (24 + 12 + 8 * w.max_logprobs)
    asm_bytes = 2 * 4.0 * rows * vocab
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12 if flops else None
    smp_gbs = sampler_bytes / (smp_ms * 1e-3) / 1e9
    asm_gbs = asm_bytes / (asm_ms * 1e-3) / 1e9
    # The projection's algorithmic bytes: hidden and lm_head read once, logits
    # written once.  Below the ridge (peak flop/s over peak bytes/s) HBM bounds it.
    gemm_bytes = (2.0 * rows * w.hidden + 2.0 * vocab * w.hidden + 4.0 * rows * vocab
                  if w.hidden else 0.0)
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops and flops / gemm_bytes >= ridge:
        roof = {"kernel": "lmhead_gemm", "bound": "mfma", "achieved": round(gemm_tflops, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
                "traffic": recorded_traffic(w.name)}
    elif flops:
        gemm_gbs = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"kernel": "lmhead_gemm", "bound": "hbm", "achieved": round(gemm_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(w.name)}
    else:
        roof = {"kernel": "sampler", "bound": "hbm", "achieved": round(smp_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(smp_gbs / HBM_PEAK_GBS, 4),
                "traffic": None}

    metric = METRIC if w.name == "spec_decode" else (
        f"sampled rows/s + sampler HBM GB/s + lm_head TFLOP/s at {rows} rows x V={vocab:,}")
    line = {
        "metric": metric,
        "value": round(rows / (ms_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": rows, "hidden": w.hidden, "vocab": vocab,
                   "vocab_slices": n_sl, "max_logprobs": w.max_logprobs,
                   "description": w.description},
        "kernels": {
            "lmhead_gemm": {"ms": round(gemm_ms, 4), "tflops": gemm_tflops and round(gemm_tflops, 1),
                            "frac_mfma_peak": gemm_tflops and round(gemm_tflops / BF16_PEAK_TFLOPS, 4)},
            "assemble": {"ms": round(asm_ms, 4), "gbs": round(asm_gbs, 1),
                         "frac_hbm_peak": round(asm_gbs / HBM_PEAK_GBS, 4)},
            "sampler": {"ms": round(smp_ms, 4), "gbs": round(smp_gbs, 1),
                        "frac_hbm_peak": round(smp_gbs / HBM_PEAK_GBS, 4),
                        "rows_per_s": round(rows / (smp_ms * 1e-3), 1)},
            "sampler_slices": {"ms": round(sl_ms, 4), "gbs": round(sampler_bytes / (sl_ms * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(sampler_bytes / (sl_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "saves_ms_vs_assemble_then_sample": round(asm_ms + smp_ms - sl_ms, 4),
                               "token_ids_differing_from_stitched": n_diff},
        },
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        sample_rows = min(args.cpu_rows, rows)
        logits_sample = batch[:sample_rows].cpu().numpy()
        line["cpu_baseline"] = cpu_baseline(x, wt, logits_sample, params_np, w.max_logprobs,
                                            sample_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
