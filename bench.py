#!/usr/bin/env python3
"""Throughput of one rank's share of batch-sharded sampling on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  1. lmhead_logits_local: bf16 hidden [rows, H] x lm_head [V, H] -> fp32 logits,
     written as n_slices vocabulary slices side by side (the slices the ranks
     of a tensor-parallel group each compute);
  2+3. sampler_assemble_and_sample: the received slices stitched into the
     batch buffer [rows, V] (receive side of the all-to-all) and
     temperature / top-k / top-p / log-probabilities / Gumbel-max sampling of
     every row, in one call whose first pass reads each logit once and writes
     the stitched copy as it goes.
After the timed steps the same work is timed the unfused way (projection,
then sampler_assemble_vocab_slices, then sampler_sample on the stitched
buffer), and each of those calls alone, as is sampler_sample_slices (the
sampler reading the slices in place, with no stitched copy), each over the
same number of steps; all of them are reported beside the step.
Default workload: speculative decode, 128 requests x (4 draft + 1) = 640 rows,
H = 4096, V = 151,936 (4 slices of 37,984).  --workload fp8 runs the pages'
model shape (H = 2560, V = 248,320 in 8 slices) with an FP8 lm_head: each
step quantizes the hidden states per row and projects with the E4M3 kernel.

Prints one JSON line.  Per-kernel times come from HIP events recorded on the
stream the kernels are launched on, over the timed region.  After the timed
steps each kernel is also timed alone, cold: 5 warm-up runs, then 50 runs,
each preceded by a 512 MiB scratch write so that no logit is served from the
256 MB Infinity Cache; the median with p10 / p90 is reported.  A measured
copy bandwidth, and the shader clock and bf16 matrix-core rate under a dense
MFMA load, are reported as context for the roofline fractions.
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
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="spec_decode",
                    choices=["decode", "spec_decode", "rank_share", "large", "draft",
                             "draft_share", "fp8"])
    ap.add_argument("--slices", type=int, default=4, help="vocabulary slices (TP ranks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=640,
                    help="rows of the workload the CPU oracle is timed on")
    ap.add_argument("--iso-runs", type=int, default=50,
                    help="runs of each kernel timed alone (cold); 0 skips them")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the copy-bandwidth and clock-probe context figures")
    return ap.parse_args()


def oracle_workers() -> int:
    """Host cores the oracle may use: the process's CPU affinity, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_sample_part(job):
    """One process's share of the oracle sampler: rows [a, b) of the sample,
    keyed on their global rows."""
    import oracle

    logits, params, row_offset, max_logprobs = job
    res = oracle.sample(logits, params, row_offset, max_logprobs)
    return (logits.shape[0], res.token_ids, res.topn_ids, res.row_status, res.flag_top_p,
            res.flag_tie)


def cpu_baseline(x, wt, wq, wsc, logits_sample, params, max_logprobs, rows: int, pool, workers,
                 gpu_out=None, row_offset: int = 0):
    """The CPU oracle as it stands, timed on a bounded sample of the workload:
    the float64 projection of `rows` rows against the whole lm_head (for the
    FP8 workload: the oracle's per-row quantization of those rows, then its
    projection from the same lm_head codes the GPU uses), with as many BLAS
    threads as host cores, then the full-sort sampler on those rows, split by
    rows over a process pool of the same size.  Scaled to rows/s.

    Returns (baseline, flagged): the second counts the rows the oracle flags
    as ambiguous on these logits (the step's own) and, with ``gpu_out`` (the
    step's token ids, top-N ids and row status as numpy arrays), how many
    unflagged rows differ from the GPU's."""
    import numpy as np
    import threadpoolctl

    import oracle

    torch = __import__("torch")
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    xb = bits(x[:rows]) if x is not None else None
    if wq is not None:
        wc, ws = wq.cpu().numpy().view(np.uint8), wsc.cpu().numpy()

        def project():
            q, s = oracle.quantize_rows_e4m3(xb)
            oracle.lmhead_logits_e4m3(q, s, wc, ws)
        what = "FP8 quantization and float64 projection"
    elif wt is not None:
        wb = bits(wt)

        def project():
            oracle.lmhead_logits(xb, wb)
        what = "float64 projection"
    else:
        project = None
    with threadpoolctl.threadpool_limits(limits=workers, user_api="blas"):
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        t0 = time.perf_counter()
        if project is not None:
            project()
        t1 = time.perf_counter()
    cuts = np.linspace(0, rows, workers + 1).astype(int)
    jobs = [(logits_sample[a:b], params[a:b], row_offset + int(a), max_logprobs)
            for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    parts = pool.map(_oracle_sample_part, jobs) if pool is not None else \
        list(map(_oracle_sample_part, jobs))
    t2 = time.perf_counter()
    assert sum(p[0] for p in parts) == rows
    cat = lambda i: np.concatenate([p[i] for p in parts])  # noqa: E731
    tok, topn, status, ftp, ftie = (cat(i) for i in range(1, 6))
    flagged = ftp | ftie
    counts = {"rows_checked": rows, "flagged": int(flagged.sum()),
              "flagged_top_p": int(ftp.sum()), "flagged_key_tie": int(ftie.sum()),
              "source": "the oracle on the step's own logits (first rows of the batch)"}
    if gpu_out is not None:
        g_tok, g_topn, g_status = (a[:rows] for a in gpu_out)
        ok = ~flagged
        counts["unflagged_token_id_mismatches"] = int((g_tok[ok] != tok[ok]).sum())
        counts["unflagged_topn_id_mismatches"] = int((g_topn[ok] != topn[ok]).any(axis=1).sum()) \
            if topn.ndim == 2 and topn.shape[1] else 0
        counts["row_status_mismatches"] = int((g_status != status).sum())
    procs = len(jobs) if pool is not None else 1
    proj = (f"{what} against the full lm_head ({t1 - t0:.1f}s, BLAS threads {threads}) + "
            if project is not None else "")
    return {
        "value": rows / (t2 - t0),
        "unit": "rows/s",
        "cores": int(max(threads if project is not None else 1, procs)),
        "kind": "oracle",
        "sample": f"{rows} rows: {proj}full-sort sampler ({t2 - t1:.1f}s, "
                  f"{procs} processes)",
    }, counts


def time_alone(fn, stream, scratch, runs: int, warmup: int = 5) -> dict:
    """fn timed alone with HIP events on `stream`: `warmup` untimed runs, then
    `runs` runs each preceded by a write of the whole scratch buffer (outside
    the events), so that what fn reads comes from HBM, not the Infinity Cache.
    Median, p10 and p90 in milliseconds."""
    import numpy as np
    import torch

    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(runs)]
    for i, (a, b) in enumerate(evs):
        scratch.fill_(i & 0xFF)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"median_ms": round(float(np.median(t)), 4),
            "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4)}


def measured_copy_gbs(dev, stream, nbytes: int = 1 << 30, runs: int = 20) -> float:
    """Achievable copy bandwidth (bytes read + bytes written per second, GB/s):
    the median of device-to-device copies of a 1 GiB buffer."""
    import numpy as np
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(runs)]
    for a, b in evs:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    del src, dst
    return round(2.0 * nbytes / (ms * 1e-3) / 1e9, 1)


def measured_mfma_clock(ts, dev, stream, iters: int = 1 << 18, launches: int = 3,
                        random: bool = False) -> dict:
    """The shader clock and the bf16 matrix-core rate under a dense MFMA load
    on every compute unit (the library's clock probe: per workgroup, the
    shader-clock counter against the 100 MHz real-time counter), from the
    last of `launches` back-to-back launches, after the clock has settled.
    `random` gives the MFMAs random operand bits (as real data has) instead
    of a few small values."""
    import numpy as np
    import torch

    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs = 2 * n_cu
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for a, b in ev:
        a.record(stream)
        ticks = ts.mfma_clock_probe(wgs, iters, dev, stream=stream, random=random)
        b.record(stream)
    torch.cuda.synchronize()
    t = ticks.cpu().numpy().astype(np.float64)
    mhz = (t[:, 1] - t[:, 0]) / (t[:, 3] - t[:, 2]) * 100.0
    ms = ev[-1][0].elapsed_time(ev[-1][1])
    flops = wgs * 8.0 * iters * 4 * 32768
    return {"mhz_median": round(float(np.median(mhz)), 0),
            "mhz_p10": round(float(np.percentile(mhz, 10)), 0),
            "mhz_p90": round(float(np.percentile(mhz, 90)), 0),
            "bf16_mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "load": f"{wgs} workgroups x 8 waves x {iters} rounds of 4 bf16 32x32x16 MFMA, "
                    f"{'random' if random else 'small'} operands"}


# Workloads with a committed counter summary: (summary file, projection
# kernel, kernel sources the summary's hash covers, in order).
TRAFFIC_RECORDS = {
    "spec_decode": ("spec_decode_step_hbm_traffic.txt", "lmhead_gemm",
                    ["lmhead_gemm.hip", "tile_store.hpp"]),
    "fp8": ("fp8_step_hbm_traffic.txt", "lmhead_e4m3", ["lmhead_fp8.hip", "tile_store.hpp"]),
}


def recorded_traffic(workload: str):
    """HBM bytes per projection launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when
    there is no summary for the workload or the kernel sources have changed
    since the counters were taken."""
    import hashlib

    if workload not in TRAFFIC_RECORDS:
        return None
    fname, kernel, sources = TRAFFIC_RECORDS[workload]
    path = os.path.join(ROOT, "profiles", fname)
    try:
        text = open(path).read()
        h = hashlib.sha256()
        for src in sources:
            h.update(open(os.path.join(ROOT, "top_sampling_amd", "csrc", src), "rb").read())
        digest = h.hexdigest()[:16]
    except OSError:
        return None
    for ln in text.splitlines():
        f = ln.split()
        if len(f) == 3 and f[0] == kernel and f[1].startswith("traffic_bytes_per_launch="):
            if f[2] == f"source_sha256_16={digest}":
                return int(f[1].split("=", 1)[1])
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)

    # The oracle's process pool is forked before anything touches the GPU; its
    # workers run numpy only.
    pool = None
    workers = oracle_workers()
    if not args.no_cpu_baseline and workers > 1:
        import multiprocessing as mp

        pool = mp.get_context("fork").Pool(workers)

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
    n_sl = w.n_slices if (w.hidden is None or w.n_slices > 1) else args.slices
    base, rem = divmod(vocab, n_sl)
    widths = [base + (1 if s < rem else 0) for s in range(n_sl)]
    cuts = np.concatenate([[0], np.cumsum(widths)])

    xq = xsc = wq = wsc = None
    if w.hidden is not None:
        x, wt = workloads.make_projection_device(w, dev)
        if w.fp8:
            # The checkpoint's FP8 lm_head: quantized once, outside the timed steps.
            wq, wsc = ts.quantize_rows_e4m3(wt)
            xq = torch.empty(rows, w.hidden, dtype=torch.uint8, device=dev)
            xsc = torch.empty(rows, dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
        local = torch.empty(rows, vocab, dtype=torch.float32, device=dev)
        slices = [local[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    else:
        x = wt = None
        full = torch.from_numpy(workloads.make_logits(w)).to(dev)
        slices = [full[:, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])]
        del full
    batch = torch.empty(rows, vocab, dtype=torch.float32, device=dev)
    out = ts.allocate_sample_output(rows, w.max_logprobs, dev)
    out_unf = ts.allocate_sample_output(rows, w.max_logprobs, dev)
    ws = ts.allocate_workspace(rows, vocab, w.max_logprobs, dev)

    ws_sl = torch.empty(max(256, ts.sampler_workspace_bytes_slices(rows, widths, w.max_logprobs)),
                        dtype=torch.uint8, device=dev)

    def project(ev=None):
        if x is not None and w.fp8:
            ts.quantize_rows_e4m3(x, out=xq, scales=xsc, stream=stream)
            if ev is not None:
                ev[4].record(stream)
            ts.lmhead_logits_local_e4m3(xq, xsc, wq, wsc, out=local, stream=stream)
        elif x is not None:
            ts.lmhead_logits_local(x, wt, out=local, stream=stream)

    def step(ev=None):
        project(ev)
        if ev is not None:
            ev[0].record(stream)
        ts.sampler_assemble_and_sample(slices, params, w.row_offset, w.max_logprobs,
                                       assembled=batch, out=out, workspace=ws_sl, stream=stream)

    def step_unfused(ev=None):
        project()
        if ev is not None:
            ev[0].record(stream)
        ts.sampler_assemble_vocab_slices(slices, out=batch, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        ts.sampler_sample(batch, params, w.row_offset, w.max_logprobs, out=out_unf, workspace=ws,
                          stream=stream)

    # The same work unfused (projection, assembly, sampler on the stitched
    # buffer), for comparison.  It runs before the step's warm-up and timed
    # steps: a fresh process's first few dozen projections run slower (0.79
    # against 0.70-0.72 ms at spec_decode) whichever form comes first, so
    # this block takes that start-up cost.  The isolated cold medians below
    # time both forms under the same conditions.
    for _ in range(max(1, args.warmup)):
        step_unfused()
    evu = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evu:
        e[3].record(stream)
        step_unfused(e)
        e[2].record(stream)
    torch.cuda.synchronize()
    unfused_step_ms = sum(e[3].elapsed_time(e[2]) for e in evu) / args.steps
    asm_ms = sum(e[0].elapsed_time(e[1]) for e in evu) / args.steps
    smp_ms = sum(e[1].elapsed_time(e[2]) for e in evu) / args.steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][3].record(stream)
        step(evs[i])
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    if w.fp8:  # event 4 separates the per-step quantization of the hidden states
        quant_ms = sum(e[3].elapsed_time(e[4]) for e in evs) / args.steps
        gemm_ms = sum(e[4].elapsed_time(e[0]) for e in evs) / args.steps
    else:
        quant_ms = None
        gemm_ms = sum(e[3].elapsed_time(e[0]) for e in evs) / args.steps
    fused_ms = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps

    n_diff_unfused = int((out_unf.token_ids != out.token_ids).sum())

    # The same slices sampled in place (no stitched copy), timed on its own.
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

    # The sampler on the same logits with every row's top_k forced to 1,000,
    # then to 2,048 (temperature, top-p, seeds and logprobs as drawn): a
    # top_k above 1,024 must not cost much more than one below.
    topk_ms = {}
    for k in (1000, 2048):
        pk = params_np.copy()
        pk["top_k"] = k
        pk_dev = ts.params_to_device(pk, dev)
        ws_k = ts.allocate_workspace(rows, vocab, w.max_logprobs, dev)
        out_k = ts.allocate_sample_output(rows, w.max_logprobs, dev)

        def sample_k():
            ts.sampler_sample(batch, pk_dev, w.row_offset, w.max_logprobs, out=out_k,
                              workspace=ws_k, stream=stream)

        for _ in range(max(1, args.warmup)):
            sample_k()
        ev_k = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for a, b in ev_k:
            a.record(stream)
            sample_k()
            b.record(stream)
        torch.cuda.synchronize()
        topk_ms[k] = sum(a.elapsed_time(b) for a, b in ev_k) / args.steps
        del ws_k, out_k, pk_dev

    # Each kernel alone, cold (a 512 MiB scratch write before every run).
    iso = {}
    if args.iso_runs > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        if x is not None and w.fp8:
            iso["quantize_hidden"] = time_alone(
                lambda: ts.quantize_rows_e4m3(x, out=xq, scales=xsc, stream=stream),
                stream, scratch, args.iso_runs)
            iso["lmhead_e4m3"] = time_alone(
                lambda: ts.lmhead_logits_local_e4m3(xq, xsc, wq, wsc, out=local, stream=stream),
                stream, scratch, args.iso_runs)
        elif x is not None:
            iso["lmhead_gemm"] = time_alone(
                lambda: ts.lmhead_logits_local(x, wt, out=local, stream=stream),
                stream, scratch, args.iso_runs)
        iso["assemble_and_sample"] = time_alone(
            lambda: ts.sampler_assemble_and_sample(slices, params, w.row_offset, w.max_logprobs,
                                                   assembled=batch, out=out, workspace=ws_sl,
                                                   stream=stream),
            stream, scratch, args.iso_runs)
        iso["assemble"] = time_alone(
            lambda: ts.sampler_assemble_vocab_slices(slices, out=batch, stream=stream),
            stream, scratch, args.iso_runs)
        iso["sampler"] = time_alone(
            lambda: ts.sampler_sample(batch, params, w.row_offset, w.max_logprobs, out=out,
                                      workspace=ws, stream=stream),
            stream, scratch, args.iso_runs)
        iso["sampler_slices"] = time_alone(sample_slices, stream, scratch, args.iso_runs)
        iso["step"] = time_alone(step, stream, scratch, args.iso_runs)
        iso["step_unfused"] = time_alone(step_unfused, stream, scratch, args.iso_runs)
        del scratch
    copy_gbs = None if args.no_context else measured_copy_gbs(dev, stream)
    clock = None if args.no_context else measured_mfma_clock(ts, dev, stream)
    clock_rnd = None if args.no_context else measured_mfma_clock(ts, dev, stream, random=True)

    flops = 2.0 * rows * vocab * w.hidden if w.hidden else 0.0
    sampler_bytes = 4.0 * rows * vocab + rows * (24 + 12 + 8 * w.max_logprobs)
    asm_bytes = 2 * 4.0 * rows * vocab
    # Fused: every logit read once from the slices and written once to the
    # stitched buffer, plus the sampler's parameters and outputs.
    fused_bytes = asm_bytes + sampler_bytes - 4.0 * rows * vocab
    fused_gbs = fused_bytes / (fused_ms * 1e-3) / 1e9
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12 if flops else None
    smp_gbs = sampler_bytes / (smp_ms * 1e-3) / 1e9
    asm_gbs = asm_bytes / (asm_ms * 1e-3) / 1e9
    # The projection's algorithmic bytes: hidden and lm_head read once, logits
    # written once.  Below the ridge (peak flop/s over peak bytes/s) HBM bounds it.
    # FP8 operands are one byte per element plus one fp32 scale per row.
    eb = 1.0 if w.fp8 else 2.0
    gemm_bytes = (eb * rows * w.hidden + eb * vocab * w.hidden + 4.0 * rows * vocab
                  + (4.0 * (rows + vocab) if w.fp8 else 0.0) if w.hidden else 0.0)
    peak_tf = FP8_PEAK_TFLOPS if w.fp8 else BF16_PEAK_TFLOPS
    gemm_kernel = "lmhead_e4m3" if w.fp8 else "lmhead_gemm"
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops and flops / gemm_bytes >= ridge:
        roof = {"kernel": gemm_kernel, "bound": "mfma", "achieved": round(gemm_tflops, 1),
                "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / peak_tf, 4),
                "traffic": recorded_traffic(w.name)}
    elif flops:
        gemm_gbs = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"kernel": gemm_kernel, "bound": "hbm", "achieved": round(gemm_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(w.name)}
    else:  # sampler-only workload: the step is the fused assembly + sampler call
        roof = {"kernel": "assemble_and_sample", "bound": "hbm", "achieved": round(fused_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
                "traffic": None}

    rps = lambda ms: round(rows / (ms * 1e-3), 1)  # noqa: E731
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
        "dtype": "e4m3" if w.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": rows, "hidden": w.hidden, "vocab": vocab,
                   "vocab_slices": n_sl, "max_logprobs": w.max_logprobs,
                   "description": w.description},
        "kernels": {
            gemm_kernel: {"ms": round(gemm_ms, 4), "tflops": gemm_tflops and round(gemm_tflops, 1),
                          "frac_mfma_peak": gemm_tflops and round(gemm_tflops / peak_tf, 4),
                          "rows_per_s": rps(gemm_ms)},
            "assemble_and_sample": {"ms": round(fused_ms, 4), "gbs": round(fused_gbs, 1),
                                    "frac_hbm_peak": round(fused_gbs / HBM_PEAK_GBS, 4),
                                    "rows_per_s": rps(fused_ms),
                                    "bytes": "slices read once + stitched buffer written once "
                                             "+ parameters and outputs"},
            "assemble": {"ms": round(asm_ms, 4), "gbs": round(asm_gbs, 1),
                         "frac_hbm_peak": round(asm_gbs / HBM_PEAK_GBS, 4),
                         "rows_per_s": rps(asm_ms)},
            "sampler": {"ms": round(smp_ms, 4), "gbs": round(smp_gbs, 1),
                        "frac_hbm_peak": round(smp_gbs / HBM_PEAK_GBS, 4),
                        "rows_per_s": rps(smp_ms)},
            "sampler_slices": {"ms": round(sl_ms, 4), "gbs": round(sampler_bytes / (sl_ms * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(sampler_bytes / (sl_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "rows_per_s": rps(sl_ms),
                               "saves_ms_vs_assemble_then_sample": round(asm_ms + smp_ms - sl_ms, 4),
                               "token_ids_differing_from_step": n_diff},
            "sampler_top_k_1000_every_row": {"ms": round(topk_ms[1000], 4),
                                             "rows_per_s": rps(topk_ms[1000])},
            "sampler_top_k_2048_every_row": {"ms": round(topk_ms[2048], 4),
                                             "rows_per_s": rps(topk_ms[2048]),
                                             "vs_top_k_1000": round(topk_ms[2048] / topk_ms[1000], 3)},
        },
        "roofline": roof,
        "step_unfused": {"ms_per_step": round(unfused_step_ms, 4),
                         "rows_per_s": rps(unfused_step_ms),
                         "calls": "projection, sampler_assemble_vocab_slices, sampler_sample",
                         "token_ids_differing_from_step": n_diff_unfused},
    }
    if not flops:  # sampler-only workload: there is no projection to report
        del line["kernels"][gemm_kernel]
    if quant_ms is not None:
        line["kernels"]["quantize_hidden"] = {"ms": round(quant_ms, 4), "rows_per_s": rps(quant_ms)}
    if iso:
        algo = {"lmhead_gemm": gemm_bytes, "lmhead_e4m3": gemm_bytes, "assemble": asm_bytes,
                "sampler": sampler_bytes, "sampler_slices": sampler_bytes,
                "assemble_and_sample": fused_bytes}
        for k, st in iso.items():
            if k in algo and algo[k]:
                st["gbs_median"] = round(algo[k] / (st["median_ms"] * 1e-3) / 1e9, 1)
            if k in ("lmhead_gemm", "lmhead_e4m3") and flops:
                st["tflops_median"] = round(flops / (st["median_ms"] * 1e-3) / 1e12, 1)
            if k in ("step", "step_unfused"):
                st["rows_per_s_median"] = round(rows / (st["median_ms"] * 1e-3), 1)
        line["isolated_cold"] = {"runs": args.iso_runs, "warmup": 5,
                                 "scratch_write_bytes": 512 << 20, "kernels": iso}
    line["context"] = {"copy_gbs": copy_gbs, "mfma_load": clock, "mfma_load_random": clock_rnd}
    if not args.no_cpu_baseline:
        sample_rows = min(args.cpu_rows, rows)
        logits_sample = batch[:sample_rows].cpu().numpy()
        gpu_out = (out.token_ids.cpu().numpy(), out.topn_ids.cpu().numpy(),
                   out.row_status.cpu().numpy())
        line["cpu_baseline"], line["flagged_rows"] = cpu_baseline(
            x, wt, wq, wsc, logits_sample, params_np, w.max_logprobs, sample_rows, pool, workers,
            gpu_out, w.row_offset)
    else:
        line["flagged_rows"] = None
    if pool is not None:
        pool.close()
        pool.join()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
