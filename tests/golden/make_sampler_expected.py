"""Write tests/golden/sampler_expected_<workload>.npz: the oracle's sampler
outputs on each workload's seeded fp32 logits and parameters.

Calls only ``oracle`` and the seeded generators in ``workloads``.  The GPU
parity tests regenerate the same inputs (checked by digest) and compare the
HIP sampler against these values.

    python tests/golden/make_sampler_expected.py [workload ...]
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_logits() -> np.ndarray:
    """The tiny workload samples its own projection: fp32 of the oracle's
    float64 logits of the seeded bf16 hidden states and lm_head."""
    w = workloads.get("tiny")
    xb, wb = workloads.make_projection_host(w)
    return oracle.lmhead_logits(xb, wb).astype(np.float32)


def _job(args):
    name, r0, r1 = args
    w = workloads.get(name)
    params = workloads.make_params(w)
    logits = tiny_logits()[r0:r1] if name == "tiny" else workloads.make_logits(w, slice(r0, r1))
    res = oracle.sample(logits, params[r0:r1], r0, w.max_logprobs)
    l64 = logits.astype(np.float64)
    m = l64.max(axis=1)
    lse = m + np.log(np.exp(l64 - m[:, None]).sum(axis=1))
    return r0, res, lse, digest(logits)


def make(name: str, workers: int) -> str:
    w = workloads.get(name)
    t0 = time.time()
    step = max(1, min(32, w.rows // max(1, workers)))
    jobs = [(name, r0, min(w.rows, r0 + step)) for r0 in range(0, w.rows, step)]
    with mp.get_context("fork").Pool(workers) as pool:
        parts = sorted(pool.map(_job, jobs), key=lambda x: x[0])
    cat = lambda f: np.concatenate([getattr(p[1], f) for p in parts])  # noqa: E731
    out = dict(
        token_ids=cat("token_ids"), token_logprobs=cat("token_logprobs"),
        topn_ids=cat("topn_ids"), topn_logprobs=cat("topn_logprobs"),
        row_status=cat("row_status"), flag_top_p=cat("flag_top_p"), flag_tie=cat("flag_tie"),
        kept=cat("kept"), lse=np.concatenate([p[2] for p in parts]),
        logits_digests=np.array([p[3] for p in parts]),
        digest_rows=np.array([j[1:] for j in jobs]),
        params_digest=np.array(digest(workloads.make_params(w))),
    )
    if name == "tiny":
        out["logits"] = tiny_logits()
    path = os.path.join(HERE, f"sampler_expected_{name}.npz")
    np.savez_compressed(path, **out)
    flagged = int((out["flag_top_p"] | out["flag_tie"]).sum())
    print(f"{name}: {w.rows} rows, {flagged} flagged, {time.time() - t0:.1f}s -> {path}")
    return path


if __name__ == "__main__":
    names = sys.argv[1:] or list(workloads.WORKLOADS)
    nw = max(1, min(8, len(os.sched_getaffinity(0))))
    for n in names:
        make(n, nw)
