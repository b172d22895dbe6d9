"""The CPU oracle's sampler over a large logits array, in worker processes.

Each worker is a fresh interpreter running this file on a row range (never a
fork: the test process holds a GPU context that a forked child must not
inherit).  Workers memory-map the logits and parameters from .npy files, run
only numpy (the oracle), and write their rows' results to an .npz file.

    python tests/oracle_pool.py <logits.npy> <params.npy> <r0> <r1> <row_offset>
                                <max_logprobs> <out.npz>
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
FIELDS = ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status",
          "flag_top_p", "flag_tie", "kept")


def _rows(logits_path, params_path, r0, r1, row_offset, max_lp):
    import oracle

    logits = np.asarray(np.load(logits_path, mmap_mode="r")[r0:r1])
    params = np.load(params_path)[r0:r1]
    res = oracle.sample(logits, params, row_offset + r0, max_lp)
    l64 = logits.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.where(np.isfinite(l64), l64, -np.inf).max(axis=1)
        lse = m + np.log(np.exp(l64 - m[:, None]).sum(axis=1))
    # The two best Gumbel keys of the kept set (float64), for rows that draw.
    top_ids = np.full((r1 - r0, 2), -1, dtype=np.int64)
    top_keys = np.full((r1 - r0, 2), np.nan)
    for i in range(r1 - r0):
        pr = params[i]
        t, k, p = float(pr["temperature"]), int(pr["top_k"]), float(pr["top_p"])
        if res.row_status[i] != 0 or t < oracle.GREEDY_EPS or k == 1:
            continue
        l = l64[i]
        kept, _ = oracle.kept_set(l, t, k, p)
        keys = (l[kept] - l.max()) / t + oracle.gumbel_noise(int(pr["seed"]),
                                                             row_offset + r0 + i, kept)
        order = np.lexsort((kept, -keys))[:2]
        top_ids[i, :len(order)] = kept[order]
        top_keys[i, :len(order)] = keys[order]
    out = {f: getattr(res, f) for f in FIELDS}
    out.update(lse=lse, top_ids=top_ids, top_keys=top_keys)
    return out


def sample_file(logits_path: str, params: np.ndarray, row_offset: int, max_logprobs: int,
                rows: int, workers: int | None = None, timeout: float = 600.0):
    """(oracle SampleResult, float64 log-sum-exp per row, ids [rows, 2] and
    float64 keys [rows, 2] of each row's two best Gumbel keys, -1 / NaN for
    rows that do not draw) for the logits saved at ``logits_path``."""
    import oracle

    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    base = os.path.splitext(logits_path)[0]
    params_path = base + "_params.npy"
    np.save(params_path, np.ascontiguousarray(params))
    step = max(1, -(-rows // workers))
    procs = []
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out = f"{base}_rows{r0}.npz"
        cmd = [sys.executable, os.path.abspath(__file__), logits_path, params_path, str(r0),
               str(r1), str(row_offset), str(max_logprobs), out]
        procs.append((r0, out, subprocess.Popen(cmd, env=dict(os.environ, OMP_NUM_THREADS="1"))))
    parts = []
    for r0, out, pr in procs:
        rc = pr.wait(timeout=timeout)
        assert rc == 0, f"oracle worker for rows from {r0} exited with {rc}"
        with np.load(out) as z:
            parts.append({k: z[k] for k in z.files})
    cat = lambda f: np.concatenate([p[f] for p in parts])  # noqa: E731
    res = oracle.SampleResult(**{f: cat(f) for f in FIELDS})
    return res, cat("lse"), cat("top_ids"), cat("top_keys")


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    lp, pp, r0, r1, ro, mlp, outp = sys.argv[1:8]
    res = _rows(lp, pp, int(r0), int(r1), int(ro), int(mlp))
    np.savez(outp, **res)
