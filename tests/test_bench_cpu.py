"""The bench's host-side bookkeeping, on the CPU: the oracle leg counts the
rows it flags and the GPU rows that differ from it on unflagged rows."""
import numpy as np

import bench
import oracle
import workloads


def _rank_share_sample(rows=24):
    w = workloads.get("rank_share")
    logits = workloads.make_logits(w)[:rows, :8192].astype(np.float32)
    params = workloads.make_params(w)[:rows]
    return logits, params, w.max_logprobs


def test_cpu_baseline_counts_mismatches_against_the_oracle():
    logits, params, max_lp = _rank_share_sample()
    rows = logits.shape[0]
    ref = oracle.sample(logits, params, 100, max_lp)
    gpu = (ref.token_ids.copy(), ref.topn_ids.copy(), ref.row_status.copy())
    base, counts = bench.cpu_baseline(None, None, None, None, logits, params, max_lp, rows, None,
                                      1, gpu, row_offset=100)
    assert base["kind"] == "oracle" and base["unit"] == "rows/s" and base["value"] > 0
    assert counts["rows_checked"] == rows
    assert counts["flagged"] == int((ref.flag_top_p | ref.flag_tie).sum())
    assert counts["unflagged_token_id_mismatches"] == 0
    assert counts["unflagged_topn_id_mismatches"] == 0
    assert counts["row_status_mismatches"] == 0
    # Two planted differences on unflagged rows are both counted.
    ok = np.flatnonzero(~(ref.flag_top_p | ref.flag_tie))
    tok = gpu[0].copy()
    tok[ok[:2]] += 1
    _, counts = bench.cpu_baseline(None, None, None, None, logits, params, max_lp, rows, None, 1,
                                   (tok, gpu[1], gpu[2]), row_offset=100)
    assert counts["unflagged_token_id_mismatches"] == 2


def test_cpu_baseline_keys_rows_on_the_global_row():
    """The oracle leg samples with the workload's row offset: keyed on the
    local row instead, the seeded draws (and so the tokens) change."""
    logits, params, max_lp = _rank_share_sample()
    rows = logits.shape[0]
    at_100 = oracle.sample(logits, params, 100, max_lp)
    gpu = (at_100.token_ids, at_100.topn_ids, at_100.row_status)
    _, same = bench.cpu_baseline(None, None, None, None, logits, params, max_lp, rows, None, 1,
                                 gpu, row_offset=100)
    _, other = bench.cpu_baseline(None, None, None, None, logits, params, max_lp, rows, None, 1,
                                  gpu, row_offset=0)
    assert same["unflagged_token_id_mismatches"] == 0
    assert other["unflagged_token_id_mismatches"] > 0
