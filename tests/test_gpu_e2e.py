"""End to end on the GPU's own logits, at full size.

One rank's step exactly as the bench times it: the projection writes the
whole vocabulary into a local buffer; four column slices of it (the slices
tensor-parallel ranks would exchange) are stitched into the batch buffer
inside the sampler's first pass (sampler_assemble_and_sample).  The same
slices also go through the separate assembly and the sampler on the stitched
buffer, and through the sampler in place on the slices.  The logits the
sampler saw are copied back and the CPU oracle samples exactly those
values (page "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018",
section "What batch-sharded sampling is, in one paragraph": the rank projects
its slice, the slices are swapped, and each rank samples its rows).

Also here: the whole projection output against the float64 oracle (chunked
over the vocabulary), and the sampler's fp32 Gumbel keys against float64
ones on the rows' two best kept keys, the error that decides how close two
keys may lie before a row is flagged.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import oracle_pool
import workloads
from test_gpu_parity import LOGIT_TOL, _compare

pytestmark = pytest.mark.gpu

FIELDS = ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")
# Largest |fp32 key - float64 key| on a row's two best kept keys.  Two rows'
# keys closer than twice this could be ordered differently by the two sides;
# the oracle flags rows whose two best keys lie within 1e-5.
KEY_ERR_MAX = 5e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ts():
    import top_sampling_amd

    return top_sampling_amd


def _bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _projection_inputs(w, dev):
    import torch

    if w.rows * w.vocab <= 1 << 24:   # small enough to draw on the host
        xb, wb = workloads.make_projection_host(w)
        to = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(dev)  # noqa: E731
        return to(xb), to(wb)
    return workloads.make_projection_device(w, dev)


def _even_widths(V, n):
    base, rem = divmod(V, n)
    return [base + (1 if s < rem else 0) for s in range(n)]


def _gpu_keys(ts, dev, logits, params, row_offset, ids):
    """The sampler's fp32 keys of the listed (row, id) pairs (ids [rows, 2],
    -1 where there is nothing to read)."""
    import torch

    r, c = np.nonzero(ids >= 0)
    if r.size == 0:
        return r, c, np.zeros(0)
    tok = ids[r, c]
    vals = logits[r, tok].astype(np.float32)
    rmax = logits[r].max(axis=1).astype(np.float32)
    t = params["temperature"][r].astype(np.float32)
    seeds = params["seed"][r].astype(np.uint64).view(np.int64)
    grow = (row_offset + r).astype(np.int64)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    keys, _ = ts.gumbel_keys(d(vals), d(rmax), d(t), d(seeds), d(grow), d(tok.astype(np.int32)))
    return r, c, keys.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["tiny", "spec_decode", "large"])
def test_step_end_to_end_on_gpu_logits(dev, ts, name, tmp_path):
    import torch

    w = workloads.get(name)
    rows, V = w.rows, w.vocab
    say("e2e", name, rows, V, w.hidden)
    x, wt = _projection_inputs(w, dev)
    local = torch.empty(rows, V, dtype=torch.float32, device=dev)
    ts.lmhead_logits_local(x, wt, out=local)
    cuts = np.concatenate([[0], np.cumsum(_even_widths(V, 4))])
    slices = [local[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    batch = ts.sampler_assemble_vocab_slices(slices)
    params = workloads.make_params(w)
    p = ts.params_to_device(params, dev)
    out = ts.sampler_sample(batch, p, 0, w.max_logprobs)
    out_sl = ts.sampler_sample_slices(slices, p, 0, w.max_logprobs)
    fused_batch, out_f = ts.sampler_assemble_and_sample(slices, p, 0, w.max_logprobs)
    torch.cuda.synchronize()
    got = {k: getattr(out, k).cpu().numpy() for k in FIELDS}
    got_sl = {k: getattr(out_sl, k).cpu().numpy() for k in FIELDS}
    got_f = {k: getattr(out_f, k).cpu().numpy() for k in FIELDS}
    logits = batch.cpu().numpy()
    assert np.array_equal(logits.view(np.uint32), local.cpu().numpy().view(np.uint32))
    # The one-call step: its stitched buffer is the assembly's, bit for bit,
    # and it draws what the slice sampler draws (its chunks may be narrower,
    # so the log-probabilities may differ in the last bits).
    assert np.array_equal(fused_batch.cpu().numpy().view(np.uint32), logits.view(np.uint32))
    for k in ("token_ids", "topn_ids", "row_status"):
        assert np.array_equal(got_f[k], got_sl[k]), k
    for k in ("token_logprobs", "topn_logprobs"):
        a, b = got_f[k], got_sl[k]
        assert np.array_equal(np.isfinite(a), np.isfinite(b)), k
        fin = np.isfinite(a)
        assert np.abs(a[fin] - b[fin]).max(initial=0) <= 1e-5, k
    # The in-place slice sampler draws what the stitched call draws.  Its
    # chunks follow the slice boundaries, so sums (and the log-probabilities)
    # may differ in the last bits.
    for k in ("token_ids", "topn_ids", "row_status"):
        assert np.array_equal(got[k], got_sl[k]), k
    for k in ("token_logprobs", "topn_logprobs"):
        a, b = got[k], got_sl[k]
        assert np.array_equal(np.isfinite(a), np.isfinite(b)), k
        fin = np.isfinite(a)
        assert np.abs(a[fin] - b[fin]).max(initial=0) <= 1e-5, k
    # the projection on a few whole rows against float64
    rsel = np.unique([0, rows // 2, rows - 1])
    ref = oracle.lmhead_logits(_bits(x)[rsel], _bits(wt))
    err = np.abs(logits[rsel].astype(np.float64) - ref).max()
    say(f"  projection rows {rsel.tolist()}: max |err| {err:.2e}")
    assert err <= LOGIT_TOL
    del ref, x, wt
    path = str(tmp_path / "logits.npy")
    np.save(path, logits)
    res, lse, top_ids, top_keys = oracle_pool.sample_file(path, params, 0, w.max_logprobs, rows)
    flagged = res.flagged
    say(f"  oracle: {int(flagged.sum())} flagged of {rows} "
        f"(top-p {int(res.flag_top_p.sum())}, ties {int(res.flag_tie.sum())})")
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, flagged, lse, logits, label=f"e2e/{name}")
    _compare(got_f, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, flagged, lse, logits, label=f"e2e/{name}/one-call")
    # fp32 keys of each row's two best kept keys against float64
    r, c, gk = _gpu_keys(ts, dev, logits, params, 0, top_ids)
    if r.size:
        kerr = np.abs(gk - top_keys[r, c])
        gap = np.abs(top_keys[:, 0] - top_keys[:, 1])
        say(f"  keys: {r.size} compared, max |fp32 - fp64| {kerr.max():.2e}, "
            f"smallest top-2 gap {np.nanmin(gap) if np.isfinite(gap).any() else float('nan'):.2e}")
        assert kerr.max() < KEY_ERR_MAX


@pytest.mark.parametrize("name", ["decode", "spec_decode", "large"])
def test_gemm_whole_output(dev, ts, name):
    """Every logit of the full-size projection against the float64 oracle
    (compared one vocabulary chunk at a time)."""
    import torch

    w = workloads.get(name)
    say("gemm whole", name)
    x, wt = workloads.make_projection_device(w, dev)
    out = ts.lmhead_logits_local(x, wt)
    torch.cuda.synchronize()
    xb = _bits(x)
    worst = 0.0
    step = 16384
    for v0 in range(0, w.vocab, step):
        v1 = min(w.vocab, v0 + step)
        ref = oracle.lmhead_logits(xb, _bits(wt[v0:v1]))
        got = out[:, v0:v1].cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.abs(got - ref).max()))
    say(f"  {w.rows} x {w.vocab}: max |err| {worst:.2e}")
    assert worst <= LOGIT_TOL


def test_gpu_noise_words_match_the_word_table(dev, ts):
    """The sampler's Philox words, read back through the check entry point,
    equal the hand-laid-out word table the oracle is pinned to."""
    import torch

    from test_oracle_pins import RNG_TABLE, _table_word

    n = len(RNG_TABLE)
    seeds = np.array([e[0] for e in RNG_TABLE], dtype=np.uint64).view(np.int64)
    rows = np.array([e[1] for e in RNG_TABLE], dtype=np.uint64).view(np.int64)
    ids = np.array([e[2] for e in RNG_TABLE], dtype=np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    one = d(np.ones(n, dtype=np.float32))
    _, words = ts.gumbel_keys(one, one, one, d(seeds), d(rows), d(ids))
    got = words.cpu().numpy().view(np.uint32).tolist()
    assert got == [_table_word(e) for e in RNG_TABLE]
