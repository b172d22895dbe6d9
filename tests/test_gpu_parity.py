"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: logits within 2e-3 absolute (fp32 MFMA accumulation vs float64);
log-probabilities within 1e-4; token ids, top-N ids and row status bit-exact,
except token ids on rows the oracle flags (the token depends on where within
1e-5 of p the top-p boundary falls, or the two best Gumbel keys lie within
1e-5), which must stay below 0.1% of each test's rows (so none in a test of
fewer than 1,000 rows); slice assembly bit-exact.
"""
import math
import os
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOGIT_TOL = 2e-3
LOGPROB_TOL = 1e-4


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


def _bf16_to_device(bits, dev):
    import torch

    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)


def _bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------ GEMM
# Every projection tile shape (see the dispatch in lmhead_gemm.hip); "" is the
# size-based default.
GEMM_TILES = ["", "1", "2", "3", "4", "5"]


@pytest.fixture(params=GEMM_TILES)
def gemm_tile(request, monkeypatch):
    if request.param:
        monkeypatch.setenv("TS_GEMM_TILE", request.param)
    else:
        monkeypatch.delenv("TS_GEMM_TILE", raising=False)
    return request.param


def test_gemm_tiny_workload(dev, ts, gemm_tile):
    w = workloads.get("tiny")
    xb, wb = workloads.make_projection_host(w)
    say("gemm tiny", xb.shape, wb.shape)
    out = ts.lmhead_logits_local(_bf16_to_device(xb, dev), _bf16_to_device(wb, dev))
    ref = oracle.lmhead_logits(xb, wb)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max()
    assert err <= LOGIT_TOL, err


@pytest.mark.parametrize("rows,vocab,hidden", [
    (1, 300, 64), (4, 4096, 256), (63, 1000, 520), (65, 513, 136), (129, 777, 264),
    (257, 1031, 1032), (300, 2000, 8), (640, 700, 4096), (65, 513, 128), (257, 1031, 1024),
    (333, 300, 192), (700, 1500, 64)])
def test_gemm_ragged(dev, ts, rows, vocab, hidden, gemm_tile):
    rng = np.random.default_rng(rows * 7 + vocab)
    xb = workloads.bf16_bits_from_f32(rng.standard_normal((rows, hidden)).astype(np.float32))
    wb = workloads.bf16_bits_from_f32(
        (rng.standard_normal((vocab, hidden)) / np.sqrt(hidden)).astype(np.float32))
    say("gemm", rows, vocab, hidden)
    out = ts.lmhead_logits_local(_bf16_to_device(xb, dev), _bf16_to_device(wb, dev))
    ref = oracle.lmhead_logits(xb, wb)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max()
    assert err <= LOGIT_TOL, err


def test_gemm_slices_into_wide_buffer(dev, ts, gemm_tile):
    """Vocabulary slices written through ld_logits into one buffer equal one
    full projection bit for bit, and columns outside the slices are untouched."""
    import torch

    rng = np.random.default_rng(3)
    rows, vocab, hidden = 200, 1500, 512
    x = _bf16_to_device(workloads.bf16_bits_from_f32(
        rng.standard_normal((rows, hidden)).astype(np.float32)), dev)
    wt = _bf16_to_device(workloads.bf16_bits_from_f32(
        (rng.standard_normal((vocab, hidden)) * 0.05).astype(np.float32)), dev)
    say("gemm slices")
    full = ts.lmhead_logits_local(x, wt)
    wide = torch.full((rows, vocab + 37), 7.0, device=dev)
    cuts = [0, 333, 334, 1024, vocab]
    for a, b in zip(cuts[:-1], cuts[1:]):
        ts.lmhead_logits_local(x, wt[a:b], out=wide[:, a:b])
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :vocab], full)
    assert torch.all(wide[:, vocab:] == 7.0)


@pytest.mark.parametrize("vocab,ld", [(1001, 1028), (1023, 1024), (258, 264), (5, 8)])
def test_gemm_row_stores_ragged_tail(dev, ts, vocab, ld, gemm_tile):
    """An output whose rows take 16-byte stores (aligned base, leading
    dimension a multiple of 4) but whose width is not a multiple of 4: the
    row tail is written element by element and the padding stays untouched."""
    import torch

    rng = np.random.default_rng(vocab)
    rows, hidden = 333, 256
    xb = workloads.bf16_bits_from_f32(rng.standard_normal((rows, hidden)).astype(np.float32))
    wb = workloads.bf16_bits_from_f32(
        (rng.standard_normal((vocab, hidden)) / np.sqrt(hidden)).astype(np.float32))
    say("gemm row stores", vocab, ld)
    wide = torch.full((rows, ld), float("nan"), device=dev)
    ts.lmhead_logits_local(_bf16_to_device(xb, dev), _bf16_to_device(wb, dev),
                           out=wide[:, :vocab])
    torch.cuda.synchronize()
    full = wide.cpu().numpy()
    assert np.all(np.isnan(full[:, vocab:]))
    err = np.abs(full[:, :vocab].astype(np.float64) - oracle.lmhead_logits(xb, wb)).max()
    assert err <= LOGIT_TOL, err


@pytest.mark.parametrize("name,tile", [("decode", ""), ("spec_decode", ""), ("large", ""),
                                       ("draft", ""), ("spec_decode", "3"), ("large", "4")])
def test_gemm_full_size_sampled(dev, ts, name, tile, monkeypatch):
    """Full-size projection in the launch configuration the bench times,
    checked on sampled rows and columns (including the ragged tails)."""
    import torch

    if tile:
        monkeypatch.setenv("TS_GEMM_TILE", tile)
    else:
        monkeypatch.delenv("TS_GEMM_TILE", raising=False)
    w = workloads.get(name)
    say("gemm full", name, tile)
    x, wt = workloads.make_projection_device(w, dev)
    out = ts.lmhead_logits_local(x, wt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.index)
    rows = np.unique(np.concatenate([rng.choice(w.rows, 6, replace=False), [0, w.rows - 1]]))
    cols = np.unique(np.concatenate([rng.choice(w.vocab, 3000, replace=False),
                                     np.arange(w.vocab - 300, w.vocab)]))
    xb = _bits(x)
    # whole rows for two rows (one pass over the lm_head)
    full_rows = rows[:2]
    ref = oracle.lmhead_logits(xb[full_rows], _bits(wt))
    got = out[torch.from_numpy(full_rows).to(dev)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max()
    assert err <= LOGIT_TOL, err
    # every row at the sampled columns
    wsel = _bits(wt[torch.from_numpy(cols).to(dev)])
    ref = oracle.lmhead_logits(xb, wsel)
    got = out[:, torch.from_numpy(cols).to(dev)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max()
    assert err <= LOGIT_TOL, err


# --------------------------------------------------------------- assembly
def test_assemble_rank_share(dev, ts):
    import torch

    w = workloads.get("rank_share")
    logits = torch.from_numpy(workloads.make_logits(w)).to(dev)
    cuts = np.concatenate([[0], np.cumsum(w.slice_cols)])
    slices = [logits[:, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])]
    say("assemble rank_share", [s.shape for s in slices])
    out = ts.sampler_assemble_vocab_slices(slices)
    torch.cuda.synchronize()
    assert torch.equal(out, logits)


@pytest.mark.parametrize("widths,ld_extra,rows", [
    ([5, 1, 4097, 3], 0, 7), ([4, 8, 12], 0, 3), ([4, 8, 12], 5, 9), ([9000], 3, 2),
    ([1] * 64, 0, 5), ([0, 17, 0, 4], 2, 4)])
def test_assemble_ragged(dev, ts, widths, ld_extra, rows):
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(sum(widths) + rows)
    slices = []
    for c in widths:
        base = torch.randn(rows, c + ld_extra, generator=g, device=dev)
        slices.append(base[:, :c])
    say("assemble", widths, ld_extra, rows)
    out = torch.full((rows, sum(widths) + 3), 5.0, device=dev)
    ts.sampler_assemble_vocab_slices(slices, out=out[:, :sum(widths)])
    ref = oracle.assemble_vocab_slices([s.cpu().numpy() for s in slices])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[:, :sum(widths)].view(np.uint32), ref.view(np.uint32))
    assert np.all(got[:, sum(widths):] == 5.0)


# ---------------------------------------------------------------- sampler
def _run_sampler(ts, dev, logits_np, params, row_offset, max_logprobs, ld_extra=0,
                 processed=False):
    import torch

    rows, vocab = logits_np.shape
    if ld_extra:
        buf = torch.full((rows, vocab + ld_extra), float("nan"), device=dev)
        buf[:, :vocab] = torch.from_numpy(logits_np).to(dev)
        logits = buf[:, :vocab]
    else:
        logits = torch.from_numpy(np.ascontiguousarray(logits_np)).to(dev)
    p = ts.params_to_device(params, dev)
    out = ts.sampler_sample(logits, p, row_offset=row_offset, max_logprobs=max_logprobs,
                            processed=processed)
    torch.cuda.synchronize()
    return {k: getattr(out, k).cpu().numpy() for k in
            ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")}


def _compare(got, ref_tokens, ref_tlp, ref_topn_ids, ref_topn_lp, ref_status, flagged, lse,
             logits_np, max_frac=1e-3, label=""):
    rows = ref_tokens.shape[0]
    np.testing.assert_array_equal(got["row_status"], ref_status)
    ok = ref_status == 0
    bad = ~ok
    assert np.all(got["token_ids"][bad] == -1)
    assert np.all(np.isnan(got["token_logprobs"][bad]))
    mism = (got["token_ids"] != ref_tokens) & ok
    assert not np.any(mism & ~flagged), (label, np.nonzero(mism & ~flagged)[0][:10])
    assert flagged.sum() <= max_frac * rows, (label, flagged.sum())
    np.testing.assert_array_equal(got["topn_ids"][ok], ref_topn_ids[ok])
    fin = np.isfinite(ref_topn_lp[ok])
    assert np.array_equal(np.isfinite(got["topn_logprobs"][ok]), fin)
    assert np.abs(got["topn_logprobs"][ok][fin] - ref_topn_lp[ok][fin]).max(initial=0) <= LOGPROB_TOL
    # the sampled token's raw log-probability, for whichever token was drawn
    r_ok = np.nonzero(ok)[0]
    tok = got["token_ids"][r_ok]
    want = logits_np[r_ok, tok].astype(np.float64) - lse[r_ok]
    assert np.abs(got["token_logprobs"][r_ok] - want).max(initial=0) <= LOGPROB_TOL
    return int(mism.sum())


def _load_expected(name):
    return dict(np.load(os.path.join(GOLDEN, f"sampler_expected_{name}.npz")))


ROUTES = {"fast": {}, "exact": {"TS_SAMPLER_EXACT": "1"}, "probe": {"TS_SAMPLER_FORCE_PROBE": "1"}}


@pytest.fixture(params=list(ROUTES))
def route(request, monkeypatch):
    """The sampler's routes: the single-read fast path, the exact per-row
    kernel for every row, and the probe pass for every top-p-only row.  All
    must match the oracle."""
    for k in ("TS_SAMPLER_EXACT", "TS_SAMPLER_FORCE_PROBE"):
        monkeypatch.delenv(k, raising=False)
    for k, v in ROUTES[request.param].items():
        monkeypatch.setenv(k, v)
    return request.param


@pytest.mark.parametrize("name", ["tiny", "decode", "spec_decode", "rank_share", "large", "draft",
                                  "fp8"])
def test_sampler_workloads(dev, ts, name, route):
    import torch

    w = workloads.get(name)
    exp = _load_expected(name)
    params = workloads.make_params(w)
    assert str(exp["params_digest"]) == __import__("hashlib").sha256(
        np.ascontiguousarray(params).tobytes()).hexdigest()
    if name == "tiny":
        logits = exp["logits"]
    else:
        logits = workloads.make_logits(w)
        for (r0, r1), dg in zip(exp["digest_rows"], exp["logits_digests"]):
            assert __import__("hashlib").sha256(
                np.ascontiguousarray(logits[r0:r1]).tobytes()).hexdigest() == dg
    say("sampler", name, route, logits.shape)
    if name == "rank_share":
        # receive side: four vocabulary slices assembled on the device, then sampled
        cuts = np.concatenate([[0], np.cumsum(w.slice_cols)])
        full = torch.from_numpy(logits).to(dev)
        slices = [full[:, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])]
        del full
        assembled = ts.sampler_assemble_vocab_slices(slices)
        p = ts.params_to_device(params, dev)
        out = ts.sampler_sample(assembled, p, 0, w.max_logprobs)
        torch.cuda.synchronize()
        got = {k: getattr(out, k).cpu().numpy() for k in
               ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")}
    else:
        got = _run_sampler(ts, dev, logits, params, 0, w.max_logprobs)
    flagged = exp["flag_top_p"] | exp["flag_tie"]
    mism = _compare(got, exp["token_ids"], exp["token_logprobs"], exp["topn_ids"],
                    exp["topn_logprobs"], exp["row_status"], flagged, exp["lse"], logits,
                    label=name)
    say(f"{name}/{route}: rows={w.rows} flagged={int(flagged.sum())} mismatched_flagged={mism}")


def _oracle_ref(logits, params, row_offset, max_logprobs):
    res = oracle.sample(logits, params, row_offset, max_logprobs)
    l64 = logits.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.where(np.isfinite(l64), l64, -np.inf).max(axis=1)
        lse = m + np.log(np.exp(l64 - m[:, None]).sum(axis=1))
    return res, lse


def _edge_case(rng, V, rows, kind):
    if kind == "ints":
        l = rng.integers(-4, 5, size=(rows, V)).astype(np.float32)
    elif kind == "const":
        l = np.full((rows, V), 0.25, dtype=np.float32)
    elif kind == "neginf":
        l = rng.standard_normal((rows, V)).astype(np.float32)
        l[rng.random((rows, V)) < 0.7] = -np.inf
        l[:, 0] = np.where(np.all(np.isneginf(l), axis=1), 1.0, l[:, 0])
    elif kind == "wide":
        l = (rng.standard_normal((rows, V)) * 30).astype(np.float32)
    else:
        l = rng.standard_normal((rows, V)).astype(np.float32)
    return l


@pytest.mark.parametrize("V", [1, 2, 3, 7, 64, 1000, 4097, 20000, 70001])
@pytest.mark.parametrize("kind", ["normal", "ints", "const", "neginf", "wide"])
def test_sampler_edge_cases(dev, ts, V, kind, route):
    rng = np.random.default_rng(V * 10 + len(kind))
    rows = 24
    logits = _edge_case(rng, V, rows, kind)
    max_lp = 7
    params = workloads.random_params(rng, rows, V, max_lp)
    say("sampler edge", V, kind, route)
    got = _run_sampler(ts, dev, logits, params, 5, max_lp, ld_extra=3)
    res, lse = _oracle_ref(logits, params, 5, max_lp)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=f"{V}/{kind}")


@pytest.mark.parametrize("layout", ["crowded", "spread"])
def test_sampler_large_targets(dev, ts, layout, route):
    """Large top-k / top-N rows: with the largest logits crowded into one
    stretch of the vocabulary, every chunk's share of the list is too short
    and the row must still come out exact."""
    rng = np.random.default_rng(11 if layout == "crowded" else 12)
    rows, V, max_lp = 8, 70000, 300
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    if layout == "crowded":
        for r in range(rows):
            start = int(rng.integers(0, V - 3000))
            logits[r, start:start + 3000] += 6.0
    params = workloads.random_params(rng, rows, V, max_lp)
    params["top_k"] = np.array([1000, 300, 65, 1024, 0, 1000, 200, 700], dtype=np.int32)
    params["n_logprobs"] = np.array([300, 0, 300, 5, 300, 100, 65, 299], dtype=np.int32)
    params["temperature"][:] = 0.9
    say("sampler large targets", layout, route)
    got = _run_sampler(ts, dev, logits, params, 3, max_lp)
    res, lse = _oracle_ref(logits, params, 3, max_lp)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=layout)


def test_sampler_topk_beyond_fast_route(dev, ts, route):
    """top_k between 1,024 and V: up to 2,048 on the fast route, beyond it
    the exact per-row kernel (with and without top-p, with top-N)."""
    rng = np.random.default_rng(21)
    rows, V, max_lp = 10, 20000, 20
    logits = (rng.standard_normal((rows, V)) * 1.5).astype(np.float32)
    params = workloads.random_params(rng, rows, V, max_lp, greedy_frac=0.0)
    params["top_k"] = np.array([1025, 1500, 2048, 5000, 19999, 1025, 3000, 1100, 8191, 1024],
                               dtype=np.int32)
    params["top_p"] = np.array([1.0, 0.9, 1.0, 0.7, 0.95, 0.5, 1.0, 0.8, 0.99, 0.9],
                               dtype=np.float32)
    say("sampler top_k beyond the fast route", route)
    got = _run_sampler(ts, dev, logits, params, 2, max_lp)
    res, lse = _oracle_ref(logits, params, 2, max_lp)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="topk>1024")


@pytest.mark.parametrize("p_top", [1.0, 0.8])
def test_sampler_topk2048_rows(dev, ts, p_top, route):
    """64 rows with top_k = 2,048 at the full vocabulary (the fast route's
    largest top-k, one merge list of about four thousand candidates), with
    and without top-p, against the oracle."""
    w = workloads.get("spec_decode")
    rows = 64
    logits = workloads.make_logits(w, slice(0, rows))
    params = np.zeros(rows, dtype=workloads.PARAMS_DTYPE)
    params["temperature"] = np.linspace(0.4, 1.2, rows).astype(np.float32)
    params["top_k"] = 2048
    params["top_p"] = p_top
    params["n_logprobs"] = np.arange(rows) % 21
    params["seed"] = np.arange(rows, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15) + np.uint64(5)
    say("sampler top_k 2048", p_top, route)
    got = _run_sampler(ts, dev, logits, params, 0, 20)
    res, lse = _oracle_ref(logits, params, 0, 20)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=f"topk2048/{p_top}")


def test_sampler_many_rows_mixed_kinds(dev, ts, route):
    """2,600 rows of every kind, interleaved (greedy, short and long top-k,
    top-k beyond the fast route, top-p only, no filter, invalid parameters),
    with a row offset: more rows than the chunk pass's row-order pre-pass
    keeps in registers (it reads the remaining rows' parameters twice), so
    its class counts, slots and second read are all exercised."""
    rows, V = 2600, 3000
    g = np.random.default_rng(2600)
    logits = (g.standard_normal((rows, V)) * 1.3).astype(np.float32)
    params = np.zeros(rows, dtype=workloads.PARAMS_DTYPE)
    kinds = [(0.0, 0, 1.0), (0.8, 20, 1.0), (0.7, 700, 0.9), (0.9, 2500, 0.95), (1.0, 0, 0.85),
             (0.6, 0, 1.0), (-1.0, 0, 1.0), (1.1, 50, 0.7), (0.5, 1, 1.0), (0.8, 0, 0.6)]
    for r in range(rows):
        t, k, p = kinds[(r * 7 + r // 13) % len(kinds)]
        params[r] = (t, k, p, r % 6, 0)
    params["seed"] = np.arange(rows, dtype=np.uint64) * np.uint64(0xD1B54A32D192ED03) + np.uint64(11)
    say("sampler many rows", rows, V, route)
    got = _run_sampler(ts, dev, logits, params, 77, 5)
    res, lse = _oracle_ref(logits, params, 77, 5)
    assert (res.row_status == 1).sum() == (params["temperature"] < 0).sum() > 0
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="many rows")


def test_sampler_probes_outside_nucleus(dev, ts, route):
    """Top-p-only rows whose nucleus (about 120 of 200 raised logits) is past
    the listed head but holds only a tenth of the mass: the best Gumbel keys
    mostly fall outside it, so many rows keep none of their probes and go to
    the exact kernel; every row must still match the oracle."""
    rng = np.random.default_rng(22)
    rows, V, max_lp = 16, 20000, 5
    logits = (rng.standard_normal((rows, V)) * 0.1).astype(np.float32)
    for r in range(rows):
        hot = rng.choice(V, size=200, replace=False)
        logits[r, hot] += 3.0
    params = workloads.random_params(rng, rows, V, max_lp, greedy_frac=0.0)
    params["temperature"][:] = 1.0
    params["top_k"][:] = 0
    params["top_p"][:] = 0.1
    say("sampler probes outside the nucleus", route)
    got = _run_sampler(ts, dev, logits, params, 9, max_lp)
    res, lse = _oracle_ref(logits, params, 9, max_lp)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="probe-fallback")


def test_sampler_bad_rows(dev, ts, route):
    rng = np.random.default_rng(0)
    rows, V = 12, 500
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    logits[1, 7] = np.nan
    logits[2, 9] = np.inf
    logits[3, :] = -np.inf
    params = workloads.random_params(rng, rows, V, 4)
    params["temperature"][4] = -1.0
    params["top_k"][5] = -2
    params["top_p"][6] = 0.0
    params["top_p"][7] = 1.5
    params["n_logprobs"][8] = 5
    params["temperature"][9] = np.inf
    params["top_p"][10] = np.nan
    params["temperature"][11] = np.nan
    say("sampler bad rows")
    got = _run_sampler(ts, dev, logits, params, 0, 4)
    res, lse = _oracle_ref(logits, params, 0, 4)
    assert got["row_status"].tolist() == [0, 2, 2, 2, 1, 1, 1, 1, 1, 1, 1, 1]
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits)
    assert np.all(np.isnan(got["topn_logprobs"][1:]))


@pytest.mark.parametrize("max_lp,n", [(0, 0), (300, 300), (1024, 700)])
def test_sampler_logprob_widths(dev, ts, max_lp, n, route):
    rng = np.random.default_rng(max_lp)
    rows, V = 6, 3000
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    logits[0, 100:400] = 2.0   # a long tie run inside the top-N
    params = workloads.random_params(rng, rows, V, max_lp)
    params["n_logprobs"] = n
    say("sampler widths", max_lp, n)
    got = _run_sampler(ts, dev, logits, params, 0, max_lp)
    res, lse = _oracle_ref(logits, params, 0, max_lp)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits)


def test_sampler_long_topk_tie_runs(dev, ts, route):
    """Top-k sets longer than 192 (settled by selection, not sorting) whose
    top-k boundary or top-p boundary falls inside a long run of equal
    logits: more tied entries than one per thread of the merge workgroup."""
    rng = np.random.default_rng(23)
    rows, V = 12, 3000
    logits = (rng.standard_normal((rows, V)) - 3.0).astype(np.float32)
    for r in range(rows):
        run = [600, 300, 900][r % 3]
        logits[r, rng.choice(V, run, replace=False)] = 2.0   # a tie run at the top
    logits[6:, rng.choice(V, 50, replace=False)] = 2.5      # a few above the run
    params = np.zeros(rows, dtype=workloads.PARAMS_DTYPE)
    params["temperature"] = 0.9
    params["top_k"] = np.array([500, 1000, 250, 700] * 3, dtype=np.int32)
    params["top_p"] = np.array([0.5, 0.9, 1.0] * 4, dtype=np.float32)
    params["n_logprobs"] = 5
    params["seed"] = np.arange(rows, dtype=np.uint64) + np.uint64(77)
    say("sampler long top-k tie runs", route)
    got = _run_sampler(ts, dev, logits, params, 0, 5)
    res, lse = _oracle_ref(logits, params, 0, 5)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="tie runs")
    assert np.all(got["row_status"] == 0)


def test_sampler_long_topk_probe_fallback(dev, ts, route):
    """Top-k sets longer than 192 with top-p: the merge first checks the
    list's eight best Gumbel keys against the top-p mass and searches the
    boundary only when none is kept.  With p of a few percent on flat logits
    the kept set is a handful of tokens and the eight probes all fall outside
    it (the search runs); with p near 1 the first probe is kept."""
    rng = np.random.default_rng(29)
    rows, V = 24, 20000
    logits = (rng.standard_normal((rows, V)) * 1.2).astype(np.float32)
    params = np.zeros(rows, dtype=workloads.PARAMS_DTYPE)
    params["temperature"] = np.array([0.5, 1.5] * 12, dtype=np.float32)
    params["top_k"] = np.array([300, 1000, 2000] * 8, dtype=np.int32)
    params["top_p"] = np.repeat(np.array([0.01, 0.03, 0.9, 0.99], dtype=np.float32), 6)
    params["n_logprobs"] = np.arange(rows) % 9
    params["seed"] = np.arange(rows, dtype=np.uint64) * np.uint64(977) + np.uint64(13)
    say("sampler long top-k probe fallback", route)
    got = _run_sampler(ts, dev, logits, params, 5, 8)
    res, lse = _oracle_ref(logits, params, 5, 8)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="probe fallback")
    assert np.all(got["row_status"] == 0)


def _kept_by_definition(l, t, k, p):
    """The kept set written out from its definition, by brute force on a
    short row: v is in the top-k set iff fewer than k logits are strictly
    larger (k = 0: every token), and kept iff the temperature-scaled mass of
    the top-k tokens with a strictly larger logit is below p times the set's
    mass."""
    n = len(l)
    top = [v for v in range(n) if k == 0 or sum(l[u] > l[v] for u in range(n)) < k]
    if p >= 1.0:
        return top
    m = max(l)
    w = {u: math.exp((l[u] - m) / t) for u in top}
    z = math.fsum(w.values())
    return [v for v in top if math.fsum(w[u] for u in top if l[u] > l[v]) < p * z]


@pytest.mark.parametrize("t,k,p", [(1.0, 0, 1.0), (0.6, 0, 0.8), (1.4, 4, 1.0), (0.9, 5, 0.7)])
def test_gumbel_max_frequencies_chi_square(dev, ts, t, k, p, route):
    """The sampled tokens follow the filtered softmax (the Gumbel-max
    theorem): one row repeated over 200,000 rows, each drawing its own noise
    (the generator is keyed on the row), token frequencies against
    softmax(l / T) over the kept set under a chi-square test; no token outside
    the kept set is ever drawn."""
    import scipy.stats

    l = np.array([1.2, 0.3, -0.4, 0.9, 0.0, -1.0, 0.5], dtype=np.float32)
    kept = _kept_by_definition([float(x) for x in l], t, k, p)
    z = np.exp((l[kept].astype(np.float64) - l.max()) / t)
    probs = z / z.sum()
    draws = 200_000
    logits = np.ascontiguousarray(np.broadcast_to(l, (draws, l.size)))
    params = np.zeros(draws, dtype=workloads.PARAMS_DTYPE)
    params["temperature"], params["top_k"], params["top_p"] = t, k, p
    params["seed"] = 1234
    say("gumbel chi-square", t, k, p, route)
    got = _run_sampler(ts, dev, logits, params, 0, 0)
    assert np.all(got["row_status"] == 0)
    counts = np.bincount(got["token_ids"], minlength=l.size)
    assert counts[[v for v in range(l.size) if v not in kept]].sum() == 0
    if len(kept) > 1:
        assert scipy.stats.chisquare(counts[kept], probs * draws).pvalue > 1e-3
    else:
        assert counts[kept[0]] == draws


def test_sampler_row_offset_split_matches_single_call(dev, ts):
    """A rank's share of rows (row_offset) draws exactly what one call over all
    rows draws: the RNG is keyed on the global row."""
    w = workloads.get("spec_decode")
    rng = np.random.default_rng(8)
    rows, V = 40, 5000
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    params = workloads.random_params(rng, rows, V, 5, greedy_frac=0.0)
    say("sampler split", w.name)
    whole = _run_sampler(ts, dev, logits, params, 100, 5)
    a = _run_sampler(ts, dev, logits[:17], params[:17], 100, 5)
    b = _run_sampler(ts, dev, logits[17:], params[17:], 117, 5)
    for k in whole:
        np.testing.assert_array_equal(np.concatenate([a[k], b[k]]), whole[k])


def test_sampler_deterministic(dev, ts):
    rng = np.random.default_rng(4)
    rows, V = 32, 30000
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    params = workloads.random_params(rng, rows, V, 8)
    say("sampler determinism")
    a = _run_sampler(ts, dev, logits, params, 0, 8)
    b = _run_sampler(ts, dev, logits, params, 0, 8)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_gumbel_noise_on_flat_rows(dev, ts, route):
    """With every logit equal, the sampled token is the argmax of the Gumbel
    noise alone, so these rows check the noise itself (Philox words, the
    uniform map and both logarithms) against the oracle's float64 values."""
    rows, V = 48, 50000
    logits = np.full((rows, V), 0.5, dtype=np.float32)
    params = np.zeros(rows, dtype=workloads.PARAMS_DTYPE)
    params["temperature"] = np.linspace(0.3, 1.7, rows).astype(np.float32)
    params["top_p"] = np.where(np.arange(rows) % 2 == 0, 1.0, 0.999).astype(np.float32)
    params["n_logprobs"] = 3
    params["seed"] = np.arange(rows, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
    say("flat rows", route)
    got = _run_sampler(ts, dev, logits, params, 1 << 33, 3)
    res, lse = _oracle_ref(logits, params, 1 << 33, 3)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="flat")
    assert res.flagged.sum() <= 1


# ------------------------------------------------ sampler over vocab slices
def _run_sampler_slices(ts, dev, logits_np, widths, params, row_offset, max_logprobs, ld_extra=0,
                        processed=False):
    """sampler_sample_slices over ``logits_np`` cut column-wise into ``widths``
    (each slice its own buffer; with ld_extra, a NaN-padded wider buffer)."""
    import torch

    rows, vocab = logits_np.shape
    assert sum(widths) == vocab
    cuts = np.concatenate([[0], np.cumsum(widths)]).astype(np.int64)
    full = torch.from_numpy(np.ascontiguousarray(logits_np)).to(dev)
    slices = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if ld_extra:
            buf = torch.full((rows, b - a + ld_extra), float("nan"), device=dev)
            buf[:, :b - a] = full[:, a:b]
            slices.append(buf[:, :b - a])
        else:
            slices.append(full[:, a:b].contiguous())
    del full
    p = ts.params_to_device(params, dev)
    out = ts.sampler_sample_slices(slices, p, row_offset=row_offset, max_logprobs=max_logprobs,
                                   processed=processed)
    torch.cuda.synchronize()
    return {k: getattr(out, k).cpu().numpy() for k in
            ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")}


def _even_widths(V, n, align=1):
    base = V // n // align * align
    w = [base] * n
    w[-1] += V - base * n
    return w


@pytest.mark.parametrize("name,n", [("spec_decode", 4), ("spec_decode", 8), ("rank_share", 0),
                                    ("large", 8), ("fp8", 0)])
def test_sampler_slices_workloads(dev, ts, name, n, route):
    """The receive side without the stitching copy: the sampler reads the
    vocabulary slices where the exchange left them."""
    w = workloads.get(name)
    exp = _load_expected(name)
    params = workloads.make_params(w)
    logits = workloads.make_logits(w)
    widths = list(w.slice_cols) if n == 0 else _even_widths(w.vocab, n)
    say("sampler slices", name, widths, route)
    got = _run_sampler_slices(ts, dev, logits, widths, params, 0, w.max_logprobs)
    flagged = exp["flag_top_p"] | exp["flag_tie"]
    mism = _compare(got, exp["token_ids"], exp["token_logprobs"], exp["topn_ids"],
                    exp["topn_logprobs"], exp["row_status"], flagged, exp["lse"], logits,
                    label=f"{name}/slices")
    say(f"{name}/slices/{route}: flagged={int(flagged.sum())} mismatched_flagged={mism}")


SLICE_LAYOUTS = {
    "one": lambda V: [V],
    "aligned4": lambda V: _even_widths(V, 4, align=4),
    "ragged_tail": lambda V: [4, 1236] + _even_widths(V - 1240, 2, align=4),
    "misaligned": lambda V: [V // 3 + 1, V // 3 - 2, V - 2 * (V // 3) + 1],
    "empties": lambda V: [0, V // 2 // 4 * 4, 0, V - V // 2 // 4 * 4, 0],
    "many64": lambda V: _even_widths(V, 64, align=4),
    "many64_odd": lambda V: [469] * 63 + [V - 469 * 63],
}


@pytest.mark.parametrize("layout", list(SLICE_LAYOUTS))
@pytest.mark.parametrize("kind", ["normal", "neginf", "ints"])
def test_sampler_slices_layouts(dev, ts, layout, kind, route):
    rng = np.random.default_rng(len(layout) * 7 + len(kind))
    rows = 20
    V = 30011 if layout in ("ragged_tail", "misaligned", "many64_odd") else 30008
    logits = _edge_case(rng, V, rows, kind)
    params = workloads.random_params(rng, rows, V, 9)
    widths = SLICE_LAYOUTS[layout](V)
    say("sampler slice layout", layout, kind, route, widths[:6])
    ld_extra = {"normal": 0, "neginf": 4, "ints": 5}[kind]
    got = _run_sampler_slices(ts, dev, logits, widths, params, 11, 9, ld_extra=ld_extra)
    res, lse = _oracle_ref(logits, params, 11, 9)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=f"{layout}/{kind}")


@pytest.mark.parametrize("V,widths", [(1, [1]), (3, [1, 1, 1]), (7, [0, 4, 3]), (9, [4, 4, 1]),
                                      (1000, [1000, 0])])
def test_sampler_slices_tiny(dev, ts, V, widths, route):
    rng = np.random.default_rng(V)
    rows = 10
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    params = workloads.random_params(rng, rows, V, 3)
    say("sampler slices tiny", V, widths, route)
    got = _run_sampler_slices(ts, dev, logits, widths, params, 0, 3)
    res, lse = _oracle_ref(logits, params, 0, 3)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=f"tiny{V}")


@pytest.mark.parametrize("layout", ["crowded", "spread"])
def test_sampler_slices_large_targets(dev, ts, layout, route):
    """Large top-k / top-N with the heavy stretch of the row inside one slice
    or across a slice boundary."""
    rng = np.random.default_rng(21 if layout == "crowded" else 22)
    rows, V, max_lp = 8, 70000, 300
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    if layout == "crowded":
        for r in range(rows):
            start = 17500 * (r % 4) - 1500 if r % 4 else 100
            logits[r, start:start + 3000] += 6.0
    params = workloads.random_params(rng, rows, V, max_lp)
    params["top_k"] = np.array([1000, 300, 65, 1024, 0, 1000, 200, 700], dtype=np.int32)
    params["n_logprobs"] = np.array([300, 0, 300, 5, 300, 100, 65, 299], dtype=np.int32)
    params["temperature"][:] = 0.9
    say("sampler slices large targets", layout, route)
    got = _run_sampler_slices(ts, dev, logits, [17500] * 4, params, 3, max_lp)
    res, lse = _oracle_ref(logits, params, 3, max_lp)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=layout)


def test_sampler_one_slice_matches_buffer_call(dev, ts):
    """One slice is the stitched buffer itself: same chunking, so the two
    calls agree bit for bit."""
    rng = np.random.default_rng(31)
    rows, V = 48, 40000
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    params = workloads.random_params(rng, rows, V, 6)
    say("sampler one slice vs buffer")
    a = _run_sampler(ts, dev, logits, params, 7, 6)
    b = _run_sampler_slices(ts, dev, logits, [V], params, 7, 6)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


@pytest.mark.parametrize("in_place", [True, False])
def test_sampler_draft_share(dev, ts, in_place, route):
    """Sharded draft logits: one tensor-parallel rank's share of the draft
    step, received as eight vocabulary slices and sampled with the share's
    global row offset, draws exactly the draft step's tokens for those rows."""
    import torch

    w = workloads.get("draft_share")
    parent = workloads.get(w.parent)
    exp = _load_expected(parent.name)
    sl = slice(w.row_offset, w.row_offset + w.rows)
    logits = workloads.make_logits(w)
    params = workloads.make_params(w)
    say("draft share", in_place, route, logits.shape, w.slice_cols[:2])
    if in_place:
        got = _run_sampler_slices(ts, dev, logits, w.slice_cols, params, w.row_offset,
                                  w.max_logprobs)
    else:
        cuts = np.concatenate([[0], np.cumsum(w.slice_cols)])
        full = torch.from_numpy(logits).to(dev)
        slices = [full[:, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])]
        batch = ts.sampler_assemble_vocab_slices(slices)
        out = ts.sampler_sample(batch, ts.params_to_device(params, dev), w.row_offset,
                                w.max_logprobs)
        torch.cuda.synchronize()
        got = {k: getattr(out, k).cpu().numpy() for k in
               ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")}
    flagged = exp["flag_top_p"][sl] | exp["flag_tie"][sl]
    _compare(got, exp["token_ids"][sl], exp["token_logprobs"][sl], exp["topn_ids"][sl],
             exp["topn_logprobs"][sl], exp["row_status"][sl], flagged, exp["lse"][sl], logits,
             label="draft_share")


# ------------------------------------------ processed log-probabilities (R11)
def _compare_processed(got, res, label=""):
    """Ids and status exact; -inf pattern exact and finite values within
    1e-4 of the oracle's, except on rows whose top-p boundary or best keys the
    oracle flags (there the kept set, and so the values, may differ)."""
    np.testing.assert_array_equal(got["row_status"], res.row_status)
    ok = res.row_status == 0
    firm = ok & ~res.flagged
    mism = (got["token_ids"] != res.token_ids) & ok
    assert not np.any(mism & firm), (label, np.nonzero(mism & firm)[0][:10])
    np.testing.assert_array_equal(got["topn_ids"][ok], res.topn_ids[ok])
    g, w = got["topn_logprobs"][firm], res.topn_logprobs[firm]
    assert np.array_equal(np.isfinite(g), np.isfinite(w)), label
    fin = np.isfinite(w)
    assert np.abs(g[fin] - w[fin]).max(initial=0) <= LOGPROB_TOL, label
    gt, wt = got["token_logprobs"][firm], res.token_logprobs[firm]
    assert np.all(np.isfinite(gt)) and np.abs(gt - wt).max(initial=0) <= LOGPROB_TOL, label
    assert np.all(got["token_logprobs"][ok] <= LOGPROB_TOL)   # probabilities, not above 1


@pytest.mark.parametrize("name,slices", [("spec_decode", 1), ("spec_decode", 8),
                                         ("rank_share", 1), ("draft", 1)])
def test_sampler_processed_workloads(dev, ts, name, slices, route):
    w = workloads.get(name)
    logits = workloads.make_logits(w)
    params = workloads.make_params(w)
    say("sampler processed", name, slices, route)
    if slices > 1:
        got = _run_sampler_slices(ts, dev, logits, _even_widths(w.vocab, slices), params, 0,
                                  w.max_logprobs, processed=True)
    else:
        got = _run_sampler(ts, dev, logits, params, 0, w.max_logprobs, processed=True)
    res = oracle.sample(logits, params, 0, w.max_logprobs, processed=True)
    assert res.flagged.sum() <= 1e-3 * w.rows
    _compare_processed(got, res, label=name)


@pytest.mark.parametrize("V", [1, 7, 1000, 20000, 70001])
@pytest.mark.parametrize("kind", ["normal", "ints", "neginf", "wide"])
def test_sampler_processed_edge_cases(dev, ts, V, kind, route):
    rng = np.random.default_rng(V * 7 + len(kind))
    rows, max_lp = 24, 9
    logits = _edge_case(rng, V, rows, kind)
    params = workloads.random_params(rng, rows, V, max_lp)
    say("sampler processed edge", V, kind, route)
    got = _run_sampler(ts, dev, logits, params, 2, max_lp, ld_extra=3, processed=True)
    res = oracle.sample(logits, params, 2, max_lp, processed=True)
    assert res.flagged.sum() <= 1e-3 * rows
    _compare_processed(got, res, label=f"{V}/{kind}")


def test_sampler_processed_large_targets(dev, ts, route):
    rng = np.random.default_rng(41)
    rows, V, max_lp = 8, 70000, 300
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    for r in range(0, rows, 2):
        s0 = int(rng.integers(0, V - 3000))
        logits[r, s0:s0 + 3000] += 6.0
    params = workloads.random_params(rng, rows, V, max_lp)
    params["top_k"] = np.array([1000, 300, 65, 1024, 0, 1000, 200, 700], dtype=np.int32)
    params["top_p"] = np.array([1.0, 0.9, 0.5, 1.0, 0.7, 0.95, 1.0, 0.3], dtype=np.float32)
    params["n_logprobs"] = np.array([300, 0, 300, 5, 300, 100, 65, 299], dtype=np.int32)
    params["temperature"][:] = 0.9
    say("sampler processed large targets", route)
    got = _run_sampler(ts, dev, logits, params, 0, max_lp, processed=True)
    res = oracle.sample(logits, params, 0, max_lp, processed=True)
    assert res.flagged.sum() <= 1e-3 * rows
    _compare_processed(got, res, label="large targets")
