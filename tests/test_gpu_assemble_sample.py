"""GPU parity of sampler_assemble_and_sample: the stitched batch buffer is the
received slices bit for bit (every row, whatever route the sampler takes for
it), and the sampling outputs are the oracle's to the bars of test_gpu_parity,
with the same token ids, top-N ids and row status as the slice sampler."""
import numpy as np
import pytest

import workloads
from test_gpu_parity import (SLICE_LAYOUTS, _compare, _compare_processed, _edge_case,  # noqa: F401
                             _even_widths, _load_expected, _oracle_ref, dev, route, say, ts)

pytestmark = pytest.mark.gpu

FIELDS = ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")


def _slices_of(full, widths, ld_extra):
    import torch

    rows = full.shape[0]
    cuts = np.concatenate([[0], np.cumsum(widths)]).astype(np.int64)
    out = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if ld_extra:
            buf = torch.full((rows, b - a + ld_extra), float("nan"), device=full.device)
            buf[:, :b - a] = full[:, a:b]
            out.append(buf[:, :b - a])
        else:
            out.append(full[:, a:b].contiguous())
    return out


def _run(ts, dev, logits_np, widths, params, row_offset, max_lp, ld_extra=0, ld_out_extra=0,
         processed=False):
    """sampler_assemble_and_sample over logits_np cut into widths; returns the
    assembled buffer (host, with the padding columns), the outputs and the
    outputs of sampler_sample_slices on the same slices."""
    import torch

    rows, vocab = logits_np.shape
    full = torch.from_numpy(np.ascontiguousarray(logits_np)).to(dev)
    slices = _slices_of(full, widths, ld_extra)
    del full
    p = ts.params_to_device(params, dev)
    wide = torch.full((rows, vocab + ld_out_extra), 7.0, device=dev)
    assembled, out = ts.sampler_assemble_and_sample(
        slices, p, row_offset, max_lp, assembled=wide[:, :vocab], processed=processed)
    ref = ts.sampler_sample_slices(slices, p, row_offset=row_offset, max_logprobs=max_lp,
                                   processed=processed)
    torch.cuda.synchronize()
    got = {k: getattr(out, k).cpu().numpy() for k in FIELDS}
    sep = {k: getattr(ref, k).cpu().numpy() for k in FIELDS}
    return wide.cpu().numpy(), got, sep


def _check_assembled(wide, logits_np, ld_out_extra):
    vocab = logits_np.shape[1]
    assert np.array_equal(wide[:, :vocab].view(np.uint32), logits_np.view(np.uint32))
    if ld_out_extra:
        assert np.all(wide[:, vocab:] == 7.0)


def _same_outputs(got, sep):
    """The one-call sampler draws what the slice sampler draws.  It may cut
    the rows into narrower chunks, so its fp32 sums (and log-probabilities)
    may round differently in the last bits."""
    for k in ("token_ids", "topn_ids", "row_status"):
        assert np.array_equal(got[k], sep[k]), k
    for k in ("token_logprobs", "topn_logprobs"):
        a, b = got[k], sep[k]
        assert np.array_equal(np.isfinite(a), np.isfinite(b)), k
        assert np.array_equal(np.isnan(a), np.isnan(b)), k
        fin = np.isfinite(a)
        assert np.abs(a[fin] - b[fin]).max(initial=0) <= 1e-5, k


@pytest.mark.parametrize("name,n", [("spec_decode", 4), ("rank_share", 0), ("fp8", 0)])
def test_assemble_and_sample_workloads(dev, ts, name, n, route):
    w = workloads.get(name)
    exp = _load_expected(name)
    params = workloads.make_params(w)
    logits = workloads.make_logits(w)
    widths = list(w.slice_cols) if n == 0 else _even_widths(w.vocab, n)
    say("assemble+sample", name, widths[:4], route)
    wide, got, sep = _run(ts, dev, logits, widths, params, 0, w.max_logprobs)
    _check_assembled(wide, logits, 0)
    _same_outputs(got, sep)
    flagged = exp["flag_top_p"] | exp["flag_tie"]
    _compare(got, exp["token_ids"], exp["token_logprobs"], exp["topn_ids"], exp["topn_logprobs"],
             exp["row_status"], flagged, exp["lse"], logits, label=f"{name}/assemble")


def _special_values(rng, logits):
    """Bit patterns a copy must keep: -0.0, a NaN with a payload, +-inf and
    denormals, in a few rows (rows with NaN or +inf are reported bad)."""
    rows, V = logits.shape
    bits = logits.view(np.uint32)
    cols = rng.integers(0, V, size=6)
    bits[0, cols[0]] = 0x80000000            # -0.0
    bits[1, cols[1]] = 0x7FC0BEEF            # quiet NaN with a payload
    bits[2, cols[2]] = 0x7F800000            # +inf
    bits[3, cols[3]] = 0xFF800000            # -inf
    bits[4, cols[4]] = 0x00000001            # smallest denormal
    bits[5, cols[5]] = 0x807FFFFF            # largest negative denormal
    return logits


@pytest.mark.parametrize("layout", list(SLICE_LAYOUTS))
@pytest.mark.parametrize("ld_extra,ld_out_extra", [(0, 0), (3, 3), (0, 3)])
def test_assemble_and_sample_layouts(dev, ts, layout, ld_extra, ld_out_extra, route):
    """Every slice layout (aligned, ragged, misaligned starts, empty slices, 64
    slices), padded slice buffers, an output whose rows do or do not take
    16-byte stores, special bit patterns, rows with bad parameters and rows
    whose top_k sends them to the exact kernel: the copy is bit-exact in every
    row and the outputs are the oracle's."""
    rng = np.random.default_rng(len(layout) * 11 + ld_out_extra * 3 + ld_extra)
    rows = 24
    V = 30011 if layout in ("ragged_tail", "misaligned", "many64_odd") else 30008
    logits = _special_values(rng, _edge_case(rng, V, rows, "normal"))
    params = workloads.random_params(rng, rows, V, 9)
    params["top_k"][6] = 3000                # beyond the fast route: exact kernel
    params["temperature"][7] = -1.0          # bad parameters
    params["top_p"][8] = np.nan
    widths = SLICE_LAYOUTS[layout](V)
    say("assemble+sample layout", layout, ld_extra, ld_out_extra, route, widths[:6])
    wide, got, sep = _run(ts, dev, logits, widths, params, 5, 9, ld_extra=ld_extra,
                          ld_out_extra=ld_out_extra)
    _check_assembled(wide, logits, ld_out_extra)
    _same_outputs(got, sep)
    res, lse = _oracle_ref(logits, params, 5, 9)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=f"{layout}/assemble")


def test_assemble_and_sample_processed(dev, ts, route):
    """The processed-log-probability mode through the same call equals the
    slice sampler's."""
    w = workloads.get("spec_decode")
    params = workloads.make_params(w)[:160]
    logits = workloads.make_logits(w, slice(0, 160))
    say("assemble+sample processed", route)
    wide, got, sep = _run(ts, dev, logits, _even_widths(w.vocab, 4), params, 0, w.max_logprobs,
                          processed=True)
    _check_assembled(wide, logits, 0)
    _same_outputs(got, sep)


@pytest.mark.parametrize("V,widths", [(1, [1]), (7, [0, 4, 3]), (9, [4, 4, 1])])
def test_assemble_and_sample_tiny(dev, ts, V, widths, route):
    rng = np.random.default_rng(V + 100)
    rows = 5
    logits = rng.standard_normal((rows, V)).astype(np.float32)
    params = workloads.random_params(rng, rows, V, 3)
    wide, got, sep = _run(ts, dev, logits, widths, params, 0, 3, ld_out_extra=1)
    _check_assembled(wide, logits, 1)
    _same_outputs(got, sep)
    res, lse = _oracle_ref(logits, params, 0, 3)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label="tiny/assemble")


UNIFORM_KINDS = {
    "greedy": (0.0, 0, 1.0),
    "top_k_20": (0.7, 20, 1.0),
    "top_k_1000_top_p_0.8": (0.7, 1000, 0.8),
    "top_p_0.9": (0.9, 0, 0.9),
    "full_vocabulary": (1.0, 0, 1.0),
}


@pytest.mark.parametrize("n_slices", [4, 16])
@pytest.mark.parametrize("kind", list(UNIFORM_KINDS))
def test_assemble_and_sample_uniform_kind(dev, ts, kind, n_slices):
    """160 spec_decode rows, every row given the same temperature, top_k and
    top_p (the mix's n_logprobs): one route carries the whole grid.  The
    slice sampler and the buffer sampler draw the same as the one call.  Four
    slices take narrow chunks (20 a row) in the rows' own order; sixteen
    would make 32 narrow chunks a row, so they take wide ones (16 a row, 2,560
    in all) behind the row-order pre-pass.  With every row top-p-only each
    row is probed, 3,200 or 2,560 probe items for a 2,048-workgroup probe
    pass, so some of its workgroups take more than one."""
    w = workloads.get("spec_decode")
    params = workloads.make_params(w)[:160]
    params["temperature"], params["top_k"], params["top_p"] = UNIFORM_KINDS[kind]
    logits = workloads.make_logits(w, slice(0, 160))
    say("assemble+sample uniform kind", kind, n_slices)
    wide, got, sep = _run(ts, dev, logits, _even_widths(w.vocab, n_slices), params, 0,
                          w.max_logprobs)
    _check_assembled(wide, logits, 0)
    _same_outputs(got, sep)
    # The buffer sampler on the stitched rows draws the same.
    import torch

    buf = ts.sampler_sample(torch.from_numpy(wide).to(dev), ts.params_to_device(params, dev), 0,
                            w.max_logprobs)
    torch.cuda.synchronize()
    _same_outputs(got, {k: getattr(buf, k).cpu().numpy() for k in FIELDS})
    res, lse = _oracle_ref(logits, params, 0, w.max_logprobs)
    _compare(got, res.token_ids, res.token_logprobs, res.topn_ids, res.topn_logprobs,
             res.row_status, res.flagged, lse, logits, label=f"{kind}/{n_slices}/assemble")


@pytest.mark.parametrize("kind", list(UNIFORM_KINDS))
def test_assemble_and_sample_uniform_kind_processed(dev, ts, kind):
    """The processed-distribution log-probabilities of the one call on the
    one-row-kind batches (four slices) are the oracle's."""
    import oracle

    w = workloads.get("spec_decode")
    params = workloads.make_params(w)[:160]
    params["temperature"], params["top_k"], params["top_p"] = UNIFORM_KINDS[kind]
    logits = workloads.make_logits(w, slice(0, 160))
    say("assemble+sample uniform kind processed", kind)
    wide, got, sep = _run(ts, dev, logits, _even_widths(w.vocab, 4), params, 0, w.max_logprobs,
                          processed=True)
    _check_assembled(wide, logits, 0)
    _same_outputs(got, sep)
    res = oracle.sample(logits, params, 0, w.max_logprobs, processed=True)
    assert res.flagged.sum() <= 1e-3 * 160
    _compare_processed(got, res, label=f"{kind}/processed")
