"""Pins for the CPU oracle: each check ties it to something other than itself.

* Philox4x32-10: published known-answer vectors (tests/golden).
* Projection: exact rational dot products of bf16 values; one-hot weights.
* Top-k: O(V^2) rank counting.  Top-p: the membership characterisation
  "v is kept iff the mass of strictly larger logits in the top-k set is below
  p times that set's mass", evaluated by a double loop.
* Worked examples derived by hand (tests/golden/sampler_worked_examples.json).
* Log-softmax: closed forms and scipy's logsumexp.
* Gumbel-max: chi-square of sampled frequencies against the filtered softmax.
* RNG uniformity: Kolmogorov-Smirnov.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# -------------------------------------------------------------------- Philox
def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 3
    for ln in lines:
        v = [int(x, 16) for x in ln]
        out = oracle.philox4x32_10(*[np.array([x]) for x in v[:4]], v[4], v[5])
        assert [int(o[0]) for o in out] == v[6:10]


def test_uniform_range_and_ks():
    ids = np.arange(200_000)
    w = oracle.random_words(0x123456789ABCDEF, 7, ids)
    u = oracle.uniform_from_words(w)
    assert u.min() > 0.0 and u.max() < 1.0
    # 23-bit grid: u * 2^23 - 1/2 is an integer.
    g = u * 2.0**23 - 0.5
    assert np.all(g == np.round(g))
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-3


def test_rng_rows_and_seeds_independent():
    ids = np.arange(4096)
    a = oracle.random_words(1, 0, ids)
    b = oracle.random_words(1, 1, ids)
    c = oracle.random_words(2, 0, ids)
    d = oracle.random_words(1 << 32, 0, ids)   # high seed word matters
    e = oracle.random_words(1, 1 << 32, ids)   # high row word matters
    for x, y in [(a, b), (a, c), (a, d), (a, e)]:
        assert np.mean(x == y) < 0.01
    # Words of one counter block are distinct outputs of one Philox call.
    assert len(set(a[:4].tolist())) == 4


# RNG word layout (the contract of the sampler's noise): key = (seed low 32
# bits, seed high 32 bits), counter = (v >> 2, row low 32 bits, row high 32
# bits, 0), token v takes output word v & 3.  Each entry below spells the key
# and counter words out by hand (hex), so a swapped key half, a swapped row
# half, a counter word in the wrong slot or a wrong word index all change some
# expected word.  Seeds and rows set both 32-bit halves; v covers all four
# word slots and the counter's high bits.
#   (seed, global row, token v, key0, key1, ctr1, ctr2)
RNG_TABLE = [
    (0x0000000000000000, 0x0000000000000000, 0, 0x00000000, 0x00000000, 0x00000000, 0x00000000),
    (0x0000000000000000, 0x0000000000000000, 3, 0x00000000, 0x00000000, 0x00000000, 0x00000000),
    (0x0123456789ABCDEF, 0x0000000500000007, 13, 0x89ABCDEF, 0x01234567, 0x00000007, 0x00000005),
    (0x0123456789ABCDEF, 0x0000000500000007, 14, 0x89ABCDEF, 0x01234567, 0x00000007, 0x00000005),
    (0x0123456789ABCDEF, 0x0000000700000005, 13, 0x89ABCDEF, 0x01234567, 0x00000005, 0x00000007),
    (0x89ABCDEF01234567, 0x0000000500000007, 13, 0x01234567, 0x89ABCDEF, 0x00000007, 0x00000005),
    (0xFFFFFFFF00000001, 0x0000000100000000, 151935, 0x00000001, 0xFFFFFFFF, 0x00000000, 0x00000001),
    (0x00000001FFFFFFFF, 0x00000000FFFFFFFF, 151932, 0xFFFFFFFF, 0x00000001, 0xFFFFFFFF, 0x00000000),
    (0x9E3779B97F4A7C15, 0x0000000200000280, 262143, 0x7F4A7C15, 0x9E3779B9, 0x00000280, 0x00000002),
    (0x9E3779B97F4A7C15, 0x0000000200000280, 1, 0x7F4A7C15, 0x9E3779B9, 0x00000280, 0x00000002),
    (0x00000000DEADBEEF, 0x000000000000027F, 2147483646, 0xDEADBEEF, 0x00000000, 0x0000027F, 0x00000000),
    (0xCAFEF00D00000000, 0xFFFFFFFFFFFFFFFF, 7, 0x00000000, 0xCAFEF00D, 0xFFFFFFFF, 0xFFFFFFFF),
    (0x0000000000000001, 0x0000000000000001, 4, 0x00000001, 0x00000000, 0x00000001, 0x00000000),
    (0x0000000000000001, 0x0000000000000001, 5, 0x00000001, 0x00000000, 0x00000001, 0x00000000),
]


def _table_word(entry):
    """The expected word of one table entry: the known-answer-pinned Philox
    on the hand-written counter and key, output word v & 3."""
    _, _, v, key0, key1, ctr1, ctr2 = entry
    out = oracle.philox4x32_10(np.array([v >> 2]), np.array([ctr1]), np.array([ctr2]),
                               np.array([0]), key0, key1)
    return int(out[v & 3][0])


def test_rng_word_table_layout():
    slots = set()
    for entry in RNG_TABLE:
        seed, row, v, key0, key1, ctr1, ctr2 = entry
        # the hand-split words are the halves of seed and row
        assert (key1 << 32) | key0 == seed and (ctr2 << 32) | ctr1 == row, entry
        got = int(oracle.random_words(seed, row, np.array([v]))[0])
        assert got == _table_word(entry), entry
        slots.add(v & 3)
    assert slots == {0, 1, 2, 3}


def test_rng_word_table_discriminates_layouts():
    """The table is sensitive to the layout: the words a mis-wired generator
    would produce (key halves swapped, row halves swapped, word slot
    reversed) differ from the table on some entry."""
    def wrong(entry, how):
        seed, row, v, key0, key1, ctr1, ctr2 = entry
        if how == "key":
            key0, key1 = key1, key0
        elif how == "row":
            ctr1, ctr2 = ctr2, ctr1
        out = oracle.philox4x32_10(np.array([v >> 2]), np.array([ctr1]), np.array([ctr2]),
                                   np.array([0]), key0, key1)
        return int(out[(3 - (v & 3)) if how == "slot" else (v & 3)][0])
    for how in ("key", "row", "slot"):
        assert any(wrong(e, how) != _table_word(e) for e in RNG_TABLE), how


def test_uniform_endpoints_and_grid():
    """u = ((x >> 9) + 1/2) * 2^-23: the nine low bits are dropped, the
    smallest word gives 2^-24 and the largest 1 - 2^-24 (both exact)."""
    x = np.array([0, 0x1FF, 0x200, 0x3FF, 0x80000000, 0xFFFFFE00, 0xFFFFFFFF], dtype=np.uint64)
    u = oracle.uniform_from_words(x)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[2] == 3 * 2.0 ** -24 and u[3] == 3 * 2.0 ** -24
    assert u[4] == 0.5 + 2.0 ** -24
    assert u[5] == 1.0 - 2.0 ** -24 and u[6] == 1.0 - 2.0 ** -24
    # the Gumbel range these give
    g = -np.log(-np.log(u[[0, 6]]))
    assert abs(g[0] - (-math.log(24 * math.log(2)))) < 1e-12
    assert 16.63 < g[1] < 16.64


def _two_token_row_with_key_gap(gap, t=1.0, seed=0x5EED, row=3):
    """Logits of a two-token row whose Gumbel keys (l - m)/T + g differ by
    `gap` (token 0 ahead), from the noise written out by hand: g = -ln(-ln u)
    with u from the table-pinned word layout."""
    words = [_table_word((seed, row, v, seed & 0xFFFFFFFF, seed >> 32, row & 0xFFFFFFFF,
                          row >> 32)) for v in (0, 1)]
    u = [((w >> 9) + 0.5) * 2.0 ** -23 for w in words]
    g = [-math.log(-math.log(x)) for x in u]
    l1 = 0.0
    l0 = t * (gap + g[1] - g[0]) + l1
    return np.array([l0, l1], dtype=np.float64), t, seed, row


@pytest.mark.parametrize("scale,flag", [(0.5, True), (2.0, False), (-0.5, True), (-2.0, False)])
def test_tie_flag_window(scale, flag):
    """flag_tie marks a row exactly when its two best Gumbel keys lie closer
    than KEY_TIE_WINDOW: half the window apart is flagged, twice the window
    apart is not, whichever token leads."""
    gap = scale * oracle.KEY_TIE_WINDOW
    l, t, seed, row = _two_token_row_with_key_gap(gap)
    r = oracle.sample_row(l, t, 0, 1.0, 0, seed, row, 0)
    assert r.flag_tie == flag
    assert r.token == (0 if gap > 0 else 1)
    assert not r.flag_top_p


def test_tie_flag_needs_two_kept_tokens():
    """With top-k = 1 (greedy) or a one-token kept set there is no second key
    and no flag, however close the two keys are."""
    l, t, seed, row = _two_token_row_with_key_gap(0.1 * oracle.KEY_TIE_WINDOW)
    assert not oracle.sample_row(l, t, 1, 1.0, 0, seed, row, 0).flag_tie
    assert oracle.sample_row(l, t, 0, 1.0, 0, seed, row, 0).flag_tie
    # top-p keeping only the larger logit: one kept token, no flag
    big = np.array([8.0, 0.0])
    assert not oracle.sample_row(big, 1.0, 0, 0.5, 0, seed, row, 0).flag_tie


# ----------------------------------------------------------------- projection
def _bf16_fraction(bits: int) -> Fraction:
    """Exact value of a bf16 bit pattern, from the IEEE binary32 layout."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    assert exp != 0xFF
    if exp == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(man, 1 << 7)) * (Fraction(2) ** (exp - 127))


@pytest.mark.parametrize("rows,vocab,hidden", [(3, 5, 7), (2, 9, 16), (5, 4, 33)])
def test_projection_exact_rational(rows, vocab, hidden):
    rng = np.random.default_rng(rows * 100 + vocab)
    xb = workloads.bf16_bits_from_f32(rng.standard_normal((rows, hidden)).astype(np.float32))
    wb = workloads.bf16_bits_from_f32(
        (rng.standard_normal((vocab, hidden)) * 0.1).astype(np.float32))
    got = oracle.lmhead_logits(xb, wb, vocab_chunk=3)
    assert got.shape == (rows, vocab)
    for r in range(rows):
        for v in range(vocab):
            exact = sum(_bf16_fraction(int(xb[r, h])) * _bf16_fraction(int(wb[v, h]))
                        for h in range(hidden))
            bound = sum(abs(_bf16_fraction(int(xb[r, h])) * _bf16_fraction(int(wb[v, h])))
                        for h in range(hidden))
            assert abs(Fraction(got[r, v]) - exact) <= float(bound) * hidden * 2.0**-52 + 1e-300


def test_projection_one_hot_rows_reproduce_hidden_columns():
    rng = np.random.default_rng(5)
    hidden = 24
    xb = workloads.bf16_bits_from_f32(rng.standard_normal((6, hidden)).astype(np.float32))
    w = np.zeros((hidden, hidden), dtype=np.float32)
    perm = rng.permutation(hidden)
    w[np.arange(hidden), perm] = 1.0
    wb = workloads.bf16_bits_from_f32(w)
    got = oracle.lmhead_logits(xb, wb)
    np.testing.assert_array_equal(got, oracle.decode_bf16(xb)[:, perm])


def test_decode_bf16_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3E80, 0x7F7F, 0x0001], dtype=np.uint16)
    got = oracle.decode_bf16(bits)
    assert got[:5].tolist() == [1.0, -2.0, 0.0, -0.0, 0.25]
    assert got[5] == float(np.float32(3.3895313892515355e38))
    assert got[6] == 2.0**-133


def test_assemble_round_trip():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((7, 23)).astype(np.float32)
    parts = [a[:, :5], a[:, 5:6], a[:, 6:20], a[:, 20:]]
    np.testing.assert_array_equal(oracle.assemble_vocab_slices(parts), a)
    b = oracle.assemble_vocab_slices([np.full((2, 2), 1.0), np.full((2, 1), 2.0)])
    assert b.tolist() == [[1.0, 1.0, 2.0], [1.0, 1.0, 2.0]]


# --------------------------------------------------------- kept-set brute force
def _brute_top_k(l, k):
    """v kept iff fewer than k tokens have a strictly larger logit."""
    V = len(l)
    if k <= 0 or k >= V:
        return set(range(V))
    return {v for v in range(V) if sum(1 for u in range(V) if l[u] > l[v]) < k}


def _brute_top_p(l, t, k, p):
    """v kept iff v is in the top-k set and the temperature-scaled mass of the
    top-k tokens with a strictly larger logit is below p times the set's mass."""
    K = _brute_top_k(l, k)
    if p >= 1.0:
        return K
    m = max(l)
    w = {u: math.exp((l[u] - m) / t) for u in K}
    z = math.fsum(w.values())
    out = set()
    for v in K:
        above = math.fsum(w[u] for u in K if l[u] > l[v])
        if above < p * z:
            out.add(v)
    return out


def test_worked_examples_kept_sets():
    with open(os.path.join(GOLDEN, "sampler_worked_examples.json")) as f:
        cases = json.load(f)["kept"]
    for c in cases:
        l = np.array(c["logits"], dtype=np.float64)
        kept, _ = oracle.kept_set(l, c["T"], c["k"], c["p"])
        assert kept.tolist() == c["kept"], c
        assert sorted(_brute_top_p(list(l), c["T"], c["k"], c["p"])) == c["kept"], c


@pytest.mark.parametrize("seed", range(40))
def test_kept_set_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 40))
    # Coarse values force ties at the top-k and top-p boundaries.
    if seed % 2:
        l = rng.integers(-3, 4, size=V).astype(np.float64) * 0.5
    else:
        l = rng.standard_normal(V) * 2.0
    t = float(rng.uniform(0.2, 2.0))
    k = int(rng.choice([0, 1, 2, 3, V - 1, V, V + 3]))
    p = float(rng.choice([1.0, float(rng.uniform(0.05, 0.999))]))
    kept, _ = oracle.kept_set(l, t, k, p)
    assert set(kept.tolist()) == _brute_top_p(list(l), t, k, p)


def test_top_p_one_and_k_v_keep_everything():
    rng = np.random.default_rng(3)
    l = rng.standard_normal(100)
    for k in (0, 100, 1000):
        kept, amb = oracle.kept_set(l, 0.9, k, 1.0)
        assert kept.tolist() == list(range(100)) and amb.size == 0


@pytest.mark.parametrize("seed", range(12))
def test_ambiguous_set_is_the_shifted_boundaries(seed):
    """The ids near the top-p boundary are exactly those kept at p + window
    but not at p - window."""
    rng = np.random.default_rng(100 + seed)
    V = 5000
    l = rng.standard_normal(V) * 1.3
    t = float(rng.uniform(0.3, 1.5))
    k = int(rng.choice([0, 50, 1000]))
    p = float(rng.uniform(0.3, 0.99999))
    w = oracle.TOP_P_FLAG_WINDOW
    kept, amb = oracle.kept_set(l, t, k, p)
    small, _ = oracle.kept_set(l, t, k, p - w)
    big, _ = oracle.kept_set(l, t, k, min(1.0, p + w))
    assert set(amb.tolist()) == set(big.tolist()) - set(small.tolist())
    assert set(small.tolist()) <= set(kept.tolist()) <= set(big.tolist())


def test_top_p_flag_means_token_depends_on_boundary():
    """A row is flagged exactly when sampling with the boundary moved to
    p - window and to p + window draws different tokens."""
    rng = np.random.default_rng(7)
    V = 20000
    l = (rng.standard_normal(V) * 1.3).astype(np.float32)
    w = oracle.TOP_P_FLAG_WINDOW
    flagged = 0
    for row in range(150):
        p = float(rng.uniform(0.5, 0.95))
        r = oracle.sample_row(l, 1.0, 0, p, 0, 5, row, 0)
        lo = oracle.sample_row(l, 1.0, 0, p - w, 0, 5, row, 0).token
        hi = oracle.sample_row(l, 1.0, 0, p + w, 0, 5, row, 0).token
        assert r.flag_top_p == (lo != hi)
        assert r.token in (lo, hi) or r.flag_top_p
        flagged += r.flag_top_p
    assert flagged < 10   # a token rarely depends on a boundary this narrow


# ---------------------------------------------------------------- logprobs
def test_logprob_closed_forms():
    with open(os.path.join(GOLDEN, "sampler_worked_examples.json")) as f:
        cases = json.load(f)["logprobs"]
    for c in cases:
        l = np.array(c["logits"], dtype=np.float64)
        V = len(l)
        r = oracle.sample_row(l, 0.0, 0, 1.0, V, 0, 0, V)
        got = np.empty(V)
        got[r.topn_ids] = r.topn_logprobs
        np.testing.assert_allclose(got, c["logprobs"], rtol=1e-12, atol=1e-12)


def test_logprobs_match_scipy_and_topn_order():
    rng = np.random.default_rng(11)
    l = rng.standard_normal(3000).astype(np.float32)
    l[17] = l[18] = l.max() + 1          # tie at the top: lower id first
    r = oracle.sample_row(l, 0.8, 0, 1.0, 20, 9, 3, 20)
    ref = l.astype(np.float64) - scipy.special.logsumexp(l.astype(np.float64))
    assert r.topn_ids[0] == 17 and r.topn_ids[1] == 18
    np.testing.assert_allclose(r.topn_logprobs, ref[r.topn_ids], atol=1e-12)
    # Top-N are the 20 largest values in non-increasing order.
    vals = l[r.topn_ids]
    assert np.all(np.diff(vals) <= 0)
    assert vals[-1] >= np.sort(l)[-20]
    assert r.token_logprob == pytest.approx(ref[r.token], abs=1e-12)


def test_top_n_wider_than_vocabulary():
    """Asking for more log-probabilities than the row has tokens lists each
    token once (a 3-token row: ids by descending logit) and leaves the other
    slots unused."""
    l = np.array([0.5, 2.0, -1.0], dtype=np.float32)
    r = oracle.sample_row(l, 1.0, 0, 1.0, 6, 3, 0, 8)
    assert r.topn_ids.tolist() == [1, 0, 2, -1, -1, -1, -1, -1]
    assert np.all(np.isneginf(r.topn_logprobs[3:]))
    r1 = oracle.sample_row(np.array([4.0], dtype=np.float32), 0.7, 0, 1.0, 5, 3, 0, 5)
    assert r1.topn_ids.tolist() == [0, -1, -1, -1, -1] and r1.token == 0
    assert r1.topn_logprobs[0] == 0.0


def test_unused_slots_and_zero_logprobs():
    l = np.linspace(-1, 1, 50).astype(np.float32)
    r = oracle.sample_row(l, 1.0, 0, 1.0, 0, 1, 0, 6)
    assert r.topn_ids.tolist() == [-1] * 6
    assert np.all(np.isneginf(r.topn_logprobs))


# ------------------------------------------------------------------ greedy
def test_greedy_cases():
    rng = np.random.default_rng(2)
    l = rng.standard_normal(500).astype(np.float32)
    l[[40, 300]] = l.max() + 2.0   # tie for the maximum
    for t, k in [(0.0, 0), (0.0, 50), (5e-7, 0), (1.3, 1), (0.0, 1)]:
        r = oracle.sample_row(l, t, k, 0.5, 3, 77, 5, 3)
        assert r.token == 40
    # A small temperature with a wide gap is argmax for every seed.
    l2 = l.copy()
    l2[300] -= 1.0
    for s in range(50):
        assert oracle.sample_row(l2, 0.01, 0, 1.0, 0, s, 0, 0).token == 40


# ----------------------------------------------------------------- statuses
def test_row_status():
    l = np.zeros(8, dtype=np.float32)
    bad = [(-0.1, 0, 1.0, 1), (math.nan, 0, 1.0, 1), (math.inf, 0, 1.0, 1), (1.0, -1, 1.0, 1),
           (1.0, 0, 0.0, 1), (1.0, 0, 1.01, 1), (1.0, 0, math.nan, 1), (1.0, 0, 1.0, -1),
           (1.0, 0, 1.0, 5)]
    for t, k, p, n in bad:
        r = oracle.sample_row(l, t, k, p, n, 0, 0, 4)
        assert r.status == oracle.STATUS_BAD_PARAMS and r.token == -1
        assert math.isnan(r.token_logprob) and np.all(r.topn_ids == -1)
    for bad_val in (math.nan, math.inf):
        l2 = l.copy()
        l2[3] = bad_val
        assert oracle.sample_row(l2, 1.0, 0, 1.0, 1, 0, 0, 4).status == oracle.STATUS_BAD_LOGITS
    l3 = np.full(8, -np.inf, dtype=np.float32)
    assert oracle.sample_row(l3, 1.0, 0, 1.0, 1, 0, 0, 4).status == oracle.STATUS_BAD_LOGITS
    # -inf entries are allowed and never sampled.
    l4 = np.full(8, -np.inf, dtype=np.float32)
    l4[5] = 0.0
    l4[2] = -1.0
    r = oracle.sample_row(l4, 1.0, 0, 1.0, 4, 0, 0, 4)
    assert r.status == 0 and r.token in (2, 5)
    assert r.topn_ids.tolist() == [5, 2, 0, 1]


# ------------------------------------------------------------- Gumbel-max
@pytest.mark.parametrize("t,k,p", [(1.0, 0, 1.0), (0.6, 0, 0.8), (1.4, 4, 1.0), (0.9, 5, 0.7)])
def test_gumbel_max_frequencies_chi_square(t, k, p):
    l = np.array([1.2, 0.3, -0.4, 0.9, 0.0, -1.0, 0.5], dtype=np.float32)
    kept = sorted(_brute_top_p([float(x) for x in l], t, k, p))
    probs = scipy.special.softmax(l[kept].astype(np.float64) / t)
    draws = 12_000
    counts = {v: 0 for v in range(len(l))}
    for row in range(draws):
        counts[oracle.sample_row(l, t, k, p, 0, 1234, row, 0).token] += 1
    assert all(counts[v] == 0 for v in range(len(l)) if v not in kept)
    obs = np.array([counts[v] for v in kept])
    if len(kept) > 1:
        assert scipy.stats.chisquare(obs, probs * draws).pvalue > 1e-3
    else:
        assert obs[0] == draws


def test_rows_share_seed_but_differ():
    """Spec-decode rows of one request share a seed; the global row index
    separates their draws, and row_offset shifts it."""
    l = np.zeros((6, 64), dtype=np.float32)
    params = np.zeros(6, dtype=workloads.PARAMS_DTYPE)
    params["temperature"] = 1.0
    params["top_p"] = 1.0
    params["seed"] = 99
    a = oracle.sample(l, params, 0, 0)
    assert len(set(a.token_ids.tolist())) > 1
    b = oracle.sample(l[3:], params[3:], 3, 0)
    np.testing.assert_array_equal(a.token_ids[3:], b.token_ids)


def test_workload_params_in_domain():
    for w in workloads.WORKLOADS.values():
        p = workloads.make_params(w)
        assert p.shape == (w.rows,)
        for r in p:
            assert oracle.params_valid(float(r["temperature"]), int(r["top_k"]),
                                       float(r["top_p"]), int(r["n_logprobs"]), w.max_logprobs)


# ------------------------------------------------------------- FP8 (E4M3)
def test_e4m3_decode_matches_torch_and_the_format():
    """Every code against torch's float8_e4m3fn (a library decoding of the
    same OCP format), plus values fixed by the bit layout itself."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    d = oracle.decode_e4m3(codes)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])
    assert np.isnan(d).sum() == 2 and np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in fixed.items():
        assert d[c] == v, hex(c)
    assert np.signbit(d[0x80]) and d[0x80] == 0.0


def test_e4m3_encode_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3(oracle.decode_e4m3(codes)), codes)
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf])
    assert oracle.encode_e4m3(big).tolist() == [0x7E] * 6 + [0xFE] * 2
    assert oracle.encode_e4m3(np.array([np.nan]))[0] == 0x7F


def test_e4m3_encode_matches_torch_rounding():
    """Nearest code with ties to even, against torch's conversion, on random
    values, every exact midpoint between neighbouring codes, and the
    subnormal range (all inside +-448, where torch does not overflow)."""
    import torch

    rng = np.random.default_rng(5)
    pos = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000), rng.uniform(-2 ** -6, 2 ** -6, 5000),
        mids, -mids, pos, np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    got = oracle.encode_e4m3(vals.astype(np.float64))
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]


def _bf16_bits(x):
    x32 = np.asarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def test_e4m3_quantize_rows_definition():
    """Per-row amax scaling written out element by element in fp32, and the
    properties the scheme guarantees: the amax element lands on +-448, a zero
    row gets scale 1 and zero codes, and decoding reproduces the row within
    half an E4M3 step."""
    import struct

    rng = np.random.default_rng(9)
    x = rng.normal(0, 3, size=(6, 40)).astype(np.float32)
    x[2] = 0.0
    x[3, 5] = 1e-30
    x[4, :3] = [-7.0, 0.0, 7.0]
    bits = _bf16_bits(x)
    codes, scales = oracle.quantize_rows_e4m3(bits)
    xb = oracle.decode_bf16(bits)
    f32 = lambda v: struct.unpack("f", struct.pack("f", v))[0]  # noqa: E731
    for r in range(x.shape[0]):
        amax = max(abs(v) for v in xb[r])
        s = f32(f32(amax) / 448.0) if amax > 0 else 1.0
        assert scales[r] == np.float32(s)
        for h in range(x.shape[1]):
            q = f32(f32(xb[r, h]) / s)
            assert codes[r, h] == oracle.encode_e4m3(np.array([q]))[0]
        dec = oracle.decode_e4m3(codes[r]) * s
        if amax > 0:
            assert np.max(np.abs(oracle.decode_e4m3(codes[r]))) == 448.0
            rel = np.abs(dec - xb[r]) / np.maximum(np.abs(xb[r]), 2.0 ** -6 * s)
            assert rel.max() <= 2.0 ** -4 + 1e-12
    assert scales[2] == 1.0 and not codes[2].any()


def test_e4m3_quantize_rows_non_finite():
    """The scale follows amax = the largest |x| with NaN ignored: +inf makes it
    infinite (finite values then code as signed zeros, inf itself as NaN), a
    row of NaN gets scale 1 and NaN codes."""
    x = np.array([[np.inf, 5.0, -0.0, -3.0],
                  [np.nan, np.nan, np.nan, np.nan],
                  [np.nan, 2.0, -448.0, 0.5]], dtype=np.float32)
    codes, scales = oracle.quantize_rows_e4m3(_bf16_bits(x))
    assert np.isinf(scales[0]) and scales[1] == 1.0 and scales[2] == 1.0
    assert codes[0].tolist() == [0x7F, 0x00, 0x80, 0x80]
    assert codes[1].tolist() == [0x7F] * 4
    assert codes[2].tolist() == [0x7F, 0x40, 0xFE, 0x30]


def test_e4m3_projection_exact_on_integer_codes():
    """Codes whose values are small integers and power-of-two scales make every
    product and sum exact: the oracle must equal an integer matmul scaled by
    the two scales, element for element (a transposed operand or a dropped
    scale breaks it)."""
    rng = np.random.default_rng(13)
    ints = np.arange(-8, 9)
    enc = {int(v): int(oracle.encode_e4m3(np.array([float(v)]))[0]) for v in ints}
    xi = rng.integers(-8, 9, size=(5, 64))
    wi = rng.integers(-8, 9, size=(37, 64))
    xc = np.vectorize(enc.get)(xi).astype(np.uint8)
    wc = np.vectorize(enc.get)(wi).astype(np.uint8)
    xs = 2.0 ** rng.integers(-6, 3, size=5)
    ws = 2.0 ** rng.integers(-9, 1, size=37)
    got = oracle.lmhead_logits_e4m3(xc, xs.astype(np.float32), wc, ws.astype(np.float32),
                                    vocab_chunk=16)
    want = (xi @ wi.T).astype(np.float64) * xs[:, None] * ws[None, :]
    assert np.array_equal(got, want)


# --------------------------------------------------- processed log-probs (R11)
def _row(l, t, k, p, n, seed=3):
    return oracle.sample_row(np.asarray(l, dtype=np.float32), t, k, p, n, seed, 0, n,
                             processed=True)


def test_processed_logprobs_without_filters_are_log_softmax_of_scaled_logits():
    from scipy.special import log_softmax

    rng = np.random.default_rng(21)
    l = rng.normal(0, 2, 500).astype(np.float32)
    r = _row(l, 0.7, 0, 1.0, 8)
    ref = log_softmax(l.astype(np.float64) / 0.7)
    assert abs(r.token_logprob - ref[r.token]) < 1e-12
    np.testing.assert_allclose(r.topn_logprobs, ref[r.topn_ids], rtol=0, atol=1e-12)


def test_processed_logprobs_top_k_brute_force():
    rng = np.random.default_rng(22)
    l = rng.integers(-5, 6, 300).astype(np.float32)   # many ties at the k-th value
    k = 17
    r = _row(l, 1.0, k, 1.0, 40)
    kth = sorted(l.tolist(), reverse=True)[k - 1]
    kept = [i for i in range(l.shape[0]) if l[i] >= kth]
    z = sum(math.exp(float(l[i])) for i in kept)
    for i, lp in zip(r.topn_ids, r.topn_logprobs):
        want = float(l[i]) - math.log(z) if i in kept else -math.inf
        assert (lp == want) or abs(lp - want) < 1e-12, (i, lp, want)
    assert r.token in kept


def test_processed_logprobs_greedy_is_a_point_mass():
    l = np.array([1.0, 3.0, 3.0, 2.0], dtype=np.float32)
    r = _row(l, 0.0, 0, 1.0, 4)
    assert r.token == 1 and r.token_logprob == 0.0
    assert r.topn_ids.tolist() == [1, 2, 3, 0]
    assert r.topn_logprobs.tolist() == [0.0, -math.inf, -math.inf, -math.inf]


def test_processed_logprobs_top_p_sum_to_one_over_the_kept_set():
    rng = np.random.default_rng(23)
    l = rng.normal(0, 1.5, 2000).astype(np.float32)
    r = _row(l, 0.9, 0, 0.6, 2000)
    fin = np.isfinite(r.topn_logprobs)
    assert fin.sum() == r.kept and 0 < r.kept < 2000
    assert abs(np.exp(r.topn_logprobs[fin]).sum() - 1.0) < 1e-12
    # the listed ids are the raw top-N: the kept ones form its prefix
    assert fin[:r.kept].all() and not fin[r.kept:].any()
