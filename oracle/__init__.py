"""CPU oracle for the batch-sharded sampling hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``top_sampling_amd``); the two meet only through the seeded input
generators in ``workloads``.

It is the plain definition of what one tensor-parallel rank's share of
batch-sharded sampling computes, written for a reader to check by eye, in
float64 throughout:

* the local vocabulary projection -- each rank computes the logits of its own
  vocabulary slice and gathers nothing (page "Qwen4Exp batch-sharded sampling:
  inside vLLM PR #61018", orcarouter.ai blog, sections "What batch-sharded
  sampling is, in one paragraph" and "Why three lines were the whole job");
* the stitching of received vocabulary slices into the rank's batch slice
  (same page, "What batch-sharded sampling is, in one paragraph": the ranks
  swap vocabulary slices with an all-to-all);
* the per-row sampler over batch x (speculative tokens + 1) rows with
  temperature, top-k, top-p, log-probabilities and seeded sampling (same page
  and section; the page names top-k, top-p and a non-negative
  ``max_logprobs`` but not their arithmetic).

Readings taken where the page is silent (each one is listed with its reason
in the design notes of the repository):

  R1  order: temperature, then top-k, then top-p (top-p acts on the
      temperature-scaled distribution renormalised over the top-k set);
  R2  greedy when temperature < GREEDY_EPS or top_k == 1: argmax of the raw
      logits, lowest token id on ties;
  R3  top_k == 0 or top_k >= V: no top-k filter; top_p == 1: no top-p filter;
  R4  threshold semantics: every token tied with the k-th largest logit is
      kept; the token whose cumulative mass first reaches p is kept, and so
      is every token tied with it;
  R5  log-probabilities describe the raw distribution, log_softmax(logits),
      unscaled and unfiltered; top-N lists the N largest logits, ties by
      lower token id;
  R6  seeded sampling is Gumbel-max: token = argmax over the kept set of
      (l - m)/T + g, g = -ln(-ln u), u from Philox4x32-10 keyed on the row's
      seed and countered on (token id / 4, global row); lowest id on ties;
  R7  invalid parameters give row status 1, a NaN or +inf logit or a row
      with no finite logit gives row status 2; such rows return token -1 and
      NaN log-probabilities; unused top-N slots hold id -1, log-prob -inf;
  R10 the FP8 projection is W8A8 with per-row fp32 scales (see below);
  R11 on request, log-probabilities describe the distribution sampled from:
      (l - m)/T - ln(sum over the kept set of exp((l - m)/T)) for kept
      tokens, -inf for the others; a greedy row is a point mass (0 for the
      chosen token, -inf for the rest); top-N lists the same ids as R5.

Parity of every function here is pinned by tests in ``tests/test_oracle_pins.py``
(published Philox known-answer vectors, exact integer dot products, O(V^2)
brute force of top-k and top-p, closed-form log-softmax, chi-square of
Gumbel-max frequencies).
"""
from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

GREEDY_EPS = 1e-6          # R2: temperatures below this sample greedily
TOP_P_FLAG_WINDOW = 1e-5   # top-p boundaries whose mass lies this close to p are ambiguous
KEY_TIE_WINDOW = 1e-5      # rows whose two best Gumbel keys lie this close are flagged

STATUS_OK = 0
STATUS_BAD_PARAMS = 1
STATUS_BAD_LOGITS = 2


# ---------------------------------------------------------------- projection
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  A bf16 number is the upper half
    of an IEEE binary32 word, so widening is a 16-bit left shift."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def lmhead_logits(hidden_bits: np.ndarray, lm_head_bits: np.ndarray,
                  vocab_chunk: int = 8192) -> np.ndarray:
    """logits[r, v] = sum_h X[r, h] * W[v, h] in float64.

    ``hidden_bits`` is bf16 ``[rows, H]``, ``lm_head_bits`` is bf16 ``[V_local, H]``
    (the rank's own vocabulary slice).  The result covers only that slice: no
    gather.  The float64 matmul is the library step; it is chunked over V only
    to bound host memory.
    """
    x = decode_bf16(hidden_bits)
    rows, hidden = x.shape
    vocab = lm_head_bits.shape[0]
    assert lm_head_bits.shape[1] == hidden
    out = np.empty((rows, vocab), dtype=np.float64)
    for v0 in range(0, vocab, vocab_chunk):
        w = decode_bf16(lm_head_bits[v0:v0 + vocab_chunk])
        out[:, v0:v0 + w.shape[0]] = x @ w.T
    return out


# -------------------------------------------------------- FP8 projection
# The pages' measured deployment is an FP8 checkpoint and their patch cluster
# includes a kernel that unpacks e4m3 bytes (page "Qwen4Exp batch-sharded
# sampling: inside vLLM PR #61018", sections "The 1.5% estimate, and the
# measurement next to it" and "The patch cluster"); they state no scaling
# scheme.  Reading R10: W8A8 with one fp32 scale per row on both operands --
# every lm_head row and every hidden-state row is stored as OCP E4M3 codes
# times its own scale amax / 448, and the projection sums the products of the
# decoded codes and applies both scales.
E4M3_MAX = 448.0


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 (the variant without infinities) ->
    float64: one sign bit, four exponent bits with bias 7, three mantissa
    bits.  Exponent field 0 holds subnormals m/8 * 2^-6; the two all-ones
    patterns (S.1111.111) are NaN; the largest magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


_E4M3_POS = decode_e4m3(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7E, increasing


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """The E4M3 code nearest to each value; halfway cases go to the code with
    an even mantissa; magnitudes of 448 and above (infinities included)
    saturate to 448; NaN gives 0x7F.  The sign bit is the input's, so -0.0
    gives 0x80."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = np.abs(a - _E4M3_POS[lo])
    d_hi = np.abs(_E4M3_POS[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= E4M3_MAX, 0x7E, pick)
    code = pick.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_rows_e4m3(bits: np.ndarray):
    """bf16 ``[rows, cols]`` -> (E4M3 codes ``[rows, cols]``, fp32 scales ``[rows]``).

    Per row: amax = the largest |x| (NaN ignored), scale = amax / 448 in fp32
    (1 for a row of zeros), code = encode_e4m3(x / scale) with the division in
    fp32.  The codes are decided in fp32 because the kernel divides in fp32; a
    float64 quotient could round to a different code."""
    import warnings

    x32 = decode_bf16(bits).astype(np.float32)
    with np.errstate(invalid="ignore"), warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)  # a row of NaN: amax NaN -> 0 below
        amax = np.nanmax(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    amax = np.where(np.isnan(amax), np.float32(0.0), amax).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = (x32 / scale[:, None]).astype(np.float32)
    return encode_e4m3(q.astype(np.float64)), scale


def lmhead_logits_e4m3(hidden_codes: np.ndarray, hidden_scales: np.ndarray,
                       lm_head_codes: np.ndarray, lm_head_scales: np.ndarray,
                       vocab_chunk: int = 8192) -> np.ndarray:
    """logits[r, v] = s_x[r] * s_w[v] * sum_h dec(X[r, h]) * dec(W[v, h]) in
    float64, over the rank's own vocabulary slice (no gather)."""
    x = decode_e4m3(hidden_codes)
    xs = np.asarray(hidden_scales, dtype=np.float64)
    vocab = lm_head_codes.shape[0]
    assert lm_head_codes.shape[1] == x.shape[1]
    out = np.empty((x.shape[0], vocab), dtype=np.float64)
    for v0 in range(0, vocab, vocab_chunk):
        w = decode_e4m3(lm_head_codes[v0:v0 + vocab_chunk])
        ws = np.asarray(lm_head_scales[v0:v0 + vocab_chunk], dtype=np.float64)
        out[:, v0:v0 + w.shape[0]] = (x @ w.T) * xs[:, None] * ws[None, :]
    return out


def assemble_vocab_slices(slices: list[np.ndarray]) -> np.ndarray:
    """The rank's batch slice ``[rows, sum cols_s]``: slice s occupies columns
    [off_s, off_s + cols_s) with off_s = sum of the earlier slices' widths."""
    rows = slices[0].shape[0]
    total = sum(s.shape[1] for s in slices)
    out = np.empty((rows, total), dtype=slices[0].dtype)
    off = 0
    for s in slices:
        assert s.shape[0] == rows
        out[:, off:off + s.shape[1]] = s
        off += s.shape[1]
    return out


# ---------------------------------------------------------------------- RNG
# Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
# as 1, 2, 3" (SC'11).  Four 32-bit counter words, two 32-bit key words; each
# round multiplies counter words 0 and 2 by fixed odd constants, and the key
# is bumped by Weyl increments between rounds.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised Philox4x32-10 over arrays of counters; returns 4 uint64
    arrays holding the 32-bit output words."""
    m = np.uint64(_MASK32)
    c = [np.asarray(v, dtype=np.uint64) & m for v in (c0, c1, c2, c3)]
    key0 = np.uint64(k0 & _MASK32)
    key1 = np.uint64(k1 & _MASK32)
    for rnd in range(10):
        if rnd > 0:
            key0 = (key0 + np.uint64(PHILOX_W0)) & m
            key1 = (key1 + np.uint64(PHILOX_W1)) & m
        p0 = np.uint64(PHILOX_M0) * c[0]
        p1 = np.uint64(PHILOX_M1) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ key0) & m,
             p1 & m,
             ((p0 >> np.uint64(32)) ^ c[3] ^ key1) & m,
             p0 & m]
    return c


def random_words(seed: int, row: int, ids: np.ndarray) -> np.ndarray:
    """The 32-bit word drawn for token ``ids`` of global row ``row``.

    key = (seed low 32 bits, seed high 32 bits);
    counter = (id >> 2, row low 32 bits, row high 32 bits, 0);
    the id's word is output word (id & 3) of that counter.
    """
    ids = np.asarray(ids, dtype=np.int64)
    seed = int(seed) & ((1 << 64) - 1)
    row = int(row) & ((1 << 64) - 1)
    n = ids.shape[0]
    words = philox4x32_10(ids >> 2, np.full(n, row & _MASK32), np.full(n, row >> 32),
                          np.zeros(n), seed & _MASK32, seed >> 32)
    stacked = np.stack(words)                       # [4, n]
    return stacked[ids & 3, np.arange(n)]


def uniform_from_words(words: np.ndarray) -> np.ndarray:
    """u = ((x >> 9) + 1/2) * 2^-23: 23 random bits, strictly inside (0, 1)."""
    return ((np.asarray(words, dtype=np.uint64) >> np.uint64(9)).astype(np.float64) + 0.5) \
        * 2.0 ** -23


def gumbel_noise(seed: int, row: int, ids: np.ndarray) -> np.ndarray:
    """Standard Gumbel noise g = -ln(-ln u) for the given tokens of one row."""
    u = uniform_from_words(random_words(seed, row, ids))
    return -np.log(-np.log(u))


# ------------------------------------------------------------------ sampler
@dataclasses.dataclass
class RowResult:
    status: int
    token: int
    token_logprob: float
    topn_ids: np.ndarray
    topn_logprobs: np.ndarray
    flag_top_p: bool = False   # token depends on a top-p boundary within TOP_P_FLAG_WINDOW
    flag_tie: bool = False     # two best Gumbel keys within KEY_TIE_WINDOW
    kept: int = 0              # size of the kept set (diagnostic)


def params_valid(t: float, k: int, p: float, n: int, max_logprobs: int) -> bool:
    """R7: the parameter domain."""
    if not math.isfinite(t) or t < 0.0:
        return False
    if k < 0:
        return False
    if not (p > 0.0 and p <= 1.0):   # also false for NaN
        return False
    if n < 0 or n > max_logprobs:
        return False
    return True


def kept_set(l: np.ndarray, t: float, k: int, p: float,
             order: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Token ids (ascending) that survive top-k then top-p at temperature t > 0,
    and the ids whose membership is within rounding of the top-p boundary.

    ``l`` is the float64 row; ``order`` its sort by (logit desc, id asc).
    The second array lists the top-k tokens that some boundary drawn where
    the cumulative mass lies within TOP_P_FLAG_WINDOW of p would add to or
    drop from the smallest such kept set (empty without a top-p filter).
    """
    vocab = l.shape[0]
    if order is None:
        order = np.lexsort((np.arange(vocab), -l))
    m = l[order[0]]
    # R1/R3/R4 top-k: keep every token whose logit is >= the k-th largest.
    if 0 < k < vocab:
        t_k = l[order[k - 1]]
        in_k = l >= t_k
    else:
        in_k = np.ones(vocab, dtype=bool)

    # Temperature-scaled weights over the top-k set, walked in sorted order.
    sorted_ids = order[in_k[order]]
    w = np.exp((l[sorted_ids] - m) / t)
    cum = np.cumsum(w)
    z_k = cum[-1]
    if p >= 1.0:
        return np.sort(sorted_ids), np.zeros(0, dtype=np.int64)
    # Smallest prefix whose mass reaches p; the crossing token is kept, and so
    # is every token tied with it.
    frac = cum / z_k
    j_star = int(np.argmax(frac >= p))
    t_p = l[sorted_ids[j_star]]
    kept = np.sort(sorted_ids[l[sorted_ids] >= t_p])
    # Boundaries drawn where the cumulative mass is within the window of p.
    last = frac.shape[0] - 1
    j_lo = int(np.argmax(frac >= p - TOP_P_FLAG_WINDOW))
    j_hi = int(np.argmax(frac >= p + TOP_P_FLAG_WINDOW)) if frac[-1] >= p + TOP_P_FLAG_WINDOW \
        else last
    t_lo, t_hi = l[sorted_ids[j_lo]], l[sorted_ids[j_hi]]
    vals = l[sorted_ids]
    ambiguous = np.sort(sorted_ids[(vals >= t_hi) & (vals < t_lo)])
    return kept, ambiguous


def sample_row(logits: np.ndarray, temperature: float, top_k: int, top_p: float,
               n_logprobs: int, seed: int, row_global: int, max_logprobs: int,
               processed: bool = False) -> RowResult:
    """Sample one row; ``logits`` is the fp32 row, used as exact values.
    Parameters are taken as given (the callers pass the fp32 values the GPU
    receives).  ``processed`` selects R11's log-probabilities of the
    distribution sampled from instead of R5's raw ones."""
    t = float(temperature)
    p = float(top_p)
    k = int(top_k)
    n = int(n_logprobs)
    vocab = logits.shape[0]
    bad_ids = np.full(max_logprobs, -1, dtype=np.int64)
    bad_lp = np.full(max_logprobs, np.nan)

    if not params_valid(t, k, p, n, max_logprobs):
        return RowResult(STATUS_BAD_PARAMS, -1, math.nan, bad_ids, bad_lp)
    l = np.asarray(logits, dtype=np.float64)
    if np.isnan(l).any() or np.isposinf(l).any() or not np.isfinite(l).any():
        return RowResult(STATUS_BAD_LOGITS, -1, math.nan, bad_ids, bad_lp)

    ids = np.arange(vocab)
    # R5: raw log-softmax.
    m = l.max()
    lse = m + math.log(np.exp(l - m).sum())
    logprob = l - lse
    # Full sort: logit descending, token id ascending.
    order = np.lexsort((ids, -l))
    topn_ids = np.full(max_logprobs, -1, dtype=np.int64)
    topn_lp = np.full(max_logprobs, -np.inf)
    n_listed = min(n, vocab)               # a row has only V tokens to list
    topn_ids[:n_listed] = order[:n_listed]
    topn_lp[:n_listed] = logprob[order[:n_listed]]

    # R2: greedy.
    if t < GREEDY_EPS or k == 1:
        tok = int(order[0])
        if processed:  # R11: a point mass on the chosen token
            topn_lp[:n_listed] = np.where(topn_ids[:n_listed] == tok, 0.0, -np.inf)
            return RowResult(STATUS_OK, tok, 0.0, topn_ids, topn_lp, kept=1)
        return RowResult(STATUS_OK, tok, float(logprob[tok]), topn_ids, topn_lp, kept=1)

    kept_ids, ambiguous = kept_set(l, t, k, p, order)
    if processed:
        # R11: log-probabilities of the temperature-scaled distribution
        # renormalised over the kept set; -inf outside it.
        z_kept = np.exp((l[kept_ids] - m) / t).sum()
        logprob = np.full(vocab, -np.inf)
        logprob[kept_ids] = (l[kept_ids] - m) / t - math.log(z_kept)
        topn_lp[:n_listed] = logprob[order[:n_listed]]

    # R6: Gumbel-max over the kept set.
    keys = (l[kept_ids] - m) / t + gumbel_noise(seed, row_global, kept_ids)
    best = int(np.argmax(keys))             # first maximum: lowest id
    tok = int(kept_ids[best])
    flag_tie = False
    if keys.shape[0] > 1:
        top2 = np.partition(keys, -2)[-2:]
        flag_tie = bool(abs(top2[1] - top2[0]) < KEY_TIE_WINDOW)
    # Flag the row when moving the top-p boundary within the window changes
    # the winner: the winners over the smallest and the largest plausible
    # kept sets differ.
    flag_top_p = False
    if ambiguous.shape[0]:
        amb = np.isin(kept_ids, ambiguous)
        small = kept_ids[~amb]
        k_small = keys[~amb]
        w_small = int(small[int(np.argmax(k_small))])
        extra = ambiguous[~np.isin(ambiguous, kept_ids)]
        big = np.concatenate([kept_ids, extra])
        k_big = np.concatenate([keys, (l[extra] - m) / t + gumbel_noise(seed, row_global, extra)])
        ob = np.lexsort((big, -k_big))
        flag_top_p = int(big[ob[0]]) != w_small
    return RowResult(STATUS_OK, tok, float(logprob[tok]), topn_ids, topn_lp,
                     flag_top_p=flag_top_p, flag_tie=flag_tie, kept=int(kept_ids.shape[0]))


@dataclasses.dataclass
class SampleResult:
    token_ids: np.ndarray        # int64 [rows]
    token_logprobs: np.ndarray   # float64 [rows]
    topn_ids: np.ndarray         # int64 [rows, max_logprobs]
    topn_logprobs: np.ndarray    # float64 [rows, max_logprobs]
    row_status: np.ndarray       # int32 [rows]
    flag_top_p: np.ndarray       # bool [rows]
    flag_tie: np.ndarray         # bool [rows]
    kept: np.ndarray             # int64 [rows]

    @property
    def flagged(self) -> np.ndarray:
        return self.flag_top_p | self.flag_tie


def _sample_rows(args):
    logits, params, row_offset, max_logprobs, row_ids, processed = args
    out = []
    for i, r in enumerate(row_ids):
        pr = params[i]
        out.append(sample_row(logits[i], float(pr["temperature"]), int(pr["top_k"]),
                              float(pr["top_p"]), int(pr["n_logprobs"]), int(pr["seed"]),
                              row_offset + int(r), max_logprobs, processed))
    return out


def sample(logits: np.ndarray, params: np.ndarray, row_offset: int, max_logprobs: int,
           rows: np.ndarray | None = None, workers: int = 1,
           processed: bool = False) -> SampleResult:
    """Sample every row (or the listed local ``rows``) of ``logits``.

    ``params`` is a record array with fields temperature, top_k, top_p,
    n_logprobs, seed (one entry per local row); ``row_offset`` is the global
    index of local row 0 (the RNG is keyed on the global row); ``processed``
    selects R11's log-probabilities.
    """
    logits = np.asarray(logits)
    row_ids = np.arange(logits.shape[0]) if rows is None else np.asarray(rows)
    if workers > 1 and row_ids.shape[0] > 1:
        import multiprocessing as mp

        parts = np.array_split(row_ids, min(workers, row_ids.shape[0]))
        jobs = [(logits[pr], params[pr], row_offset, max_logprobs, pr, processed)
                for pr in parts if len(pr)]
        with mp.get_context("fork").Pool(len(jobs)) as pool:
            res = [r for part in pool.map(_sample_rows, jobs) for r in part]
    else:
        res = _sample_rows((logits[row_ids], params[row_ids], row_offset, max_logprobs, row_ids,
                            processed))
    return SampleResult(
        token_ids=np.array([r.token for r in res], dtype=np.int64),
        token_logprobs=np.array([r.token_logprob for r in res]),
        topn_ids=np.stack([r.topn_ids for r in res]) if res else np.zeros((0, max_logprobs), np.int64),
        topn_logprobs=np.stack([r.topn_logprobs for r in res]) if res else np.zeros((0, max_logprobs)),
        row_status=np.array([r.status for r in res], dtype=np.int32),
        flag_top_p=np.array([r.flag_top_p for r in res], dtype=bool),
        flag_tie=np.array([r.flag_tie for r in res], dtype=bool),
        kept=np.array([r.kept for r in res], dtype=np.int64),
    )


def default_workers() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))
