"""Seeded synthetic inputs for the sampling workloads.

This module is the only code shared by the CPU oracle (``oracle/``) and the
GPU path (``top_sampling_amd``).  It draws inputs and nothing else: it holds no
part of the projection, the sampler or the slice assembly.

Workload shapes follow the batch-sharded sampling setting described on the
page "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018" (orcarouter.ai
blog, ja/nl/fr editions), section "What batch-sharded sampling is, in one
paragraph": the sampler sees batch x (speculative tokens + 1) rows, and each
tensor-parallel rank projects onto its own vocabulary slice.

Input recipe (one numpy ``PCG64`` / torch generator per workload, seeded by the
workload's index):
  * hidden states and lm_head weights are drawn from N(0, sigma) in fp32 and
    rounded once to bf16 (round to nearest even);
  * sampler-only logits are drawn directly in fp32: N(0, sqrt(H) * sigma_w),
    the distribution of the projection's output for these weights, or
    Gumbel(0, 1) with spike tokens for the rank-share workload;
  * per-row sampling parameters are drawn as each workload describes.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Byte layout of one row's sampling parameters; it mirrors ``ts_row_params``
# in include/top_sampling.h (24 bytes, 8-byte aligned).
PARAMS_DTYPE = np.dtype(
    [
        ("temperature", "<f4"),
        ("top_k", "<i4"),
        ("top_p", "<f4"),
        ("n_logprobs", "<i4"),
        ("seed", "<u8"),
    ],
    align=True,
)
assert PARAMS_DTYPE.itemsize == 24


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int  # seed of every generator drawn for this workload
    rows: int
    vocab: int
    hidden: int | None  # None: sampler-only workload (no projection)
    x_std: float = 1.0
    w_std: float = 0.0
    max_logprobs: int = 20
    n_slices: int = 1  # vocab slices the rank receives (assembly step)
    requests: int | None = None
    spec_tokens: int = 0
    description: str = ""
    # A rank's share of another workload: rows [row_offset, row_offset + rows)
    # of `parent`, with the parent's logits and parameters.
    parent: str | None = None
    row_offset: int = 0
    # The projection runs in FP8: bf16 draws quantized per row to OCP E4M3
    # codes with fp32 scales (lm_head once, hidden states every step).
    fp8: bool = False

    @property
    def logit_std(self) -> float:
        """Standard deviation of one projected logit: sqrt(H) * sigma_x * sigma_w."""
        if self.parent:
            return WORKLOADS[self.parent].logit_std
        return math.sqrt(self.hidden) * self.x_std * self.w_std if self.hidden else 1.0

    @property
    def slice_cols(self) -> list[int]:
        base, rem = divmod(self.vocab, self.n_slices)
        return [base + (1 if s < rem else 0) for s in range(self.n_slices)]


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            "tiny", 0, rows=4, vocab=4096, hidden=256, x_std=1.0, w_std=0.05, max_logprobs=5,
            description="4 rows, H=256, V=4096; fp32 draws rounded to bf16; "
            "rows: greedy, (0.7,50,1.0), (1.0,0,0.9), (0.7,20,0.8); 5 logprobs; seed 0",
        ),
        Workload(
            "decode", 1, rows=64, vocab=151936, hidden=4096, x_std=1.0, w_std=0.02, max_logprobs=5,
            description="64 rows, H=4096, V=151936 bf16; all rows T=0.7, k=20, p=0.8; 5 logprobs",
        ),
        Workload(
            "spec_decode", 2, rows=640, vocab=151936, hidden=4096, x_std=1.0, w_std=0.02,
            max_logprobs=20, requests=128, spec_tokens=4,
            description="128 requests x (4 draft + 1) = 640 rows, H=4096, V=151936 bf16; "
            "per-request T~U[0,1.2], k in {0,1,20,50,1000}, p~U[0.5,1], 0-20 logprobs",
        ),
        Workload(
            "rank_share", 3, rows=256, vocab=151936, hidden=None, max_logprobs=5, n_slices=4,
            description="4 fp32 vocab slices of 256 x 37984 assembled into 256 x 151936; "
            "Gumbel logits, 1% of rows with a +15 spike; mixed k/p per row",
        ),
        Workload(
            "large", 4, rows=1024, vocab=262144, hidden=8192, x_std=1.0, w_std=0.015,
            max_logprobs=20,
            description="1024 rows, H=8192, V=262144 bf16; quarters: greedy / p=0.95 / "
            "k=5 at T=1.5 / full vocabulary; 20 logprobs",
        ),
        # The drafter's logits (page "Qwen4Exp batch-sharded sampling: inside
        # vLLM PR #61018", section "What batch-sharded sampling is, in one
        # paragraph": sharded draft logits are named as future work; the MTP
        # drafter's logits path is flagged unverified): one draft position per
        # request, the full vocabulary, the target's lm_head shape.
        Workload(
            "draft", 5, rows=128, vocab=151936, hidden=4096, x_std=1.0, w_std=0.02,
            max_logprobs=0, requests=128,
            description="draft step: 128 requests x 1 draft row, H=4096, V=151936 bf16; "
            "per-request T~U[0,1.2], k in {0,1,20,50,1000}, p~U[0.5,1]; no top-N logprobs",
        ),
        # The pages' model shape with its FP8 checkpoint (page "Qwen4Exp
        # batch-sharded sampling: inside vLLM PR #61018", sections "The patch
        # cluster" -- vocabulary 248,320, hidden size 2,560 -- and "The 1.5%
        # estimate, and the measurement next to it" -- FP8 weights, tensor
        # parallelism 8): the spec-decode batch, eight vocabulary slices of
        # 31,040.
        Workload(
            "fp8", 6, rows=640, vocab=248320, hidden=2560, x_std=1.0, w_std=0.02,
            max_logprobs=20, n_slices=8, requests=128, spec_tokens=4, fp8=True,
            description="128 requests x (4 draft + 1) = 640 rows, H=2560, V=248320 "
            "(8 slices of 31040); bf16 N(0,1) hidden and N(0,0.02) lm_head quantized per row "
            "to E4M3 with fp32 scales; per-request params as spec_decode",
        ),
        Workload(
            "draft_share", 5, rows=16, vocab=151936, hidden=None, max_logprobs=0, n_slices=8,
            parent="draft", row_offset=48,
            description="sharded draft logits, tp=8: rank 3's 16 draft rows (48-63 of the "
            "draft step) received as 8 vocab slices of 18992, sampled with row_offset 48",
        ),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([w.index, stream]))


# ---------------------------------------------------------------- parameters
def make_params(w: Workload) -> np.ndarray:
    """Per-row sampling parameters as a ``PARAMS_DTYPE`` record array."""
    if w.parent:
        return make_params(WORKLOADS[w.parent])[w.row_offset:w.row_offset + w.rows].copy()
    p = np.zeros(w.rows, dtype=PARAMS_DTYPE)
    g = _rng(w, 1)
    if w.name == "tiny":
        rows = [(0.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9), (0.7, 20, 0.8)]
        for r, (t, k, pp) in enumerate(rows):
            p[r] = (t, k, pp, 5, 0)
    elif w.name == "decode":
        p["temperature"] = 0.7
        p["top_k"] = 20
        p["top_p"] = 0.8
        p["n_logprobs"] = 5
        p["seed"] = g.integers(0, 2**64, size=w.rows, dtype=np.uint64)
    elif w.name in ("spec_decode", "rank_share", "draft", "fp8"):
        n_req = w.requests if w.requests else w.rows
        per = w.rows // n_req
        t = g.uniform(0.0, 1.2, size=n_req).astype(np.float32)
        k = g.choice(np.array([0, 1, 20, 50, 1000], dtype=np.int32), size=n_req)
        pp = g.uniform(0.5, 1.0, size=n_req).astype(np.float32)
        nl = (g.integers(0, 21, size=n_req) if w.name in ("spec_decode", "fp8")
              else np.full(n_req, min(5, w.max_logprobs))).astype(np.int32)
        sd = g.integers(0, 2**64, size=n_req, dtype=np.uint64)
        for name, v in (("temperature", t), ("top_k", k), ("top_p", pp),
                        ("n_logprobs", nl), ("seed", sd)):
            p[name] = np.repeat(v, per)
    elif w.name == "large":
        q = w.rows // 4
        quarters = [(0.0, 0, 1.0), (1.0, 0, 0.95), (1.5, 5, 1.0), (1.0, 0, 1.0)]
        for i, (t, k, pp) in enumerate(quarters):
            sl = slice(i * q, (i + 1) * q)
            p["temperature"][sl] = t
            p["top_k"][sl] = k
            p["top_p"][sl] = pp
        p["n_logprobs"] = 20
        p["seed"] = g.integers(0, 2**64, size=w.rows, dtype=np.uint64)
    else:
        raise KeyError(w.name)
    return p


# ------------------------------------------------------------ sampler logits
def make_logits(w: Workload, rows: slice | None = None) -> np.ndarray:
    """fp32 sampler input ``[rows, vocab]``.

    Projection workloads: N(0, sqrt(H) * sigma_w) (the projection's output
    distribution).  Rank-share workload: Gumbel(0, 1) with one spike token
    (+15) in ceil(1% of rows) rows.  Rows are drawn from per-row streams, so a
    row range gives the same values as slicing the whole array.
    """
    if w.parent:
        rr = range(w.rows)[rows] if rows is not None else range(w.rows)
        ro = w.row_offset
        return make_logits(WORKLOADS[w.parent], slice(ro + rr.start, ro + rr.stop, rr.step))
    rr = range(w.rows)[rows] if rows is not None else range(w.rows)
    out = np.empty((len(rr), w.vocab), dtype=np.float32)
    for i, r in enumerate(rr):
        g = np.random.Generator(np.random.PCG64([w.index, 2, r]))
        if w.name == "rank_share":
            out[i] = g.gumbel(0.0, 1.0, size=w.vocab).astype(np.float32)
        else:
            out[i] = (g.standard_normal(w.vocab) * w.logit_std).astype(np.float32)
    if w.name == "rank_share":
        spikes = spike_rows(w)
        for i, r in enumerate(rr):
            if r in spikes:
                out[i, spikes[r]] += np.float32(15.0)
    return out


def spike_rows(w: Workload) -> dict[int, int]:
    """Rank-share workload: {row: spiked token} for ceil(1% of rows) rows."""
    g = _rng(w, 3)
    n = math.ceil(0.01 * w.rows)
    rows = g.choice(w.rows, size=n, replace=False)
    toks = g.integers(0, w.vocab, size=n)
    return {int(r): int(t) for r, t in zip(rows, toks)}


# --------------------------------------------------- projection inputs (bf16)
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_projection_host(w: Workload, rows: int | None = None, vocab: int | None = None,
                         hidden: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Host-drawn bf16 bits (uint16) of hidden ``[rows, H]`` and lm_head ``[V, H]``.

    For workloads small enough to draw on the host (the tiny workload, and
    reduced shapes used by tests).
    """
    rows = rows or w.rows
    vocab = vocab or w.vocab
    hidden = hidden or w.hidden
    g = _rng(w, 4)
    x = g.standard_normal((rows, hidden), dtype=np.float32) * np.float32(w.x_std)
    wt = g.standard_normal((vocab, hidden), dtype=np.float32) * np.float32(w.w_std)
    return bf16_bits_from_f32(x), bf16_bits_from_f32(wt)


def make_projection_device(w: Workload, device, rows: int | None = None,
                           vocab: int | None = None, hidden: int | None = None):
    """Device-drawn bf16 tensors (hidden ``[rows, H]``, lm_head ``[V, H]``).

    Drawn with a seeded torch generator on ``device`` in fp32 slabs and
    rounded to bf16; used for the full-size workloads.
    """
    import torch

    rows = rows or w.rows
    vocab = vocab or w.vocab
    hidden = hidden or w.hidden
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + w.index)
    x = (torch.randn(rows, hidden, generator=gen, device=device) * w.x_std).to(torch.bfloat16)
    wt = torch.empty(vocab, hidden, dtype=torch.bfloat16, device=device)
    slab = max(1, (1 << 26) // hidden)
    for v0 in range(0, vocab, slab):
        v1 = min(vocab, v0 + slab)
        wt[v0:v1] = (torch.randn(v1 - v0, hidden, generator=gen, device=device) * w.w_std).to(
            torch.bfloat16)
    return x, wt


def random_params(rng: np.random.Generator, rows: int, vocab: int, max_logprobs: int,
                  greedy_frac: float = 0.1) -> np.ndarray:
    """Mixed parameters for edge-case tests: every filter combination appears."""
    p = np.zeros(rows, dtype=PARAMS_DTYPE)
    t = rng.uniform(0.05, 1.5, size=rows).astype(np.float32)
    t[rng.random(rows) < greedy_frac] = 0.0
    kchoices = np.array([0, 1, 2, 5, 20, 50, 1000, vocab, vocab + 7], dtype=np.int64)
    k = np.minimum(rng.choice(kchoices, size=rows), 2**31 - 1).astype(np.int32)
    pp = rng.uniform(0.3, 1.0, size=rows).astype(np.float32)
    pp[rng.random(rows) < 0.3] = 1.0
    p["temperature"] = t
    p["top_k"] = k
    p["top_p"] = pp
    p["n_logprobs"] = rng.integers(0, max_logprobs + 1, size=rows)
    p["seed"] = rng.integers(0, 2**64, size=rows, dtype=np.uint64)
    return p
