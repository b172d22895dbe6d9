"""Python binding of ``libtopsampling.so`` (MI355X / gfx950).

Argument marshalling only: every step of the sampling path runs in the HIP
kernels behind the C ABI (``include/top_sampling.h``).  PyTorch supplies device
memory and the current stream.  Importing this package fails if the library is
not built (``python top_sampling_amd/build.py``); there is no fallback.

Calls mirror the C entry points:
  lmhead_logits_local            local vocabulary projection, bf16 -> fp32
  quantize_rows_e4m3             per-row FP8 (E4M3) quantization of bf16 rows
  lmhead_logits_local_e4m3       the same projection from FP8 codes and scales
  sampler_assemble_vocab_slices  stitch received vocabulary slices
  sampler_sample                 per-row temperature / top-k / top-p /
                                 logprobs / Gumbel-max sampling
  sampler_sample_slices          the same, reading the received vocabulary
                                 slices in place (no stitched buffer)
  sampler_sample_ex              slices plus flags (processed log-probabilities)
  sampler_workspace_bytes(_slices)  workspace size queries
and ``compute_logits_local`` returns the rank's own ``[rows, V_local]`` slice,
the local-logits hook of batch-sharded sampling (page "Qwen4Exp batch-sharded
sampling: inside vLLM PR #61018", section "Why three lines were the whole
job").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtopsampling.so")

TS_OK, TS_EINVAL, TS_EUNSUPPORTED, TS_EWORKSPACE, TS_EHIP = 0, -1, -2, -3, -4
TS_ROW_OK, TS_ROW_BAD_PARAMS, TS_ROW_BAD_LOGITS = 0, 1, 2
TS_MAX_LOGPROBS = 1024
TS_MAX_SLICES = 64
TS_LOGPROBS_PROCESSED = 1
TS_PROBE_SMALL_OPERANDS, TS_PROBE_RANDOM_OPERANDS = 0, 1
TS_NOALLOC_SCRATCH_BYTES = 96 << 20
PARAMS_BYTES = 24

# (name, restype, argtypes) of every symbol the headers declare
# (include/top_sampling.h and the measurement aids of top_sampling_measure.h).
_VP, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SYMBOLS = {
    "lmhead_logits_local": (ctypes.c_int, [_VP, _I64, _I64, _I64, _VP, _I64, _I64, _VP, _I64, _VP]),
    "quantize_rows_e4m3": (ctypes.c_int, [_VP, _I64, _I64, _I64, _VP, _I64, _VP, _VP]),
    "lmhead_logits_local_e4m3": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I64, _VP, _VP, _I64, _I64,
                                                _VP, _I64, _VP]),
    "sampler_workspace_bytes": (_SZ, [_I64, _I64, _I32]),
    "sampler_sample": (ctypes.c_int, [_VP, _I64, _I64, _I64, _VP, _I64, _I32, _VP, _VP, _VP, _VP,
                                      _VP, _VP, _SZ, _VP]),
    "sampler_sample_noalloc": (ctypes.c_int, [_VP, _I64, _I64, _I64, _VP, _I64, _I32, _VP, _VP,
                                              _VP, _VP, _VP, _VP]),
    "sampler_workspace_bytes_slices": (_SZ, [_I64, _VP, _I32, _I32]),
    "sampler_sample_slices": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I64, _VP, _I64, _I32, _VP, _VP,
                                             _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sampler_sample_ex": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I64, _VP, _I64, _I32, _I32, _VP,
                                         _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sampler_assemble_vocab_slices": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I64, _VP, _I64, _VP]),
    "sampler_assemble_and_sample": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I64, _VP, _I64, _VP, _I64,
                                                   _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                                   _VP]),
    "ts_mfma_clock_probe": (ctypes.c_int, [_VP, _I32, _I64, _I32, _VP]),
    "ts_gumbel_keys": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP]),
    "ts_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ts_last_error": (ctypes.c_char_p, []),
}


def _load() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime.  Load it first so the library binds to
    # that same runtime: a second copy of the HIP/HSA runtime in the process
    # (the one under /opt/rocm) would own the device independently.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python top_sampling_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SYMBOLS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class TopSamplingError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{lib.ts_status_string(code).decode()}: {msg}")
        self.code = code


class TopSamplingValueError(TopSamplingError, ValueError):
    pass


def _check(code: int) -> None:
    if code == TS_OK:
        return
    msg = lib.ts_last_error().decode()
    if code in (TS_EINVAL, TS_EUNSUPPORTED, TS_EWORKSPACE):
        raise TopSamplingValueError(code, msg)
    raise TopSamplingError(code, msg)


def _torch():
    import torch

    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


# ---------------------------------------------------------------- projection
def lmhead_logits_local(hidden, lm_head, out=None, stream=None):
    """fp32 ``[rows, V_local]`` logits of bf16 ``hidden [rows, H]`` against the
    bf16 vocabulary slice ``lm_head [V_local, H]``.  ``out`` may be a column
    slice of a wider fp32 buffer (its row stride is the leading dimension)."""
    torch = _torch()
    rows, h = hidden.shape
    vocab, h2 = lm_head.shape
    if h != h2:
        raise ValueError(f"hidden size mismatch: {h} vs {h2}")
    if hidden.dtype != torch.bfloat16 or lm_head.dtype != torch.bfloat16:
        raise TypeError("hidden and lm_head must be bfloat16")
    if hidden.stride(1) != 1 or lm_head.stride(1) != 1:
        raise ValueError("hidden and lm_head must be K-contiguous")
    if out is None:
        out = torch.empty(rows, vocab, dtype=torch.float32, device=hidden.device)
    if out.shape != (rows, vocab) or out.dtype != torch.float32 or out.stride(1) != 1:
        raise ValueError("out must be fp32 [rows, V_local] with unit column stride")
    _check(lib.lmhead_logits_local(_ptr(hidden), rows, h, hidden.stride(0), _ptr(lm_head), vocab,
                                   lm_head.stride(0), _ptr(out), out.stride(0),
                                   _stream_ptr(stream)))
    return out


def compute_logits_local(hidden, lm_head, out=None, stream=None):
    """The rank's own vocabulary shard ``[rows, V_local]``: no gather, no
    full-vocabulary buffer anywhere."""
    return lmhead_logits_local(hidden, lm_head, out=out, stream=stream)


# ---------------------------------------------------------- FP8 projection
def quantize_rows_e4m3(x, out=None, scales=None, stream=None):
    """bf16 ``[rows, cols]`` -> (uint8 E4M3 codes ``[rows, cols]``, fp32 per-row
    scales ``[rows]``): scale = max|x| / 448, code = nearest E4M3 of x / scale."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be bf16 [rows, cols] with unit column stride")
    rows, cols = x.shape
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib.quantize_rows_e4m3(_ptr(x), rows, cols, x.stride(0), _ptr(out), out.stride(0),
                                  _ptr(scales), _stream_ptr(stream)))
    return out, scales


def lmhead_logits_local_e4m3(hidden, hidden_scales, lm_head, lm_head_scales, out=None,
                             stream=None):
    """fp32 ``[rows, V_local]`` = s_x[r] * s_w[v] * (codes_x @ codes_w^T) for
    uint8 E4M3 codes ``hidden [rows, H]``, ``lm_head [V_local, H]`` and fp32
    per-row scales: the rank's own vocabulary slice, no gather."""
    torch = _torch()
    rows, h = hidden.shape
    vocab, h2 = lm_head.shape
    if h != h2 or hidden.dtype != torch.uint8 or lm_head.dtype != torch.uint8:
        raise ValueError("hidden and lm_head must be uint8 codes with the same hidden size")
    if hidden.stride(1) != 1 or lm_head.stride(1) != 1:
        raise ValueError("codes must have unit column stride")
    if out is None:
        out = torch.empty(rows, vocab, dtype=torch.float32, device=hidden.device)
    _check(lib.lmhead_logits_local_e4m3(
        _ptr(hidden), _ptr(hidden_scales), rows, h, hidden.stride(0), _ptr(lm_head),
        _ptr(lm_head_scales), vocab, lm_head.stride(0), _ptr(out), out.stride(0),
        _stream_ptr(stream)))
    return out


# ------------------------------------------------------------------ assembly
def sampler_assemble_vocab_slices(slices, out=None, stream=None):
    """``out[:, off_s:off_s+cols_s] = slices[s]`` (bit-exact)."""
    torch = _torch()
    n, rows, ptrs, cols, lds = _slice_arrays(slices)
    total = sum(int(s.shape[1]) for s in slices)
    if out is None:
        out = torch.empty(rows, total, dtype=torch.float32, device=slices[0].device)
    if out.shape != (rows, total) or out.stride(1) != 1 or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [rows, sum cols] with unit column stride")
    _check(lib.sampler_assemble_vocab_slices(ptrs, cols, lds, n, rows, _ptr(out), out.stride(0),
                                             _stream_ptr(stream)))
    return out


# ------------------------------------------------------------------- sampler
def sampler_workspace_bytes(rows: int, vocab: int, max_logprobs: int) -> int:
    return int(lib.sampler_workspace_bytes(rows, vocab, max_logprobs))


def params_to_device(params: np.ndarray, device):
    """Copy a record array of row parameters (24-byte records) to the device."""
    torch = _torch()
    raw = np.ascontiguousarray(params).view(np.uint8).reshape(-1)
    if raw.shape[0] != PARAMS_BYTES * params.shape[0]:
        raise ValueError("parameter records must be 24 bytes")
    return torch.from_numpy(raw.copy()).to(device)


@dataclass
class SampleOutput:
    token_ids: object       # int32 [rows]
    token_logprobs: object  # fp32 [rows]
    topn_ids: object        # int32 [rows, max_logprobs]
    topn_logprobs: object   # fp32 [rows, max_logprobs]
    row_status: object      # int32 [rows]


def allocate_sample_output(rows: int, max_logprobs: int, device) -> SampleOutput:
    torch = _torch()
    return SampleOutput(
        torch.empty(rows, dtype=torch.int32, device=device),
        torch.empty(rows, dtype=torch.float32, device=device),
        torch.empty(rows, max_logprobs, dtype=torch.int32, device=device),
        torch.empty(rows, max_logprobs, dtype=torch.float32, device=device),
        torch.empty(rows, dtype=torch.int32, device=device),
    )


def allocate_workspace(rows: int, vocab: int, max_logprobs: int, device):
    torch = _torch()
    n = max(256, sampler_workspace_bytes(rows, vocab, max_logprobs))
    return torch.empty(n, dtype=torch.uint8, device=device)


def sampler_sample(logits, params, row_offset: int = 0, max_logprobs: int = 0, out=None,
                   workspace=None, stream=None, processed: bool = False) -> SampleOutput:
    """Sample one token per row of fp32 ``logits [rows, V]`` (row stride = its
    leading dimension).  ``params`` is a device uint8 tensor of 24-byte
    ``ts_row_params`` records (see ``params_to_device``).  ``processed``
    returns log-probabilities of the sampled distribution (sampler_sample_ex
    with TS_LOGPROBS_PROCESSED) instead of the raw log_softmax."""
    if processed:
        return sampler_sample_slices([logits], params, row_offset, max_logprobs, out=out,
                                     workspace=workspace, stream=stream, processed=True)
    torch = _torch()
    rows, vocab = logits.shape
    if logits.dtype != torch.float32 or logits.stride(1) != 1:
        raise ValueError("logits must be fp32 with unit column stride")
    if params.dtype != torch.uint8 or params.numel() != PARAMS_BYTES * rows:
        raise ValueError("params must be rows x 24 bytes (uint8)")
    if out is None:
        out = allocate_sample_output(rows, max_logprobs, logits.device)
    if workspace is None:
        workspace = allocate_workspace(rows, vocab, max_logprobs, logits.device)
    _check(lib.sampler_sample(
        _ptr(logits), rows, vocab, logits.stride(0), _ptr(params), row_offset, max_logprobs,
        _ptr(out.token_ids), _ptr(out.token_logprobs),
        _ptr(out.topn_ids) if max_logprobs > 0 else None,
        _ptr(out.topn_logprobs) if max_logprobs > 0 else None,
        _ptr(out.row_status), _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return out


def sampler_sample_noalloc(logits, params, row_offset: int = 0, max_logprobs: int = 0, out=None,
                           stream=None) -> SampleOutput:
    """``sampler_sample`` with the library's built-in scratch as the
    workspace (no workspace argument; nothing is allocated by the call
    itself, ``out`` aside when it is not given).  Calls that overlap on one
    GPU share the scratch and must be serialised."""
    torch = _torch()
    rows, vocab = logits.shape
    if logits.dtype != torch.float32 or logits.stride(1) != 1:
        raise ValueError("logits must be fp32 with unit column stride")
    if params.dtype != torch.uint8 or params.numel() != PARAMS_BYTES * rows:
        raise ValueError("params must be rows x 24 bytes (uint8)")
    if out is None:
        out = allocate_sample_output(rows, max_logprobs, logits.device)
    _check(lib.sampler_sample_noalloc(
        _ptr(logits), rows, vocab, logits.stride(0), _ptr(params), row_offset, max_logprobs,
        _ptr(out.token_ids), _ptr(out.token_logprobs),
        _ptr(out.topn_ids) if max_logprobs > 0 else None,
        _ptr(out.topn_logprobs) if max_logprobs > 0 else None,
        _ptr(out.row_status), _stream_ptr(stream)))
    return out


def _slice_arrays(slices):
    torch = _torch()
    n = len(slices)
    if n < 1 or n > TS_MAX_SLICES:
        raise ValueError(f"need 1..{TS_MAX_SLICES} slices")
    rows = slices[0].shape[0]
    for s in slices:
        if s.dtype != torch.float32 or s.dim() != 2 or s.shape[0] != rows or s.stride(1) != 1:
            raise ValueError("slices must be fp32 [rows, cols_s] with unit column stride")
    ptrs = (ctypes.c_void_p * n)(*[_ptr(s) for s in slices])
    cols = (ctypes.c_int64 * n)(*[int(s.shape[1]) for s in slices])
    lds = (ctypes.c_int64 * n)(*[max(int(s.stride(0)), int(s.shape[1])) for s in slices])
    return n, rows, ptrs, cols, lds


def sampler_workspace_bytes_slices(rows: int, slice_cols, max_logprobs: int) -> int:
    n = len(slice_cols)
    cols = (ctypes.c_int64 * max(n, 1))(*[int(c) for c in slice_cols])
    return int(lib.sampler_workspace_bytes_slices(rows, cols, n, max_logprobs))


def sampler_sample_slices(slices, params, row_offset: int = 0, max_logprobs: int = 0, out=None,
                          workspace=None, stream=None, processed: bool = False) -> SampleOutput:
    """``sampler_sample`` over the column-wise concatenation of ``slices``
    (fp32 ``[rows, cols_s]`` each), read in place.  Token ids are global
    columns of that concatenation."""
    torch = _torch()
    n, rows, ptrs, cols, lds = _slice_arrays(slices)
    if params.dtype != torch.uint8 or params.numel() != PARAMS_BYTES * rows:
        raise ValueError("params must be rows x 24 bytes (uint8)")
    device = slices[0].device
    if out is None:
        out = allocate_sample_output(rows, max_logprobs, device)
    if workspace is None:
        nb = max(256, sampler_workspace_bytes_slices(rows, list(cols), max_logprobs))
        workspace = torch.empty(nb, dtype=torch.uint8, device=device)
    head = (ptrs, cols, lds, n, rows, _ptr(params), row_offset, max_logprobs)
    call = (lambda *t: lib.sampler_sample_ex(*head, TS_LOGPROBS_PROCESSED, *t)) if processed \
        else (lambda *t: lib.sampler_sample_slices(*head, *t))
    _check(call(
        _ptr(out.token_ids), _ptr(out.token_logprobs),
        _ptr(out.topn_ids) if max_logprobs > 0 else None,
        _ptr(out.topn_logprobs) if max_logprobs > 0 else None,
        _ptr(out.row_status), _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return out


def sampler_assemble_and_sample(slices, params, row_offset: int = 0, max_logprobs: int = 0,
                                assembled=None, out=None, workspace=None, stream=None,
                                processed: bool = False):
    """``sampler_assemble_vocab_slices`` into ``assembled`` and
    ``sampler_sample_slices`` of the same slices in one call, which reads the
    logits once.  Returns ``(assembled, SampleOutput)``."""
    torch = _torch()
    n, rows, ptrs, cols, lds = _slice_arrays(slices)
    total = sum(int(c) for c in cols)
    if params.dtype != torch.uint8 or params.numel() != PARAMS_BYTES * rows:
        raise ValueError("params must be rows x 24 bytes (uint8)")
    device = slices[0].device
    if assembled is None:
        assembled = torch.empty(rows, total, dtype=torch.float32, device=device)
    if assembled.shape != (rows, total) or assembled.stride(1) != 1 or \
            assembled.dtype != torch.float32:
        raise ValueError("assembled must be fp32 [rows, sum cols] with unit column stride")
    if out is None:
        out = allocate_sample_output(rows, max_logprobs, device)
    if workspace is None:
        nb = max(256, sampler_workspace_bytes_slices(rows, list(cols), max_logprobs))
        workspace = torch.empty(nb, dtype=torch.uint8, device=device)
    _check(lib.sampler_assemble_and_sample(
        ptrs, cols, lds, n, rows, _ptr(assembled), assembled.stride(0), _ptr(params), row_offset,
        max_logprobs, TS_LOGPROBS_PROCESSED if processed else 0,
        _ptr(out.token_ids), _ptr(out.token_logprobs),
        _ptr(out.topn_ids) if max_logprobs > 0 else None,
        _ptr(out.topn_logprobs) if max_logprobs > 0 else None,
        _ptr(out.row_status), _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return assembled, out


def mfma_clock_probe(workgroups: int, iters: int, device, stream=None, random: bool = False):
    """Launch the matrix-core clock probe (a measurement aid) and return the
    device tensor of per-workgroup ticks [workgroups, 4] (uint64 stored as
    int64): shader clock start / end, 100 MHz real time start / end.
    ``random`` selects random operand bits instead of a few small values."""
    torch = _torch()
    ticks = torch.zeros(workgroups, 4, dtype=torch.int64, device=device)
    mode = TS_PROBE_RANDOM_OPERANDS if random else TS_PROBE_SMALL_OPERANDS
    _check(lib.ts_mfma_clock_probe(_ptr(ticks), workgroups, iters, mode, _stream_ptr(stream)))
    return ticks


def gumbel_keys(logits, row_max, temperature, seeds, rows, ids, stream=None):
    """The sampler's own fp32 Gumbel-max keys and Philox noise words for listed
    tokens (a check aid): all arguments are 1-D device tensors of one length
    (fp32 logits / row_max / temperature, int64 seeds (uint64 bits) and rows,
    int32 ids).  Returns (keys fp32, words int32 holding the uint32 bits)."""
    torch = _torch()
    n = int(ids.numel())
    keys = torch.empty(n, dtype=torch.float32, device=ids.device)
    words = torch.empty(n, dtype=torch.int32, device=ids.device)
    _check(lib.ts_gumbel_keys(_ptr(logits), _ptr(row_max), _ptr(temperature), _ptr(seeds),
                              _ptr(rows), _ptr(ids), n, _ptr(keys), _ptr(words),
                              _stream_ptr(stream)))
    return keys, words
