"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and its host-side validation rejects bad calls before any HIP call (so these
run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import top_sampling_amd as ts
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "top_sampling.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "top_sampling_measure.h")

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _declared_functions(path):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M))


def test_header_symbols_exported():
    product = _declared_functions(HEADER)
    measure = _declared_functions(MEASURE_HEADER)
    names = product | measure
    assert names == set(ts.SYMBOLS), names
    # the measurement aids are not part of the product header
    assert measure == {"ts_mfma_clock_probe", "ts_gumbel_keys"}
    assert not (product & measure)
    lib = ctypes.CDLL(ts.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read() + open(MEASURE_HEADER).read()
    for name, val in [("TS_MAX_LOGPROBS", ts.TS_MAX_LOGPROBS), ("TS_MAX_SLICES", ts.TS_MAX_SLICES),
                      ("TS_LOGPROBS_PROCESSED", ts.TS_LOGPROBS_PROCESSED),
                      ("TS_PROBE_SMALL_OPERANDS", ts.TS_PROBE_SMALL_OPERANDS),
                      ("TS_NOALLOC_SCRATCH_BYTES", "(96ull << 20)"),
                      ("TS_PROBE_RANDOM_OPERANDS", ts.TS_PROBE_RANDOM_OPERANDS)]:
        assert re.search(rf"#define {name} {re.escape(str(val))}", text), name
    assert ts.TS_NOALLOC_SCRATCH_BYTES == 96 << 20
    assert workloads.PARAMS_DTYPE.itemsize == ts.PARAMS_BYTES


def test_status_strings():
    assert ts.lib.ts_status_string(0) == b"TS_OK"
    assert ts.lib.ts_status_string(-1) == b"TS_EINVAL"
    assert ts.lib.ts_status_string(-3) == b"TS_EWORKSPACE"
    assert ts.lib.ts_status_string(99) == b"TS_UNKNOWN"


def test_workspace_query_is_host_only():
    assert ts.sampler_workspace_bytes(640, 151936, 20) > 0
    assert ts.sampler_workspace_bytes(-1, 10, 0) == 0


def _gemm(**kw):
    a = dict(hidden=FAKE, rows=4, hidden_dim=256, ld_hidden=256, lm_head=FAKE, vocab=64,
             ld_lm_head=256, logits=FAKE, ld_logits=64)
    a.update(kw)
    return ts.lib.lmhead_logits_local(a["hidden"], a["rows"], a["hidden_dim"], a["ld_hidden"],
                                      a["lm_head"], a["vocab"], a["ld_lm_head"], a["logits"],
                                      a["ld_logits"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), ts.TS_EINVAL),
    (dict(vocab=-5), ts.TS_EINVAL),
    (dict(hidden=None), ts.TS_EINVAL),
    (dict(ld_hidden=128), ts.TS_EINVAL),
    (dict(ld_logits=63), ts.TS_EINVAL),
    (dict(hidden_dim=0), ts.TS_EINVAL),
    (dict(hidden_dim=250, ld_hidden=256, ld_lm_head=256), ts.TS_EUNSUPPORTED),
    (dict(ld_hidden=260), ts.TS_EUNSUPPORTED),
    (dict(hidden=FAKE + 8), ts.TS_EUNSUPPORTED),
    (dict(rows=1 << 31), ts.TS_EUNSUPPORTED),
])
def test_gemm_validation(kw, code):
    assert _gemm(**kw) == code
    assert ts.lib.ts_last_error()


def test_gemm_empty_is_noop():
    assert _gemm(rows=0, hidden=None, lm_head=None, logits=None) == ts.TS_OK
    assert _gemm(vocab=0) == ts.TS_OK


def _sample(**kw):
    a = dict(logits=FAKE, rows=8, vocab=100, ld=100, params=FAKE, row_offset=0, max_logprobs=5,
             tok=FAKE, tlp=FAKE, tid=FAKE, tnlp=FAKE, status=FAKE, ws=None, ws_bytes=0)
    a.update(kw)
    return ts.lib.sampler_sample(a["logits"], a["rows"], a["vocab"], a["ld"], a["params"],
                                 a["row_offset"], a["max_logprobs"], a["tok"], a["tlp"],
                                 a["tid"], a["tnlp"], a["status"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), ts.TS_EINVAL),
    (dict(max_logprobs=-1), ts.TS_EINVAL),
    (dict(max_logprobs=ts.TS_MAX_LOGPROBS + 1), ts.TS_EUNSUPPORTED),
    (dict(row_offset=-3), ts.TS_EINVAL),
    (dict(vocab=0), ts.TS_EINVAL),
    (dict(ld=99), ts.TS_EINVAL),
    (dict(logits=None), ts.TS_EINVAL),
    (dict(params=None), ts.TS_EINVAL),
    (dict(tok=None), ts.TS_EINVAL),
    (dict(tid=None), ts.TS_EINVAL),
    (dict(params=FAKE + 4), ts.TS_EUNSUPPORTED),
    (dict(), ts.TS_EWORKSPACE),                       # no workspace
    (dict(ws=FAKE, ws_bytes=1), ts.TS_EWORKSPACE),    # too small
])
def test_sampler_validation(kw, code):
    assert _sample(**kw) == code


def test_sampler_empty_is_noop():
    assert _sample(rows=0, logits=None, params=None, tok=None) == ts.TS_OK


def test_sampler_null_topn_allowed_only_without_logprobs():
    # max_logprobs == 0: NULL top-N is fine, so validation reaches the workspace check.
    assert _sample(max_logprobs=0, tid=None, tnlp=None) == ts.TS_EWORKSPACE


def _assemble(ptrs, cols, lds, rows=4, out=FAKE * 16, ld_out=None):
    n = len(ptrs)
    ld_out = sum(cols) if ld_out is None else ld_out
    P = (ctypes.c_void_p * max(n, 1))(*ptrs)
    C = (ctypes.c_int64 * max(n, 1))(*cols)
    L = (ctypes.c_int64 * max(n, 1))(*lds)
    return ts.lib.sampler_assemble_vocab_slices(P, C, L, n, rows, out, ld_out, None)


def test_assemble_validation():
    assert _assemble([], [], []) == ts.TS_EINVAL
    assert _assemble([FAKE] * 65, [4] * 65, [4] * 65) == ts.TS_EUNSUPPORTED
    assert _assemble([FAKE, FAKE * 2], [4, -1], [4, 4]) == ts.TS_EINVAL
    assert _assemble([FAKE, FAKE * 2], [4, 8], [4, 4]) == ts.TS_EINVAL       # ld < width
    assert _assemble([FAKE, None], [4, 8], [4, 8]) == ts.TS_EINVAL           # NULL slice
    assert _assemble([FAKE, FAKE * 2], [4, 8], [4, 8], ld_out=11) == ts.TS_EINVAL
    assert _assemble([FAKE, FAKE * 2], [4, 8], [4, 8], out=None) == ts.TS_EINVAL
    # a slice inside the output rows is rejected
    assert _assemble([FAKE * 16 + 8, FAKE * 2], [4, 8], [12, 8]) == ts.TS_EINVAL
    assert _assemble([FAKE, FAKE * 2], [4, 8], [4, 8], rows=0) == ts.TS_OK


def test_compute_logits_local_wiring(monkeypatch):
    """Mirror of the wiring test the page describes (a recording fake in place
    of the kernel): the local-logits hook asks for the rank's own slice,
    [rows, V_local], and hands back exactly that, with no gather."""
    import torch

    calls = []

    class FakeLib:
        def lmhead_logits_local(self, *args):
            calls.append(args)
            return 0

    monkeypatch.setattr(ts, "lib", FakeLib())
    hidden = torch.zeros(6, 16, dtype=torch.bfloat16)
    lm_head_local = torch.zeros(40, 16, dtype=torch.bfloat16)   # this rank's vocabulary slice
    out = ts.compute_logits_local(hidden, lm_head_local, stream=0)
    assert tuple(out.shape) == (6, 40)
    (_, rows, h, ldh, _, vocab, ldw, _, ldl, _), = calls
    assert (rows, h, ldh, vocab, ldw, ldl) == (6, 16, 16, 40, 16, 40)
    # Writing the slice into a wider buffer uses the wider row stride.
    wide = torch.empty(6, 160)
    ts.compute_logits_local(hidden, lm_head_local, out=wide[:, 40:80], stream=0)
    assert calls[-1][8] == 160 and calls[-1][5] == 40


def test_params_layout_roundtrip():
    p = workloads.make_params(workloads.get("spec_decode"))
    raw = np.ascontiguousarray(p).view(np.uint8)
    assert raw.shape[0] == 24 * p.shape[0]
    back = raw.view(workloads.PARAMS_DTYPE)
    assert np.array_equal(back["seed"], p["seed"])


def _sample_slices(ptrs, cols, lds, **kw):
    a = dict(rows=8, params=FAKE, row_offset=0, max_logprobs=5, tok=FAKE, tlp=FAKE, tid=FAKE,
             tnlp=FAKE, status=FAKE, ws=None, ws_bytes=0)
    a.update(kw)
    n = len(ptrs)
    P = (ctypes.c_void_p * max(n, 1))(*ptrs)
    C = (ctypes.c_int64 * max(n, 1))(*cols)
    L = (ctypes.c_int64 * max(n, 1))(*lds)
    return ts.lib.sampler_sample_slices(P, C, L, a.get("n", n), a["rows"], a["params"],
                                        a["row_offset"], a["max_logprobs"], a["tok"], a["tlp"],
                                        a["tid"], a["tnlp"], a["status"], a["ws"], a["ws_bytes"],
                                        None)


def test_sampler_slices_validation():
    two = ([FAKE, FAKE * 2], [40, 60], [40, 60])
    assert _sample_slices([], [], []) == ts.TS_EINVAL
    assert _sample_slices([FAKE] * 65, [4] * 65, [4] * 65) == ts.TS_EUNSUPPORTED
    assert _sample_slices([FAKE, FAKE * 2], [40, -1], [40, 4]) == ts.TS_EINVAL
    assert _sample_slices([FAKE, FAKE * 2], [40, 60], [40, 59]) == ts.TS_EINVAL   # ld < width
    assert _sample_slices([FAKE, None], [40, 60], [40, 60]) == ts.TS_EINVAL       # NULL slice
    assert _sample_slices([FAKE, FAKE + 2], [40, 60], [40, 60]) == ts.TS_EUNSUPPORTED
    assert _sample_slices([FAKE, FAKE * 2], [0, 0], [0, 0]) == ts.TS_EINVAL       # vocab 0
    assert _sample_slices(*two, rows=-1) == ts.TS_EINVAL
    assert _sample_slices(*two, max_logprobs=-1) == ts.TS_EINVAL
    assert _sample_slices(*two, row_offset=-1) == ts.TS_EINVAL
    assert _sample_slices(*two, params=None) == ts.TS_EINVAL
    assert _sample_slices(*two) == ts.TS_EWORKSPACE
    assert _sample_slices(*two, ws=FAKE, ws_bytes=255) == ts.TS_EWORKSPACE
    # An empty slice may be NULL; rows == 0 is a no-op.
    assert _sample_slices([FAKE, None, FAKE * 2], [40, 0, 60], [40, 0, 60]) == ts.TS_EWORKSPACE
    assert _sample_slices(*two, rows=0, params=None, tok=None) == ts.TS_OK


def test_slices_workspace_query():
    V = 151936
    assert ts.sampler_workspace_bytes_slices(640, [V], 20) == ts.sampler_workspace_bytes(640, V, 20)
    four = ts.sampler_workspace_bytes_slices(640, [V // 4] * 4, 20)
    # more, shorter chunks: more records, fewer candidate slots per chunk
    assert 0 < four <= 2 * ts.sampler_workspace_bytes(640, V, 20)
    assert ts.sampler_workspace_bytes_slices(640, [V // 64] * 64, 20) > 0
    assert ts.sampler_workspace_bytes_slices(640, [], 20) == 0
    assert ts.sampler_workspace_bytes_slices(640, [10, -1], 20) == 0
    assert ts.sampler_workspace_bytes_slices(640, [4] * 65, 20) == 0


def _gemm8(**kw):
    a = dict(hidden=FAKE, xs=FAKE, rows=4, hidden_dim=256, ld_hidden=256, lm_head=FAKE, ws=FAKE,
             vocab=64, ld_lm_head=256, logits=FAKE, ld_logits=64)
    a.update(kw)
    return ts.lib.lmhead_logits_local_e4m3(a["hidden"], a["xs"], a["rows"], a["hidden_dim"],
                                           a["ld_hidden"], a["lm_head"], a["ws"], a["vocab"],
                                           a["ld_lm_head"], a["logits"], a["ld_logits"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), ts.TS_EINVAL),
    (dict(hidden=None), ts.TS_EINVAL),
    (dict(xs=None), ts.TS_EINVAL),
    (dict(ws=None), ts.TS_EINVAL),
    (dict(ld_hidden=128), ts.TS_EINVAL),
    (dict(ld_logits=63), ts.TS_EINVAL),
    (dict(hidden_dim=0), ts.TS_EINVAL),
    (dict(hidden_dim=192, ld_hidden=256, ld_lm_head=256), ts.TS_EUNSUPPORTED),   # not x128
    (dict(ld_hidden=264), ts.TS_EUNSUPPORTED),                                  # not x16
    (dict(hidden=FAKE + 8), ts.TS_EUNSUPPORTED),
    (dict(xs=FAKE + 2), ts.TS_EUNSUPPORTED),
    (dict(vocab=1 << 31), ts.TS_EUNSUPPORTED),
])
def test_gemm_e4m3_validation(kw, code):
    assert _gemm8(**kw) == code
    assert ts.lib.ts_last_error()


def test_gemm_e4m3_empty_is_noop():
    assert _gemm8(rows=0, hidden=None, xs=None) == ts.TS_OK
    assert _gemm8(vocab=0) == ts.TS_OK


def test_quantize_e4m3_validation():
    q = ts.lib.quantize_rows_e4m3
    assert q(FAKE, -1, 8, 8, FAKE, 8, FAKE, None) == ts.TS_EINVAL
    assert q(FAKE, 4, 8, 7, FAKE, 8, FAKE, None) == ts.TS_EINVAL      # ld_in < cols
    assert q(FAKE, 4, 8, 8, FAKE, 7, FAKE, None) == ts.TS_EINVAL      # ld_out < cols
    assert q(None, 4, 8, 8, FAKE, 8, FAKE, None) == ts.TS_EINVAL
    assert q(FAKE, 4, 8, 8, FAKE, 8, None, None) == ts.TS_EINVAL
    assert q(FAKE + 1, 4, 8, 8, FAKE, 8, FAKE, None) == ts.TS_EUNSUPPORTED
    assert q(None, 0, 8, 8, None, 8, None, None) == ts.TS_OK


def test_sampler_ex_validation():
    P = (ctypes.c_void_p * 2)(FAKE, FAKE * 2)
    C = (ctypes.c_int64 * 2)(40, 60)
    L = (ctypes.c_int64 * 2)(40, 60)
    ex = lambda flags, ws=None, nb=0: ts.lib.sampler_sample_ex(  # noqa: E731
        P, C, L, 2, 8, FAKE, 0, 5, flags, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nb, None)
    assert ex(2) == ts.TS_EINVAL                       # unknown flag bit
    assert ex(-1) == ts.TS_EINVAL
    assert ex(0) == ts.TS_EWORKSPACE                   # valid up to the workspace
    assert ex(ts.TS_LOGPROBS_PROCESSED) == ts.TS_EWORKSPACE


def _assemble_sample(ptrs, cols, lds, rows=8, out=FAKE * 64, ld_out=None, flags=0,
                     params=FAKE, max_logprobs=5, tok=FAKE, ws=None, nb=0):
    n = len(ptrs)
    ld_out = sum(cols) if ld_out is None else ld_out
    P = (ctypes.c_void_p * max(n, 1))(*ptrs)
    C = (ctypes.c_int64 * max(n, 1))(*cols)
    L = (ctypes.c_int64 * max(n, 1))(*lds)
    return ts.lib.sampler_assemble_and_sample(P, C, L, n, rows, out, ld_out, params, 0,
                                              max_logprobs, flags, tok, FAKE, FAKE, FAKE, FAKE,
                                              ws, nb, None)


def test_assemble_and_sample_validation():
    """Both calls' checks, every one before anything is enqueued: the
    assembly's (output width, NULL or overlapping output) and the sampler's
    (flags, parameters, workspace)."""
    two = ([FAKE, FAKE * 2], [40, 60], [40, 60])
    assert _assemble_sample([], [], []) == ts.TS_EINVAL
    assert _assemble_sample([FAKE] * 65, [4] * 65, [4] * 65) == ts.TS_EUNSUPPORTED
    assert _assemble_sample([FAKE, FAKE * 2], [40, -1], [40, 4]) == ts.TS_EINVAL
    assert _assemble_sample([FAKE, None], [40, 60], [40, 60]) == ts.TS_EINVAL     # NULL slice
    assert _assemble_sample(*two, ld_out=99) == ts.TS_EINVAL                      # ld_out < width
    assert _assemble_sample(*two, out=None) == ts.TS_EINVAL                       # NULL out
    assert _assemble_sample(*two, out=FAKE * 64 + 2) == ts.TS_EUNSUPPORTED        # misaligned out
    assert _assemble_sample(*two, out=FAKE) == ts.TS_EINVAL                       # overlaps slice 0
    assert _assemble_sample(*two, flags=2) == ts.TS_EINVAL                        # unknown flag
    assert _assemble_sample(*two, max_logprobs=-1) == ts.TS_EINVAL
    assert _assemble_sample(*two, params=None) == ts.TS_EINVAL
    assert _assemble_sample(*two, tok=None) == ts.TS_EINVAL
    assert _assemble_sample(*two) == ts.TS_EWORKSPACE                             # valid up to here
    assert _assemble_sample(*two, flags=ts.TS_LOGPROBS_PROCESSED, ws=FAKE, nb=255) == \
        ts.TS_EWORKSPACE
    assert _assemble_sample(*two, rows=-1) == ts.TS_EINVAL
    assert _assemble_sample(*two, rows=0, out=None, params=None, tok=None) == ts.TS_OK


def test_mfma_clock_probe_validation():
    probe = ts.lib.ts_mfma_clock_probe
    rnd = ts.TS_PROBE_RANDOM_OPERANDS
    assert probe(None, 4, 16, rnd, None) == ts.TS_EINVAL
    assert probe(FAKE + 4, 4, 16, rnd, None) == ts.TS_EINVAL        # misaligned
    assert probe(FAKE, 0, 16, rnd, None) == ts.TS_EINVAL
    assert probe(FAKE, 65537, 16, rnd, None) == ts.TS_EINVAL
    assert probe(FAKE, 4, 0, rnd, None) == ts.TS_EINVAL
    assert probe(FAKE, 4, (1 << 24) + 1, rnd, None) == ts.TS_EINVAL
    assert probe(FAKE, 4, 16, 2, None) == ts.TS_EINVAL              # unknown operand mode


def test_gumbel_keys_validation():
    gk = ts.lib.ts_gumbel_keys
    args = [FAKE] * 6
    assert gk(*args, 0, None, None, None) == ts.TS_OK                 # empty: no-op
    assert gk(*args, -1, FAKE, FAKE, None) == ts.TS_EINVAL
    assert gk(*args, 1 << 31, FAKE, FAKE, None) == ts.TS_EINVAL
    for i in range(6):
        bad = list(args)
        bad[i] = None
        assert gk(*bad, 4, FAKE, FAKE, None) == ts.TS_EINVAL, i
    bad = list(args)
    bad[3] = FAKE + 4                                                  # seeds need 8 bytes
    assert gk(*bad, 4, FAKE, FAKE, None) == ts.TS_EINVAL
    assert gk(*args, 4, FAKE + 2, FAKE, None) == ts.TS_EINVAL          # keys misaligned
    assert b"misaligned" in ts.lib.ts_last_error()


def test_sampler_noalloc_validation():
    """The no-allocation variant validates on the host: bad sizes, and shapes
    whose workspace exceeds the built-in scratch, are rejected before any HIP
    call."""
    f = ts.lib.sampler_sample_noalloc
    args = lambda rows, vocab, lp: (FAKE, rows, vocab, vocab, FAKE, 0, lp, FAKE, FAKE, FAKE,  # noqa: E731
                                    FAKE, FAKE, None)
    assert f(*args(-1, 100, 5)) == ts.TS_EINVAL
    assert f(*args(8, 100, -1)) == ts.TS_EINVAL
    assert f(*args(0, 100, 5)) == ts.TS_OK
    big = (4096, 262144, 20)
    assert ts.sampler_workspace_bytes(*big) > ts.TS_NOALLOC_SCRATCH_BYTES
    assert f(*args(*big)) == ts.TS_EUNSUPPORTED
    assert b"scratch" in ts.lib.ts_last_error()
    # the headline shapes fit the built-in scratch
    for shape in [(640, 151936, 20), (256, 151936, 5), (1024, 262144, 20)]:
        assert ts.sampler_workspace_bytes(*shape) <= ts.TS_NOALLOC_SCRATCH_BYTES, shape
