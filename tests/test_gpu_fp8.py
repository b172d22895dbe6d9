"""GPU parity of the FP8 (OCP E4M3, per-row fp32 scales) projection path
against the CPU oracle, through the C ABI.

Bars: quantization codes and scales bit-exact (both sides divide in fp32 and
round to the nearest code, ties to even); logits within 2e-3 absolute of the
oracle's float64 sum of the same decoded codes times the same scales.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-3
GEMM_TILES = ["", "1", "2", "3", "4"]


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


@pytest.fixture(params=GEMM_TILES)
def gemm_tile(request, monkeypatch):
    if request.param:
        monkeypatch.setenv("TS_GEMM_TILE", request.param)
    else:
        monkeypatch.delenv("TS_GEMM_TILE", raising=False)
    return request.param


def _bf16_to_device(bits, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _u8(t):
    return t.cpu().numpy().view(np.uint8)


def _bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols,ld_extra", [(1, 1, 0), (3, 7, 5), (5, 2560, 0),
                                                (17, 4100, 3), (64, 300, 64)])
def test_quantize_matches_oracle(dev, ts, rows, cols, ld_extra):
    import torch

    rng = np.random.default_rng(rows * 1000 + cols)
    x = (rng.standard_normal((rows, cols)) * rng.uniform(0.01, 50, size=(rows, 1))).astype(np.float32)
    if rows >= 5 and cols >= 8:
        x[1] = 0.0                                  # zero row: scale 1, zero codes
        x[2, :4] = [np.nan, 1.0, -2.0, -0.0]        # NaN is ignored by the scale, coded 0x7F
        x[3, :3] = [np.inf, 5.0, -0.0]              # +inf: infinite scale, finite values -> +-0
        x[4, :5] = [1e-30, -3e-20, 7e-10, 6e4, -6e4]
    bits = workloads.bf16_bits_from_f32(x)
    buf = np.zeros((rows, cols + ld_extra), dtype=np.uint16)
    buf[:, :cols] = bits
    xin = _bf16_to_device(buf, dev)[:, :cols]
    out = torch.full((rows, cols + ld_extra), 0xAB, dtype=torch.uint8, device=dev)
    codes, scales = ts.quantize_rows_e4m3(xin, out=out[:, :cols])
    torch.cuda.synchronize()
    say("quantize", rows, cols, ld_extra)
    want_c, want_s = oracle.quantize_rows_e4m3(bits)
    got_s = scales.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    got = _u8(out)
    assert np.array_equal(got[:, :cols], want_c)
    assert np.all(got[:, cols:] == 0xAB)             # the padding is untouched


def _codes(rng, rows, hidden, std):
    x = (rng.standard_normal((rows, hidden)) * std).astype(np.float32)
    return oracle.quantize_rows_e4m3(workloads.bf16_bits_from_f32(x))


def _run_gemm(ts, dev, xc, xs, wc, ws, ld_extra=0):
    import torch

    rows, vocab = xc.shape[0], wc.shape[0]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    if ld_extra:
        wide = torch.full((rows, vocab + ld_extra), float("nan"), device=dev)
        ts.lmhead_logits_local_e4m3(to(xc), to(xs), to(wc), to(ws), out=wide[:, :vocab])
        torch.cuda.synchronize()
        full = wide.cpu().numpy()
        assert np.all(np.isnan(full[:, vocab:]))
        return full[:, :vocab].astype(np.float64)
    out = ts.lmhead_logits_local_e4m3(to(xc), to(xs), to(wc), to(ws))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("rows,vocab,hidden", [(1, 1, 128), (5, 300, 256), (64, 1000, 2560),
                                               (129, 777, 384), (321, 513, 640),
                                               (640, 1200, 2560)])
def test_gemm_e4m3_ragged(dev, ts, rows, vocab, hidden, gemm_tile):
    rng = np.random.default_rng(rows + vocab + hidden)
    xc, xs = _codes(rng, rows, hidden, 1.0)
    wc, ws = _codes(rng, vocab, hidden, 0.02)
    say("gemm e4m3", rows, vocab, hidden, gemm_tile)
    got = _run_gemm(ts, dev, xc, xs, wc, ws)
    want = oracle.lmhead_logits_e4m3(xc, xs, wc, ws)
    assert np.abs(got - want).max() <= LOGIT_TOL


def test_gemm_e4m3_into_wide_buffer(dev, ts):
    """A vocabulary slice written straight into its columns of a wider buffer."""
    rng = np.random.default_rng(3)
    xc, xs = _codes(rng, 40, 512, 1.0)
    wc, ws = _codes(rng, 700, 512, 0.05)
    say("gemm e4m3 wide")
    got = _run_gemm(ts, dev, xc, xs, wc, ws, ld_extra=9)
    assert np.abs(got - oracle.lmhead_logits_e4m3(xc, xs, wc, ws)).max() <= LOGIT_TOL


@pytest.mark.parametrize("vocab,ld", [(1001, 1028), (258, 264), (5, 8)])
def test_gemm_e4m3_row_stores_ragged_tail(dev, ts, vocab, ld, gemm_tile):
    """Rows that take 16-byte stores with a width that is not a multiple of 4:
    the scaled tail is written element by element, the padding untouched."""
    rng = np.random.default_rng(vocab + 1)
    xc, xs = _codes(rng, 333, 256, 1.0)
    wc, ws = _codes(rng, vocab, 256, 0.05)
    say("gemm e4m3 row stores", vocab, ld)
    got = _run_gemm(ts, dev, xc, xs, wc, ws, ld_extra=ld - vocab)
    assert np.abs(got - oracle.lmhead_logits_e4m3(xc, xs, wc, ws)).max() <= LOGIT_TOL


def test_gemm_e4m3_special_codes(dev, ts):
    """Saturated codes, subnormal codes and zero scales' neighbours: codes
    drawn uniformly over every finite E4M3 value."""
    rng = np.random.default_rng(17)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    xc = rng.choice(finite, size=(33, 256))
    wc = rng.choice(finite, size=(300, 256))
    xs = (2.0 ** rng.integers(-12, -6, size=33)).astype(np.float32)
    ws = (2.0 ** rng.integers(-12, -6, size=300)).astype(np.float32)
    say("gemm e4m3 special codes")
    got = _run_gemm(ts, dev, xc, xs, wc, ws)
    want = oracle.lmhead_logits_e4m3(xc, xs, wc, ws)
    assert np.abs(got - want).max() <= LOGIT_TOL * max(1.0, np.abs(want).max() * 1e-3)


def test_fp8_workload_full_size_sampled(dev, ts):
    """The FP8 workload at full size in the launch configuration the bench
    times: the hidden states and lm_head quantized on the GPU (checked code
    for code on sampled rows), then the projection checked on two whole rows
    and on every row at sampled columns, including the ragged tail."""
    import torch

    w = workloads.get("fp8")
    say("fp8 full", w.rows, w.vocab, w.hidden)
    x, wt = workloads.make_projection_device(w, dev)
    xq, xs = ts.quantize_rows_e4m3(x)
    wq, ws = ts.quantize_rows_e4m3(wt)
    out = ts.lmhead_logits_local_e4m3(xq, xs, wq, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.index)
    # quantization of sampled rows of both operands against the oracle
    for t, q, s, n in ((x, xq, xs, w.rows), (wt, wq, ws, w.vocab)):
        sel = np.unique(np.concatenate([rng.choice(n, 24, replace=False), [0, n - 1]]))
        idx = torch.from_numpy(sel).to(dev)
        want_c, want_s = oracle.quantize_rows_e4m3(_bits(t[idx]))
        assert np.array_equal(_u8(q[idx]), want_c)
        assert np.array_equal(s[idx].cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    xc, xsc = _u8(xq), xs.cpu().numpy()
    rows = np.unique(np.concatenate([rng.choice(w.rows, 6, replace=False), [0, w.rows - 1]]))
    cols = np.unique(np.concatenate([rng.choice(w.vocab, 3000, replace=False),
                                     np.arange(w.vocab - 300, w.vocab)]))
    full_rows = rows[:2]
    want = oracle.lmhead_logits_e4m3(xc[full_rows], xsc[full_rows], _u8(wq), ws.cpu().numpy())
    got = out[torch.from_numpy(full_rows).to(dev)].cpu().numpy().astype(np.float64)
    assert np.abs(got - want).max() <= LOGIT_TOL
    ci = torch.from_numpy(cols).to(dev)
    want = oracle.lmhead_logits_e4m3(xc, xsc, _u8(wq[ci]), ws[ci].cpu().numpy())
    got = out[:, ci].cpu().numpy().astype(np.float64)
    assert np.abs(got - want).max() <= LOGIT_TOL
