"""The matrix-core clock probe (a measurement aid for the bench's context
figures) through the C ABI: every workgroup's counters advance, and the clock
they imply lies in the part's range."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_mfma_clock_probe_ticks():
    import torch

    import top_sampling_amd as ts

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    for random in (False, True):
        print("mfma clock probe 64 x 4096, random operands:", random, flush=True)
        ticks = ts.mfma_clock_probe(64, 4096, dev, random=random)
        torch.cuda.synchronize()
        t = ticks.cpu().numpy().astype(np.float64)
        assert np.all(t[:, 1] > t[:, 0]) and np.all(t[:, 3] > t[:, 2])
        mhz = (t[:, 1] - t[:, 0]) / (t[:, 3] - t[:, 2]) * 100.0
        assert np.all((mhz > 300) & (mhz < 3500)), mhz
