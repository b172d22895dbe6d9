"""The no-allocation sampler entry point against the workspace one.

sampler_sample_noalloc runs the sampler's kernels on the library's built-in
device scratch instead of a caller workspace.  Through the C ABI it must
give exactly what sampler_sample gives on the same inputs, on two calls in a
row (the second smaller, on a scratch still holding the first call's
contents), and reject a shape whose workspace exceeds the scratch.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

FIELDS = ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")


def say(*a):
    print(*a, flush=True)


def test_noalloc_matches_workspace_call_twice():
    import torch

    import top_sampling_amd as ts

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    for rows, V, max_lp, seed in [(640, 151936, 20, 1), (24, 30011, 7, 2)]:
        say("noalloc", rows, V, max_lp)
        rng = np.random.default_rng(seed)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        logits = torch.randn(rows, V, generator=g, device=dev) * 1.28
        params = workloads.random_params(rng, rows, V, max_lp)
        p = ts.params_to_device(params, dev)
        ref = ts.sampler_sample(logits, p, 3, max_lp)
        got = ts.sampler_sample_noalloc(logits, p, 3, max_lp)
        torch.cuda.synchronize()
        for k in FIELDS:
            a = getattr(ref, k).cpu().numpy()
            b = getattr(got, k).cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (rows, k)
        assert (got.row_status.cpu().numpy() == 0).any()


def test_noalloc_rejects_too_large():
    import torch

    import top_sampling_amd as ts

    dev = torch.device("cuda:0")
    rows, V = 4096, 262144
    assert ts.sampler_workspace_bytes(rows, V, 20) > ts.TS_NOALLOC_SCRATCH_BYTES
    logits = torch.empty(1, 1, device=dev)   # never read: rejected on the host
    code = ts.lib.sampler_sample_noalloc(logits.data_ptr(), rows, V, V, logits.data_ptr(), 0, 20,
                                         logits.data_ptr(), None, logits.data_ptr(),
                                         logits.data_ptr(), None, None)
    assert code == ts.TS_EUNSUPPORTED
