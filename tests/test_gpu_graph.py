"""The whole step captured in a HIP graph and replayed.

Serving replays fixed graph buckets, so every call of the path must be
stream-ordered, with no allocation, memset or synchronisation inside it.  The
step (projection, the slices a rank would receive, their assembly, the
sampler) is captured once and replayed several times, with eager work that
overwrites every buffer and a synchronisation between replays; every replay
must equal the eager run bit for bit.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ts():
    import top_sampling_amd

    return top_sampling_amd


def say(*a):
    print(*a, flush=True)


FIELDS = ("token_ids", "token_logprobs", "topn_ids", "topn_logprobs", "row_status")


def _bits(t):
    import torch

    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("one_call", [False, True])
def test_step_graph_replays(dev, ts, one_call):
    """one_call: assembly and sampler through sampler_assemble_and_sample (the
    bench's step); else the assembly kernel, then the sampler on the buffer."""
    import torch

    rng = np.random.default_rng(31)
    rows, H, V, max_lp = 40, 512, 20000, 8
    widths = [6000, 4000, 7000, 3000]
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    hidden = torch.randn(rows, H, device=dev, generator=g).to(torch.bfloat16)
    lm_head = (torch.randn(V, H, device=dev, generator=g) * 0.05).to(torch.bfloat16)
    params = ts.params_to_device(workloads.random_params(rng, rows, V, max_lp), dev)
    local = torch.empty(rows, V, device=dev)
    slices = [torch.empty(rows, w, device=dev) for w in widths]
    batch = torch.empty(rows, V, device=dev)
    ws = ts.allocate_workspace(rows, V, max_lp, dev)
    if one_call:
        ws = torch.empty(max(256, ts.sampler_workspace_bytes_slices(rows, widths, max_lp)),
                         dtype=torch.uint8, device=dev)
    out = ts.allocate_sample_output(rows, max_lp, dev)

    def step():
        ts.lmhead_logits_local(hidden, lm_head, out=local)
        c0 = 0
        for s, w in zip(slices, widths):  # the exchange's delivery, as device copies
            s.copy_(local[:, c0:c0 + w])
            c0 += w
        if one_call:
            ts.sampler_assemble_and_sample(slices, params, 3, max_lp, assembled=batch, out=out,
                                           workspace=ws)
        else:
            ts.sampler_assemble_vocab_slices(slices, out=batch)
            ts.sampler_sample(batch, params, row_offset=3, max_logprobs=max_lp, out=out,
                              workspace=ws)

    say("graph: eager step", rows, H, V, "one call" if one_call else "two calls")
    step()
    torch.cuda.synchronize()
    ref_logits = batch.clone()
    ref = {k: getattr(out, k).clone() for k in FIELDS}
    assert (ref["row_status"] == 0).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        local.fill_(float("nan"))
        batch.fill_(-1.0)
        ws.fill_(0xA5)
        for k in FIELDS:
            getattr(out, k).fill_(-7)
        torch.cuda.synchronize()
        say("graph: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(batch), _bits(ref_logits)), f"replay {rep}: assembled logits"
        for k in FIELDS:
            assert torch.equal(_bits(getattr(out, k)), _bits(ref[k])), f"replay {rep}: {k}"
