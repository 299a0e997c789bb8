"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

Neither path enqueues a memset or allocates, and the one-kernel path clears
its shared counters and flag at the end of every call, so a captured call can
be replayed. Each case captures one call, replays it three times with the
program's own eager work and synchronisations between the replays, and checks
main_grad after every replay against the same number of eager calls, bit for
bit (every call adds the same gradient again).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import _bits

pytestmark = pytest.mark.gpu

# a missing or unloadable library fails the module (no skip)
import sparse_embedding_weight_amd as ewg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield


def _replays_match_eager(call, ids, grad, mg0, workspace):
    eager = mg0.clone()
    captured = mg0.clone()
    side = torch.cuda.Stream()
    # warm-up on a side stream (torch's recommendation before capture)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        scratch = mg0.clone()
        call(ids, grad, scratch, workspace)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(ids, grad, captured, workspace)
    torch.cuda.synchronize()
    # capture does not run the call: captured still holds mg0
    assert torch.equal(_bits(captured), _bits(mg0))
    noise = torch.randn(1 << 20, device="cuda")
    for k in range(3):
        g.replay()
        noise.mul_(1.0001).add_(1.0)          # unrelated eager work between replays
        call(ids, grad, eager, workspace)     # the eager reference, same workspace
        torch.cuda.synchronize()
        assert torch.equal(_bits(captured), _bits(eager)), f"replay {k} differs from eager"


def test_one_kernel_call_in_a_graph():
    w = wl.WORKLOADS["zipf1.1_4096_v32000_h4096"]
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg0 = wl.make_main_grad(w, "cuda")
    ws = ewg.new_workspace(ids.numel(), w.hidden, "cuda")
    _replays_match_eager(lambda i, g, m, wsp: ewg.accumulate_embedding_wgrad(i, g, m, workspace=wsp),
                         ids, grad, mg0, ws)


def test_vocab_shard_call_in_a_graph():
    w = wl.WORKLOADS["zipf1.1_4096_v32000_h4096"]
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg0 = wl.make_main_grad(w, "cuda")[:16000]
    ws = ewg.new_workspace(ids.numel(), w.hidden, "cuda")
    _replays_match_eager(
        lambda i, g, m, wsp: ewg.accumulate_embedding_wgrad_vocab_shard(i, g, m, 0, workspace=wsp),
        ids, grad, mg0, ws)


def test_many_token_call_in_a_graph():
    rng = np.random.default_rng(3)
    n, vocab, hidden = 20000, 9000, 1024
    ids = torch.from_numpy(wl.zipf_ids(rng, n, vocab, 1.1)).cuda()
    grad = wl.normal_tensor(rng, (n, hidden), 0.01, "bf16").cuda()
    mg0 = wl.normal_tensor(rng, (vocab, hidden), 1e-3, "fp32").cuda()
    ws = ewg.new_many_tokens_workspace(n, hidden, "cuda")
    _replays_match_eager(
        lambda i, g, m, wsp: ewg.accumulate_embedding_wgrad_many_tokens(i, g, m, workspace=wsp),
        ids, grad, mg0, ws)
