"""The entry point that allocates nothing (accumulate_embedding_wgrad_no_alloc:
the library's static per-device scratch serves as the workspace), called
through the C ABI and compared bit for bit with accumulate_embedding_wgrad on
a workspace of its own, on two calls in a row, the second with a smaller
input, so that the second call starts from what the first left in the
scratch. The arithmetic both follow is the page's (Megatron-Core API docs,
"core.fusions.fused_embedding_wgrad", introduction); the one-kernel path's
parity with the oracle is tested elsewhere.
"""
import pytest
import torch

import workloads as wl
from parity_util import _bits

pytestmark = pytest.mark.gpu

# a missing or unloadable library fails the module (no skip)
import sparse_embedding_weight_amd as ewg  # noqa: E402
from sparse_embedding_weight_amd import _binding as B  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield


def no_alloc_equals_workspace_call(name):
    w = wl.WORKLOADS[name]
    print(f"[no-alloc] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    ref = mg.clone()
    ws = ewg.new_workspace(w.num_tokens, w.hidden, "cuda")
    ewg.accumulate_embedding_wgrad(ids, grad, ref, workspace=ws, checked=True)
    ewg.accumulate_embedding_wgrad_no_alloc(ids, grad, mg)
    torch.cuda.synchronize()
    assert torch.equal(_bits(mg), _bits(ref)), f"{name}: no-alloc result differs"


@pytest.mark.parametrize("first,second", [
    ("zipf1.1_8192_v129280_h7168", "uniform3073_v512_h128"),
    ("zipf1.3_4x2048_v129280_h7168_bf16mg", "zipf1.1_4096_v32000_h4096"),
])
def test_no_alloc_matches_workspace_call_twice(first, second):
    for name in (first, second):
        no_alloc_equals_workspace_call(name)


def test_no_alloc_rejects_bad_arguments_without_touching_main_grad():
    """Arguments the call rejects (an unsupported token count, a stride below hidden)
    return their status before anything is enqueued: main_grad keeps its bits."""
    n, hidden = 8192, 256
    ids = torch.randint(0, 100, (n,), dtype=torch.int32, device="cuda")
    grad = torch.randn(n, hidden, device="cuda").to(torch.bfloat16)
    mg = torch.randn(100, hidden, device="cuda")
    before = mg.clone()
    stream = torch.cuda.current_stream().cuda_stream
    f = B.lib.accumulate_embedding_wgrad_no_alloc
    assert f(ids.data_ptr(), grad.data_ptr(), mg.data_ptr(), 3072, hidden, 100, hidden, hidden,
             B.EWG_INT32, B.EWG_BF16, B.EWG_FP32, stream) == B.EWG_UNSUPPORTED
    assert f(ids.data_ptr(), grad.data_ptr(), mg.data_ptr(), n, hidden, 100, hidden - 1, hidden,
             B.EWG_INT32, B.EWG_BF16, B.EWG_FP32, stream) == B.EWG_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.equal(_bits(mg), _bits(before))
    with pytest.raises(ValueError):
        ewg.accumulate_embedding_wgrad_no_alloc(ids, grad.t(), mg)
