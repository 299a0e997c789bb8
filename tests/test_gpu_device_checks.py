"""The one-kernel path built with its device-side bounds checks
(libembedding_wgrad_checked.so, -DEWG_DEVICE_CHECKS=1) on the GPU.

On the five generated workloads at full size and on the edge cases of the
sort (one id everywhere, every id distinct), the checked build must count no
failed check in the workspace word at EWG_WS_CHECK_FAILURES_OFFSET and give
main_grad bit-identical to the default build's. The checks clamp any index
that fails them, so the checked library accesses no memory out of bounds either way.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

# a missing or unloadable library fails the module (no skip)
import sparse_embedding_weight_amd as ewg  # noqa: E402
from sparse_embedding_weight_amd import _binding as B  # noqa: E402

CHECKED = os.path.join(os.path.dirname(B.LIBRARY), "libembedding_wgrad_checked.so")
CHECK_FAILURES_OFFSET = B.WS_CHECK_FAILURES_OFFSET


@pytest.fixture(scope="module")
def checked_lib():
    if not os.path.exists(CHECKED):
        raise FileNotFoundError(f"{CHECKED} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(CHECKED)
    lib.accumulate_embedding_wgrad.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 5 + \
        [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.accumulate_embedding_wgrad.restype = ctypes.c_int
    return lib


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield


def run_both(lib, ids, grad, mg):
    """main_grad after one call of the checked build, after one of the default
    build, and the checked build's failed-check count."""
    n, hidden = ids.numel(), grad.shape[-1]
    mg_checked, mg_default = mg.clone(), mg.clone()
    ws = torch.zeros(ewg.workspace_bytes(n, hidden), dtype=torch.uint8, device="cuda")
    st = lib.accumulate_embedding_wgrad(
        ids.data_ptr(), grad.data_ptr(), mg_checked.data_ptr(), n, hidden, mg.shape[0],
        grad.stride(-2), mg.stride(0), B.DTYPE_CODE[ids.dtype], B.DTYPE_CODE[grad.dtype],
        B.DTYPE_CODE[mg.dtype], ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == B.EWG_OK, st
    ewg.accumulate_embedding_wgrad(ids, grad, mg_default)
    torch.cuda.synchronize()
    failures = int(ws[CHECK_FAILURES_OFFSET:CHECK_FAILURES_OFFSET + 4].view(torch.int32).item())
    timeouts = int(ws[B.WS_WAIT_TIMEOUTS_OFFSET:B.WS_WAIT_TIMEOUTS_OFFSET + 4].view(torch.int32).item())
    return mg_checked, mg_default, failures, timeouts


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_checked_build_workloads(checked_lib, name):
    w = wl.WORKLOADS[name]
    print(f"[device checks] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    got, want, failures, timeouts = run_both(checked_lib, ids.reshape(-1), grad.reshape(-1, w.hidden), mg)
    assert failures == 0 and timeouts == 0
    assert torch.equal(bits(got), bits(want))


@pytest.mark.parametrize("kind", ["same", "distinct"])
def test_checked_build_sort_edges(checked_lib, kind):
    print(f"[device checks] {kind} ids", flush=True)
    rng = np.random.default_rng(5)
    n, vocab, hidden = 8192, 9000, 520
    ids_np = np.full(n, 17) if kind == "same" else rng.permutation(vocab)[:n]
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    grad = wl.normal_tensor(rng, (n, hidden), 0.01, "bf16").cuda()
    mg = wl.normal_tensor(rng, (vocab, hidden), 1e-3, "fp32").cuda()
    got, want, failures, timeouts = run_both(checked_lib, ids, grad, mg)
    assert failures == 0 and timeouts == 0
    assert torch.equal(bits(got), bits(want))
