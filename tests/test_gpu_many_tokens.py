"""GPU parity of the many-token entry point (more tokens than one LDS sort
holds): the HIP library against the CPU oracle, bit for bit, and against the
one-kernel entry point where both apply.

The arithmetic does not depend on the token count (Megatron-Core API docs,
"core.fusions.fused_embedding_wgrad", introduction): the same chunks of 10
rows counted from each id's first position, the same ordered combine. The
cases cover runs that span several tiles of 8192 positions, a ragged last
tile, the largest token count and vocabulary, and the degenerate runs (one id
everywhere, every id once, a one-row table).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import _bits, assert_rows_match

pytestmark = pytest.mark.gpu

# a missing or unloadable library fails the module (no skip)
import sparse_embedding_weight_amd as ewg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield


def check_many(ids, grad, main_grad, workspace=None):
    """One many-token call on the GPU, compared with the oracle; returns the touched rows."""
    rows = torch.unique(ids.reshape(-1).long())
    before_rows = main_grad[rows].clone()
    before = main_grad.clone()
    ewg.accumulate_embedding_wgrad_many_tokens(ids, grad, main_grad, workspace=workspace)
    torch.cuda.synchronize()
    assert_rows_match(ids, grad, main_grad, before, rows, before_rows)
    return rows


def make_case(n, vocab, hidden, grad_dtype="bf16", mg_dtype="fp32", ids=None, seed=0,
              ids_dtype=torch.int32, shape=None):
    rng = np.random.default_rng(seed)
    if ids is None:
        ids = rng.integers(0, vocab, size=n)
    ids = torch.from_numpy(np.asarray(ids).reshape(shape or (n,))).to(ids_dtype).cuda()
    grad = wl.normal_tensor(rng, (*ids.shape, hidden), 0.01, grad_dtype).cuda()
    mg = wl.normal_tensor(rng, (vocab, hidden), 1e-3, mg_dtype).cuda()
    return ids, grad, mg


# ---- the many-token workloads at full size --------------------------------------

@pytest.mark.parametrize("name", list(wl.MANY_WORKLOADS))
def test_many_workload_full_size_bit_exact(name):
    w = wl.MANY_WORKLOADS[name]
    print(f"[many] workload {name}", flush=True)
    ids_np = wl.make_ids(w)
    ids = torch.from_numpy(ids_np).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    rows = check_many(ids, grad, mg)
    assert rows.numel() == np.unique(ids_np).size


@pytest.mark.parametrize("name", list(wl.MANY_WORKLOADS))
def test_many_matches_torch_dense_embedding_backward(name):
    """PyTorch-ROCm's aten::embedding_dense_backward + main_grad.add_ at these token
    counts: bit for bit on the touched rows (NaNs compared as a class)."""
    w = wl.MANY_WORKLOADS[name]
    print(f"[many dense reference] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w).reshape(-1)).cuda()
    grad = wl.make_grad(w).reshape(w.num_tokens, w.hidden).cuda()
    mg0 = wl.make_main_grad(w, "cuda")
    ours = mg0.clone()
    ewg.accumulate_embedding_wgrad_many_tokens(ids, grad, ours)
    gw = torch.ops.aten.embedding_dense_backward(grad, ids.long(), w.vocab, -1, False)
    dense = mg0.add_(gw)
    del gw
    torch.cuda.synchronize()
    rows = torch.unique(ids.long())
    a, b = ours[rows], dense[rows]
    both_nan = torch.isnan(a) & torch.isnan(b)
    mism = (_bits(a) != _bits(b)) & ~both_nan
    assert int(mism.sum()) == 0, f"{int(mism.sum())} elements differ from the dense path"


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_many_equals_one_kernel_path(name):
    """Where both entry points apply (up to 8192 tokens) they give the same bits
    on the whole of main_grad."""
    w = wl.WORKLOADS[name]
    print(f"[many vs one-kernel] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    a = wl.make_main_grad(w, "cuda")
    b = a.clone()
    ewg.accumulate_embedding_wgrad(ids, grad, a)
    ewg.accumulate_embedding_wgrad_many_tokens(ids, grad, b)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))


# ---- sizes, types and layouts ---------------------------------------------------

@pytest.mark.parametrize("n", [8193, 12289, 16384, 65537])
@pytest.mark.parametrize("hidden", [1, 7, 129, 1000])
def test_many_token_counts_and_ragged_hidden(n, hidden):
    # 3000 ids: most runs span several tiles and have more than 10 rows
    print(f"[many] n={n} hidden={hidden}", flush=True)
    rng = np.random.default_rng(n + hidden)
    ids = wl.zipf_ids(rng, n, 3000, 1.1)
    check_many(*make_case(n, 3000, hidden, ids=ids, seed=n * 7 + hidden))


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mg_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("hidden", [8, 1024, 7169])
def test_many_dtype_pairs(grad_dtype, mg_dtype, hidden):
    rng = np.random.default_rng(hidden)
    ids = wl.zipf_ids(rng, 20000, 9000, 1.2)
    check_many(*make_case(20000, 9000, hidden, grad_dtype, mg_dtype, ids=ids, seed=hidden + 1))


@pytest.mark.parametrize("n,hidden", [(131072, 64), (50000, 1000)])
def test_many_all_same_id(n, hidden):
    # one run through every tile: 13108 chunks at the largest size
    check_many(*make_case(n, 50, hidden, ids=np.full(n, 37), seed=1))


def test_many_all_distinct_ids_largest_vocabulary():
    # 131072 runs of one row; ids up to the largest table the entry point takes
    vocab = ewg.MANY_MAX_EMBEDDINGS
    rng = np.random.default_rng(2)
    ids = rng.permutation(vocab)[:ewg.MANY_MAX_TOKENS]
    ids[0] = vocab - 1
    check_many(*make_case(ewg.MANY_MAX_TOKENS, vocab, 8, ids=ids, seed=2))


def test_many_single_row_vocabulary():
    check_many(*make_case(20000, 1, 96, ids=np.zeros(20000, dtype=np.int64), seed=3))


def test_many_runs_ending_on_tile_edges():
    # runs whose rows end exactly at, just before and just after a tile edge,
    # and chunks that straddle it
    n = 3 * 8192 + 11
    ids = np.empty(n, dtype=np.int64)
    ids[:8192] = np.arange(8192) % 7           # ids 0..6, every tile
    ids[8192:16384] = 7 + (np.arange(8192) % 3)
    ids[16384:] = np.arange(n - 16384) % 11
    ids[8191] = 20                             # one-row run at the end of tile 0
    ids[8192] = 20                             # continued at the start of tile 1
    check_many(*make_case(n, 21, 200, ids=ids, seed=4))


def test_many_int64_and_2d_ids():
    rng = np.random.default_rng(5)
    ids = wl.zipf_ids(rng, 3 * 7000, 5000, 1.1)
    check_many(*make_case(21000, 5000, 300, ids=ids, ids_dtype=torch.int64, shape=(3, 7000),
                          seed=5))


@pytest.mark.parametrize("grad_dtype,mg_dtype", [("bf16", "fp32"), ("fp32", "bf16")])
@pytest.mark.parametrize("pad_g,pad_m", [(8, 8), (5, 3)])
def test_many_padded_row_strides(grad_dtype, mg_dtype, pad_g, pad_m):
    n, vocab, hidden = 17000, 4000, 520
    rng = np.random.default_rng(6)
    ids = torch.from_numpy(wl.zipf_ids(rng, n, vocab, 1.1)).cuda()
    g_full = wl.normal_tensor(rng, (n, hidden + pad_g), 0.01, grad_dtype).cuda()
    m_full = wl.normal_tensor(rng, (vocab, hidden + pad_m), 1e-3, mg_dtype).cuda()
    grad, mg = g_full[:, :hidden], m_full[:, :hidden]
    before_full = m_full.clone()
    check_many(ids, grad, mg)
    # the padding columns are never written
    assert torch.equal(_bits(m_full[:, hidden:]), _bits(before_full[:, hidden:]))


def test_many_repeatable_and_workspace_reuse():
    ws = ewg.new_many_tokens_workspace(40000, 2048, "cuda")
    ids, grad, mg = make_case(40000, 6000, 2048, seed=7)
    a, b = mg.clone(), mg.clone()
    ewg.accumulate_embedding_wgrad_many_tokens(ids, grad, a, workspace=ws)
    ewg.accumulate_embedding_wgrad_many_tokens(ids, grad, b, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))
    # smaller calls after a larger one through the same (uncleared) workspace
    for i, (n, vocab, hidden) in enumerate([(9000, 50, 100), (8193, 20000, 2048), (40000, 3, 17)]):
        print(f"[many] reuse case {i}: n={n} vocab={vocab} hidden={hidden}", flush=True)
        check_many(*make_case(n, vocab, hidden, seed=20 + i), workspace=ws)


def test_many_invalid_ids_change_nothing():
    n, vocab, hidden = 20000, 100, 32
    ids, grad, _ = make_case(n, vocab, hidden, seed=11)
    big = torch.randn(vocab + 2, hidden, device="cuda")
    mg = big[1:vocab + 1]
    before = big.clone()
    ws = ewg.new_many_tokens_workspace(n, hidden, "cuda")
    for bad in (vocab, -1):
        ids2 = ids.clone()
        ids2[17] = bad
        ids2[19999] = bad
        ewg.accumulate_embedding_wgrad_many_tokens(ids2, grad, mg, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(big), _bits(before))
        assert ewg.invalid_id_count(ws) == 2
    check_many(ids, grad, mg, workspace=ws)
    assert ewg.invalid_id_count(ws) == 0


def test_one_buffer_serves_both_paths():
    """One zero-filled buffer, large enough for both entry points, passed to the
    one-kernel path and the many-token path in turn: the many-token call leaves the
    one-kernel path's flags and counters alone, so every call stays bit-exact and
    no bounded wait gives up."""
    hidden = 512
    need = max(ewg.workspace_bytes(8192, hidden),
               ewg.many_tokens_workspace_bytes(20000, hidden))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i in range(2):
        print(f"[shared workspace] round {i}: one-kernel call", flush=True)
        ids, grad, mg = make_case(8192, 3000, hidden, seed=40 + i)
        rows = torch.unique(ids.long())
        before, before_rows = mg.clone(), mg[rows].clone()
        ewg.accumulate_embedding_wgrad(ids, grad, mg, workspace=ws, checked=True)
        torch.cuda.synchronize()
        assert_rows_match(ids, grad, mg, before, rows, before_rows)
        print(f"[shared workspace] round {i}: many-token call", flush=True)
        check_many(*make_case(20000, 5000, hidden, seed=50 + i), workspace=ws)
