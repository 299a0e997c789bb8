"""GPU parity: the HIP library against the CPU oracle, bit for bit.

Every case runs the library through its C ABI (via the thin binding) on the
GPU, copies the touched main_grad rows back, runs the oracle on the same
inputs and compares the bits. Rows whose id does not occur must be
bit-identical to a copy taken before the call. NaNs are compared as a class
(their payload is not part of the definition).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import _bits, assert_rows_match, oracle_rows  # noqa: F401

pytestmark = pytest.mark.gpu

# a missing or unloadable library fails the module (no skip)
import sparse_embedding_weight_amd as ewg  # noqa: E402
from sparse_embedding_weight_amd import _binding as B  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield


_SHARED_WS = {}


def shared_workspace(n: int, hidden: int) -> torch.Tensor:
    """One workspace reused by every call of this module (grown when needed), so
    the counters a call leaves behind are exercised by the next call."""
    need = ewg.workspace_bytes(n, hidden)
    ws = _SHARED_WS.get("ws")
    if ws is None or ws.numel() < need:
        ws = ewg.new_workspace(8192, max(hidden, 7232), "cuda")
        _SHARED_WS["ws"] = ws
    return ws


def check_call(ids: torch.Tensor, grad: torch.Tensor, main_grad: torch.Tensor, **kw):
    """Run one call on the GPU and compare with the oracle; returns the touched rows."""
    rows = torch.unique(ids.reshape(-1).long())
    before_rows = main_grad[rows].clone()
    before = main_grad.clone()
    ws = kw.pop("workspace", None)
    if ws is None:
        ws = shared_workspace(ids.numel(), grad.shape[-1])
    ewg.accumulate_embedding_wgrad(ids, grad, main_grad, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert ewg.wait_timeouts(ws) == 0, "a bounded wait inside the kernel gave up"

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


# ---- the five workloads at full size, in the launch configuration the benchmark times ----

@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_workload_full_size_bit_exact(name):
    w = wl.WORKLOADS[name]
    print(f"[parity] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    rows = check_call(ids, grad, mg)
    assert rows.numel() == np.unique(wl.make_ids(w)).size


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_matches_torch_dense_embedding_backward(name):
    """A second, external reference: PyTorch-ROCm's aten::embedding_dense_backward
    followed by main_grad.add_, the routine whose result, per the page's introduction,
    the fused path matches once a call has over 3072 tokens. On the touched rows the two
    agree bit for bit (NaNs compared as a class); rows of absent ids are not compared,
    since the dense path adds +0 to them."""
    w = wl.WORKLOADS[name]
    print(f"[dense reference] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w).reshape(-1)).cuda()
    grad = wl.make_grad(w).reshape(w.num_tokens, w.hidden).cuda()
    mg0 = wl.make_main_grad(w, "cuda")
    ours = mg0.clone()
    ewg.accumulate_embedding_wgrad(ids, grad, ours, workspace=shared_workspace(w.num_tokens, w.hidden))
    gw = torch.ops.aten.embedding_dense_backward(grad, ids.long(), w.vocab, -1, False)
    dense = mg0.add_(gw)
    torch.cuda.synchronize()
    rows = torch.unique(ids.long())
    a, b = ours[rows], dense[rows]
    both_nan = torch.isnan(a) & torch.isnan(b)
    mism = (_bits(a) != _bits(b)) & ~both_nan
    assert int(mism.sum()) == 0, f"{int(mism.sum())} elements differ from the dense path"


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_workload_sort_tables_exact(name):
    w = wl.WORKLOADS[name]
    ids_np = wl.make_ids(w)
    got = ewg.sort_tokens(torch.from_numpy(ids_np).cuda(), w.vocab)
    want = oracle.sort_tokens(ids_np)
    for k in want:
        assert np.array_equal(got[k].cpu().numpy().astype(np.int64), want[k]), k


# ---- edge cases ---------------------------------------------------------------

@pytest.mark.parametrize("n", [3073, 4096, 4097, 8192])
@pytest.mark.parametrize("hidden", [1, 7, 129, 1000])
def test_token_counts_and_ragged_hidden(n, hidden):
    print(f"[parity] n={n} hidden={hidden}", flush=True)
    check_call(*make_case(n, 700, hidden, seed=n + hidden))


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mg_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("hidden", [8, 1024, 7169])
def test_dtype_pairs(grad_dtype, mg_dtype, hidden):
    print(f"[parity] {grad_dtype}/{mg_dtype} hidden={hidden}", flush=True)
    rng = np.random.default_rng(hidden)
    ids = wl.zipf_ids(rng, 8192, 5000, 1.1)
    check_call(*make_case(8192, 5000, hidden, grad_dtype, mg_dtype, ids=ids, seed=hidden))


@pytest.mark.parametrize("hidden", [64, 1000])
def test_all_same_id(hidden):
    # one run of 8192 rows = 820 chunks in the ordered combine
    check_call(*make_case(8192, 50, hidden, ids=np.full(8192, 37), seed=1))


def test_all_distinct_ids():
    rng = np.random.default_rng(2)
    check_call(*make_case(8192, 20000, 300, ids=rng.permutation(20000)[:8192], seed=2))


def test_single_row_vocabulary():
    # num_embeddings = 1: no id bits, the sort has no pass
    check_call(*make_case(5000, 1, 96, ids=np.zeros(5000, dtype=np.int64), seed=3))


@pytest.mark.parametrize("n,vocab", [(8192, 1 << 18), (4096, 1 << 19)])
def test_largest_packable_vocabulary(n, vocab):
    # the largest ids that pack with the position into 31 bits; two 10/9-bit passes
    rng = np.random.default_rng(4)
    ids = rng.integers(vocab - 3000, vocab, size=n)
    ids[:5] = vocab - 1
    ids[5:9] = 0
    check_call(*make_case(n, vocab, 8, ids=ids, seed=4))


def test_int64_ids_and_2d_ids():
    rng = np.random.default_rng(5)
    ids = wl.zipf_ids(rng, 8192, 129280, 1.3)
    check_call(*make_case(8192, 129280, 256, ids=ids, seed=5, ids_dtype=torch.int64,
                          shape=(4, 2048)))


@pytest.mark.parametrize("grad_dtype,mg_dtype", [("bf16", "fp32"), ("fp32", "bf16")])
@pytest.mark.parametrize("pad_g,pad_m", [(8, 8), (5, 3), (0, 1)])
def test_padded_row_strides(grad_dtype, mg_dtype, pad_g, pad_m):
    # aligned padding keeps the 16-byte path; odd padding takes the element path
    n, vocab, hidden = 4097, 900, 520
    ids, grad, mg = make_case(n, vocab, hidden, grad_dtype, mg_dtype, seed=6 + pad_g)
    gbig = torch.zeros(n, hidden + pad_g, dtype=grad.dtype, device="cuda")
    gbig[:, :hidden] = grad
    mbig = torch.full((vocab, hidden + pad_m), 7.0, dtype=mg.dtype, device="cuda")
    mbig[:, :hidden] = mg
    check_call(ids, gbig[:, :hidden], mbig[:, :hidden])
    assert torch.all(mbig[:, hidden:] == 7.0)


def test_special_values():
    n, vocab, hidden = 4096, 300, 64
    ids, grad, mg = make_case(n, vocab, hidden, "fp32", "fp32", seed=7)
    grad[0:40] = 0.0
    grad[40:80] = -0.0
    grad[80:90, 3] = float("inf")
    grad[90:95, 5] = float("-inf")
    grad[95:99, 7] = float("nan")
    grad[100:200] *= 1e-38                      # denormal range
    mg[ids[40:80].long()] = -0.0
    mg[ids[300:310].long(), 2] = float("nan")
    check_call(ids, grad, mg)


def test_bf16_special_values():
    n, vocab, hidden = 4096, 300, 64
    ids, grad, mg = make_case(n, vocab, hidden, "bf16", "bf16", seed=8)
    grad[40:80] = -0.0
    grad[80:90, 3] = float("inf")
    grad[95:99, 7] = float("nan")
    grad[100:200] *= 1e-38
    mg[ids[40:80].long()] = -0.0
    check_call(ids, grad, mg)


def test_non_contiguous_grad_view():
    n, vocab, hidden = 4096, 500, 128
    ids, grad, mg = make_case(n, vocab, 2 * hidden, seed=9)
    check_call(ids, grad[:, ::2], mg[:, :hidden].contiguous())


def test_repeatable_bitwise():
    ids, grad, mg = make_case(8192, 3000, 512, seed=10)
    a, b = mg.clone(), mg.clone()
    ewg.accumulate_embedding_wgrad(ids, grad, a)
    ewg.accumulate_embedding_wgrad(ids, grad, b)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))


def test_workspace_reuse_across_shapes():
    # one workspace through calls of different sizes, types and run structure
    # (its counters and flag must be left clean by every call)
    ws = ewg.new_workspace(8192, 2048, "cuda")
    rng = np.random.default_rng(13)
    cases = [
        (8192, 40, 2048, "bf16", "fp32", wl.zipf_ids(rng, 8192, 40, 1.1)),     # all runs long
        (4097, 5000, 100, "fp32", "bf16", None),                               # mostly short runs
        (8192, 20000, 1024, "bf16", "bf16", rng.permutation(20000)[:8192]),    # no long run
        (3073, 3, 7, "fp32", "fp32", None),                                     # 3 long runs, ragged
        (8192, 129280, 2048, "bf16", "fp32", wl.zipf_ids(rng, 8192, 129280, 1.1)),
    ]
    for i, (n, vocab, hidden, gd, md, ids) in enumerate(cases * 2):
        print(f"[parity] reuse case {i}: n={n} vocab={vocab} hidden={hidden}", flush=True)
        check_call(*make_case(n, vocab, hidden, gd, md, ids=ids, seed=100 + i), workspace=ws)


def test_invalid_ids_change_nothing():
    # main_grad is an interior slice, so even a stray write would stay inside the
    # allocation and be seen in the guard rows
    n, vocab, hidden = 4096, 100, 32
    ids, grad, _ = make_case(n, vocab, hidden, seed=11)
    big = torch.randn(vocab + 2, hidden, device="cuda")
    mg = big[1:vocab + 1]
    before = big.clone()
    ws = ewg.new_workspace(n, hidden, "cuda")
    for bad in (vocab, -1):
        ids2 = ids.clone()
        ids2[17] = bad
        ids2[4000] = bad
        ewg.accumulate_embedding_wgrad(ids2, grad, mg, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(big), _bits(before))
        assert ewg.invalid_id_count(ws) == 2
    ewg.accumulate_embedding_wgrad(ids, grad, mg, workspace=ws)
    torch.cuda.synchronize()
    assert ewg.invalid_id_count(ws) == 0


def test_sort_tables_edge_ids():
    for ids_np, vocab in [(np.full(8192, 3), 4), (np.arange(8192)[::-1].copy(), 8192),
                          (np.zeros(3073, dtype=np.int64), 1),
                          (np.random.default_rng(12).integers(0, 1 << 19, 4096), 1 << 19)]:
        got = ewg.sort_tokens(torch.from_numpy(ids_np).cuda(), vocab)
        want = oracle.sort_tokens(ids_np)
        for k in want:
            assert np.array_equal(got[k].cpu().numpy().astype(np.int64), want[k]), k


# ---- vocabulary shards: each shard's rows equal the unsharded result, bit for bit ----

def _shard_calls(ids, grad, mg, bounds, ws=None):
    """Run the shard entry point once per [bounds[k], bounds[k+1]) on views of mg."""
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if hi > lo:
            ewg.accumulate_embedding_wgrad_vocab_shard(ids, grad, mg[lo:hi], lo, workspace=ws)
    torch.cuda.synchronize()


def _check_against_oracle(ids, grad, before, after):
    rows = torch.unique(ids.reshape(-1).long())
    assert_rows_match(ids, grad, after, before, rows, before[rows].clone())


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_vocab_shards_equal_unsharded(name):
    """Three shards of uneven size cover the vocabulary; together they give the
    unsharded result (the oracle's) on every touched row and leave the rest."""
    w = wl.WORKLOADS[name]
    print(f"[shard parity] workload {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    before = mg.clone()
    v = w.vocab
    bounds = [0, v // 7 + 3, (5 * v) // 8, v]
    _shard_calls(ids, grad, mg, bounds, ws=shared_workspace(ids.numel(), w.hidden))
    _check_against_oracle(ids, grad, before, mg)


def test_vocab_shard_edges():
    """Shards with no id, a shard of a single row, a power-of-two shard whose last row
    is used (the extra id bit), int64 ids far above 2^32, and the hottest id alone."""
    rng = np.random.default_rng(71)
    n, hidden = 4097, 136
    base = 1 << 40
    ids_np = rng.integers(0, 1 << 16, size=n)
    ids_np[rng.choice(n, 900, replace=False)] = (1 << 16) - 1      # hot id on the last row
    ids_np[:5] = 3                                                  # a run of 5 on row 3
    ids_t = torch.from_numpy(ids_np + base).to(torch.int64).cuda()
    grad = wl.normal_tensor(rng, (n, hidden), 0.01, "bf16").cuda()
    mg = wl.normal_tensor(rng, (1 << 16, hidden), 1e-3, "fp32").cuda()
    before = mg.clone()
    ws = ewg.new_workspace(n, hidden, "cuda")
    # an empty shard above every id, then a power-of-two shard of all rows
    empty = torch.zeros(10, hidden, dtype=torch.float32, device="cuda")
    ewg.accumulate_embedding_wgrad_vocab_shard(ids_t, grad, empty, base + (1 << 16), workspace=ws)
    ewg.accumulate_embedding_wgrad_vocab_shard(ids_t, grad, mg, base, workspace=ws)
    torch.cuda.synchronize()
    assert not empty.any()
    _check_against_oracle(ids_t - base, grad, before, mg)
    # the same result from single-row shards around the run and the hot id
    mg2 = before.clone()
    bounds = [0, 3, 4, (1 << 16) - 1, 1 << 16]
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        ewg.accumulate_embedding_wgrad_vocab_shard(ids_t, grad, mg2[lo:hi], base + lo, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(mg2), _bits(mg))


def test_vocab_shard_quick_check_boundary():
    """A shard call that keeps at most 2048 positions checks whether any id has more
    than 10 of them and skips the sort when none has: ids on exactly 10 and 11
    positions, and hot ids on 2000 and on 2049 positions, in single-row shards and
    inside wider ones, all equal to the oracle."""
    rng = np.random.default_rng(73)
    n, hidden, v = 6000, 72, 1 << 15
    ids_np = rng.integers(1000, v, size=n)
    perm = rng.permutation(n)
    ids_np[perm[:10]] = 100            # 10 rows: one chunk, no long run
    ids_np[perm[10:21]] = 200          # 11 rows: the smallest long run
    ids_np[perm[21:2021]] = 300        # 2000 kept positions: checked, long
    ids_np[perm[2021:4070]] = 400      # 2049 kept positions: above the check, sorted
    print("[shard quick check] n=6000 hidden=72", flush=True)
    ids_t = torch.from_numpy(ids_np).to(torch.int32).cuda()
    grad = wl.normal_tensor(rng, (n, hidden), 0.01, "bf16").cuda()
    mg = wl.normal_tensor(rng, (v, hidden), 1e-3, "fp32").cuda()
    before = mg.clone()
    ws = ewg.new_workspace(n, hidden, "cuda")
    _shard_calls(ids_t, grad, mg, [0, 100, 101, 200, 201, 300, 301, 400, 401, 1000, v], ws=ws)
    assert ewg.wait_timeouts(ws) == 0
    _check_against_oracle(ids_t, grad, before, mg)
    mg2 = before.clone()
    _shard_calls(ids_t, grad, mg2, [0, 150, 250, 350, 1000, v], ws=ws)
    assert torch.equal(_bits(mg2), _bits(mg))


# ---- launch sizes: few workgroups (long shares, many rounds) and more than fit at once ----

def test_timed_entry_point_matches_plain_calls():
    """accumulate_embedding_wgrad_timed, with the kernel's own events (4 events)
    and with plain dispatches (events 2 and 3 NULL), adds exactly what the plain
    entry point adds, and the events it records bound the kernel's own."""
    import ctypes
    from sparse_embedding_weight_amd import _binding as B
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    w = wl.WORKLOADS["zipf1.1_4096_v32000_h4096"]
    ids = torch.from_numpy(wl.make_ids(w)).cuda().reshape(-1)
    grad = wl.make_grad(w).cuda().reshape(ids.numel(), w.hidden)
    mg0 = wl.make_main_grad(w, "cuda")
    ws = ewg.new_workspace(ids.numel(), w.hidden, "cuda")
    plain = mg0.clone()
    ewg.accumulate_embedding_wgrad(ids, grad, plain, workspace=ws)
    torch.cuda.synchronize()
    evs = []
    for _ in range(4):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h.value)
    stream = torch.cuda.current_stream().cuda_stream
    try:
        for kernel_events in (True, False):
            mg = mg0.clone()
            slots = (ctypes.c_void_p * 4)(*(evs if kernel_events else evs[:2] + [None, None]))
            st = B.lib.accumulate_embedding_wgrad_timed(
                ids.data_ptr(), grad.data_ptr(), mg.data_ptr(), ids.numel(), w.hidden, w.vocab,
                grad.stride(0), mg.stride(0), B.DTYPE_CODE[ids.dtype], B.DTYPE_CODE[grad.dtype],
                B.DTYPE_CODE[mg.dtype], ws.data_ptr(), ws.numel(), stream, slots)
            assert st == 0
            torch.cuda.synchronize()
            assert torch.equal(_bits(mg), _bits(plain)), f"kernel_events={kernel_events}"
            call = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(call), evs[0], evs[1]) == 0
            assert 0.0 < call.value < 1000.0
            if kernel_events:
                kern = ctypes.c_float()
                assert hip.hipEventElapsedTime(ctypes.byref(kern), evs[2], evs[3]) == 0
                assert 0.0 < kern.value <= call.value
    finally:
        for e in evs:
            hip.hipEventDestroy(e)
    assert ewg.wait_timeouts(ws) == 0


@pytest.mark.parametrize("grid", ["2", "3", "16", "2x", "3x"])
@pytest.mark.parametrize("name", ["zipf1.1_4096_v32000_h4096", "longrun_8192_v129280_h7168"])
def test_launch_sizes(grid, name):
    """The test entry point sets the workgroups of a launch. With 2, 3 or 16 one
    follower handles many rounds of short runs and many column blocks of long
    runs; with two or three times the compute units, workgroups start as others
    finish and find fewer blocks left (or none). The result stays bit-exact and
    no bounded wait gives up."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = int(grid[:-1]) * cus if grid.endswith("x") else int(grid)
    w = wl.WORKLOADS[name]
    print(f"[launch size] {name} grid {g}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    ws = ewg.new_workspace(ids.numel(), w.hidden, "cuda")
    rows = torch.unique(ids.reshape(-1).long())
    before_rows, before = mg[rows].clone(), mg.clone()
    B.accumulate_with_grid_for_tests(ids, grad, mg, ws, g)
    torch.cuda.synchronize()
    assert ewg.wait_timeouts(ws) == 0
    assert_rows_match(ids, grad, mg, before, rows, before_rows)


@pytest.mark.parametrize("name", ["zipf1.1_8192_v129280_h7168", "longrun_8192_v129280_h7168",
                                  "zipf1.3_4x2048_v129280_h7168_bf16mg"])
def test_long_blocks_taken_by_fewer_workgroups(name):
    """The test entry point keeps every odd workgroup out of the long-run phase, as
    workgroups that start after the ticket ran out would be: the even ones take
    every column block from the shared ticket. Bit-exact, and no wait gives up."""
    w = wl.WORKLOADS[name]
    print(f"[long blocks, odd workgroups out] {name}", flush=True)
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    ws = ewg.new_workspace(ids.numel(), w.hidden, "cuda")
    rows = torch.unique(ids.reshape(-1).long())
    before_rows, before = mg[rows].clone(), mg.clone()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B.accumulate_with_grid_for_tests(ids, grad, mg, ws, cus, odd_skip_long=True)
    torch.cuda.synchronize()
    assert ewg.wait_timeouts(ws) == 0
    assert_rows_match(ids, grad, mg, before, rows, before_rows)


def test_checked_call_passes_and_leaves_the_word():
    """The checked mode synchronises after the call and raises only when a wait
    gave up; a normal call leaves the word unchanged."""
    w = wl.WORKLOADS["uniform3073_v512_h128"]
    ids = torch.from_numpy(wl.make_ids(w)).cuda()
    grad = wl.make_grad(w).cuda()
    mg = wl.make_main_grad(w, "cuda")
    ws = ewg.new_workspace(ids.numel(), w.hidden, "cuda")
    rows = torch.unique(ids.reshape(-1).long())
    before_rows, before = mg[rows].clone(), mg.clone()
    ewg.accumulate_embedding_wgrad(ids, grad, mg, workspace=ws, checked=True)
    assert ewg.wait_timeouts(ws) == 0
    assert_rows_match(ids, grad, mg, before, rows, before_rows)
