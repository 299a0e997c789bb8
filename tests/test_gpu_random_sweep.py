"""GPU parity over a seeded random sweep of shapes and types, both entry points.

Each case draws a token count, a table size, a hidden size (often ragged), the
grad and main_grad dtypes, the ids dtype, an id law (uniform, Zipf with a
random exponent, or a few hot ids over a uniform background) and row strides
with or without padding; the library's result is compared with the oracle's
bit for bit on the touched rows, and untouched rows must not change.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import assert_rows_match

pytestmark = pytest.mark.gpu

# a missing or unloadable library fails the module (no skip)
import sparse_embedding_weight_amd as ewg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield


def _draw_case(rng, n_lo, n_hi, vocab_hi):
    n = int(rng.integers(n_lo, n_hi + 1))
    vocab = int(rng.integers(1, vocab_hi + 1))
    hidden = int(rng.choice([1, 3, 64, 100, 511, 512, 513, 1000, 2048, 3000]))
    gd, md = rng.choice(["bf16", "fp32"]), rng.choice(["bf16", "fp32"])
    ids_dtype = torch.int64 if rng.random() < 0.3 else torch.int32
    law = rng.choice(["uniform", "zipf", "hot"])
    if law == "uniform":
        ids = rng.integers(0, vocab, size=n)
    elif law == "zipf":
        ids = wl.zipf_ids(rng, n, vocab, float(rng.uniform(0.8, 1.6)))
    else:   # a few hot ids (runs far longer than 10) over a uniform background
        ids = rng.integers(0, vocab, size=n)
        hot = rng.integers(0, vocab, size=int(rng.integers(1, 4)))
        mask = rng.random(n) < 0.5
        ids[mask] = rng.choice(hot, size=int(mask.sum()))
    pad_g = int(rng.choice([0, 0, 8, 5]))
    pad_m = int(rng.choice([0, 0, 8, 3]))
    return n, vocab, hidden, gd, md, ids_dtype, np.asarray(ids), pad_g, pad_m


def _tensors(rng, n, vocab, hidden, gd, md, ids_dtype, ids, pad_g, pad_m):
    ids_t = torch.from_numpy(ids).to(ids_dtype).cuda()
    g_full = wl.normal_tensor(rng, (n, hidden + pad_g), 0.01, gd).cuda()
    m_full = wl.normal_tensor(rng, (vocab, hidden + pad_m), 1e-3, md).cuda()
    return ids_t, g_full[:, :hidden], m_full[:, :hidden]


def _run(call, ids, grad, mg):
    rows = torch.unique(ids.reshape(-1).long())
    before_rows = mg[rows].clone()
    before = mg.clone()
    call(ids, grad, mg)
    torch.cuda.synchronize()
    assert_rows_match(ids, grad, mg, before, rows, before_rows)


@pytest.mark.parametrize("case", range(48))
def test_random_one_kernel_path(case):
    rng = np.random.default_rng(1000 + case)
    n, vocab, hidden, gd, md, idt, ids, pg, pm = _draw_case(rng, ewg.MIN_TOKENS, ewg.MAX_TOKENS, 200000)
    # the one-kernel path's 31-bit packing bound
    pb = ewg.position_bits(n)
    vocab = min(vocab, 1 << (31 - pb))
    ids = ids % vocab
    print(f"[random one-kernel] case {case}: n={n} vocab={vocab} hidden={hidden} {gd}->{md} "
          f"pads {pg},{pm}", flush=True)
    _run(ewg.accumulate_embedding_wgrad, *_tensors(rng, n, vocab, hidden, gd, md, idt, ids, pg, pm))


@pytest.mark.parametrize("case", range(16))
def test_random_many_token_path(case):
    rng = np.random.default_rng(2000 + case)
    n, vocab, hidden, gd, md, idt, ids, pg, pm = _draw_case(rng, ewg.MAX_TOKENS + 1, 40000,
                                                            ewg.MANY_MAX_EMBEDDINGS)
    print(f"[random many-token] case {case}: n={n} vocab={vocab} hidden={hidden} {gd}->{md} "
          f"pads {pg},{pm}", flush=True)
    _run(ewg.accumulate_embedding_wgrad_many_tokens,
         *_tensors(rng, n, vocab, hidden, gd, md, idt, ids, pg, pm))
