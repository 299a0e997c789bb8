"""Pins of the CPU oracle against things other than itself.

Each test names what it pins and where that comes from on the Megatron-Core
API page "core.fusions.fused_embedding_wgrad" (introduction: the two bullets
and the sentence after them; the three kernel docstrings). A plausible
mistake in the oracle -- a dropped row, a wrong chunk boundary, a reversed
combine, a rounding at the wrong step, a touched row that should not be --
fails at least one of these.
"""
import os

import numpy as np
import pytest
import torch

import bruteforce
import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chunk_order.txt")


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def bits32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def encode(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values that are exact in `dtype` -> the oracle's input format."""
    x_f32 = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "bf16":
        b = bits32(x_f32)
        assert np.all(b & 0xFFFF == 0), "value not exact in bf16"
        return (b >> 16).astype(np.uint16)
    return x_f32.copy()


def random_problem(rng, n, vocab, hidden, grad_dtype, mg_dtype, ids_dtype=np.int32,
                   sigma=1.0):
    ids = rng.integers(0, vocab, size=n).astype(ids_dtype)
    grad = wl.to_numpy_bits(wl.normal_tensor(rng, (n, hidden), sigma, grad_dtype))
    mg = wl.to_numpy_bits(wl.normal_tensor(rng, (vocab, hidden), 0.1, mg_dtype))
    return ids, grad, mg


# --------------------------------------------------------------------------
# Rounding: fp32 -> bf16, round to nearest even (reading of "rounds once to
# the gradient dtype"), checked against torch's CPU conversion on every one of
# the 2^32 bit patterns. NaN inputs must give a NaN; the payload is not pinned.
# --------------------------------------------------------------------------

@pytest.mark.slow
def test_round_bf16_exhaustive_vs_torch():
    chunk = 1 << 26
    base = np.arange(chunk, dtype=np.uint32)
    out = np.empty(chunk, dtype=np.uint16)
    for start in range(0, 1 << 32, chunk):
        bits = base + np.uint32(start)
        ours = oracle.round_bf16_bits(bits, out)
        ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16)
        ref = ref.view(torch.int16).numpy().view(np.uint16)
        is_nan = (bits & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal((ours & 0x7FFF) > 0x7F80, is_nan), f"NaN class near {start:#x}"
        bad = (ours != ref) & ~is_nan
        assert not bad.any(), f"first mismatch at bits {bits[np.argmax(bad)]:#010x}"


def test_round_bf16_every_kept_half():
    """All 2^16 kept halves x the dropped halves that decide the rounding."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF, 0x1234], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    ours = oracle.round_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    is_nan = (bits & 0x7FFFFFFF) > 0x7F800000
    assert np.array_equal((ours & 0x7FFF) > 0x7F80, is_nan)
    assert np.array_equal(ours[~is_nan], ref[~is_nan])


def test_round_bf16_hand_cases():
    # ties to even, carries into the exponent, overflow to inf, denormals
    cases = {
        0x3F808000: 0x3F80,  # 1 + 2^-8: tie, kept part even -> down
        0x3F818000: 0x3F82,  # 1 + 3*2^-8: tie, kept part odd -> up
        0x3F808001: 0x3F81,  # just above the tie -> up
        0x3FFF8000: 0x4000,  # carry into the exponent
        0x7F7FFFFF: 0x7F80,  # largest finite fp32 -> inf
        0x00008000: 0x0000,  # denormal tie, even -> down
        0x00018000: 0x0002,  # denormal tie, odd -> up
        0x80000000: 0x8000,  # -0 stays -0
        0xFF800000: 0xFF80,  # -inf
    }
    for x, want in cases.items():
        assert oracle._load().oracle_round_bf16(x) == want, hex(x)


# --------------------------------------------------------------------------
# Sort tables: brute force without a sort (scan of the vocabulary) must give
# the same sorted order, run bounds, long-run list and chunk starts
# (_sort_tokens_kernel docstring; introduction, first bullet: ascending positions).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_sort_tables_vs_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 80))
    vocab = int(rng.integers(1, 9))
    ids = rng.integers(0, vocab, size=n).astype(np.int64 if seed % 2 else np.int32)
    got = oracle.sort_tokens(ids)
    want = bruteforce.sort_tables(ids, vocab)
    for key in want:
        assert np.array_equal(got[key], want[key]), key


# --------------------------------------------------------------------------
# Whole accumulation vs the sort-free brute force, all four dtype pairs, runs
# long enough to cross the 10-row chunk boundary several times.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mg_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed", range(3))
def test_accumulate_vs_bruteforce(grad_dtype, mg_dtype, seed):
    rng = np.random.default_rng(200 + seed)
    n, vocab, hidden = 64, 6, 5
    ids, grad, mg = random_problem(rng, n, vocab + 2, hidden, grad_dtype, mg_dtype)
    ids = np.minimum(ids, vocab - 1).astype(np.int32)   # make a few runs long
    want = bruteforce.accumulate(ids, widen(grad, grad_dtype), widen(mg, mg_dtype),
                                 grad_dtype, mg_dtype)
    got = mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, got, grad_dtype, mg_dtype)
    assert np.array_equal(bits32(widen(got, mg_dtype)), bits32(want))


# --------------------------------------------------------------------------
# Hand-computed chunk orders (tests/golden/chunk_order.txt).
# --------------------------------------------------------------------------

def _parse_value(tok: str) -> float:
    tok = tok.strip()
    sign = 1.0
    if tok.startswith("-"):
        sign, tok = -1.0, tok[1:]
    elif tok.startswith("+"):
        tok = tok[1:]
    total = 0.0
    for term in tok.split("+"):
        if term == "B":
            total += 2.0 ** 24
        elif "^" in term:
            base, exp = term.split("^")
            total += float(base) ** float(exp)
        else:
            total += float(term)
    return sign * total if total != 0 else (-0.0 if sign < 0 else 0.0)


def _parse_values(field: str):
    out = []
    for tok in field.split(","):
        if "*" in tok:
            v, k = tok.rsplit("*", 1)
            out += [_parse_value(v)] * int(k)
        else:
            out.append(_parse_value(tok))
    return out


def golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, gd, md, before, lead, values, expected, _wrong = [x.strip() for x in line.split("|")]
            cases.append(pytest.param(gd, md, _parse_value(before), int(lead),
                                      _parse_values(values), _parse_value(expected), id=name))
    return cases


@pytest.mark.parametrize("grad_dtype,mg_dtype,before,lead,values,expected", golden_cases())
def test_golden_chunk_order(grad_dtype, mg_dtype, before, lead, values, expected):
    # id 0: an earlier run of `lead` rows; id 1: the run under test; id 2: a
    # later run. Positions are shuffled so the run is not contiguous in ids.
    rng = np.random.default_rng(7)
    labels = [0] * lead + [1] * len(values) + [2] * 4
    perm = rng.permutation(len(labels))
    ids = np.empty(len(labels), dtype=np.int32)
    grad_vals = np.zeros(len(labels), dtype=np.float32)
    run_positions = sorted(perm[lead:lead + len(values)])
    for k, lab in enumerate(labels):
        ids[perm[k]] = lab
    for p, v in zip(run_positions, values):
        grad_vals[p] = v
    grad = encode(grad_vals.reshape(-1, 1), grad_dtype)
    mg_vals = np.array([[0.0], [before], [0.0]], dtype=np.float32)
    mg = encode(mg_vals, mg_dtype)
    oracle.accumulate_embedding_wgrad(ids, grad, mg, grad_dtype, mg_dtype)
    got = widen(mg, mg_dtype)[1, 0]
    assert bits32(np.array([got]))[0] == bits32(np.array([expected]))[0], (got, expected)
    # the sort-free brute force agrees as well
    bf = bruteforce.accumulate(ids, grad_vals.reshape(-1, 1), mg_vals, grad_dtype, mg_dtype)
    assert bits32(bf[1:2, 0])[0] == bits32(np.array([expected]))[0]


# --------------------------------------------------------------------------
# Closed forms.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mg_dtype", ["bf16", "fp32"])
def test_all_distinct_ids_closed_form(grad_dtype, mg_dtype):
    """Every run has one row: main_grad[v] = rnd_M(mg + rnd_G(0 + g)) element-wise
    (torch's own conversions and fp32 add)."""
    rng = np.random.default_rng(11)
    n, vocab, hidden = 300, 400, 33
    ids = rng.permutation(vocab)[:n].astype(np.int64)
    grad_t = wl.normal_tensor(rng, (n, hidden), 1.0, grad_dtype)
    mg_t = wl.normal_tensor(rng, (vocab, hidden), 0.5, mg_dtype)
    # put signed zeros in: -0 grad rows on a -0 main_grad
    grad_t[0] = -0.0
    mg_t[int(ids[0])] = -0.0
    got = wl.to_numpy_bits(mg_t).copy()
    oracle.accumulate_embedding_wgrad(ids, wl.to_numpy_bits(grad_t), got, grad_dtype, mg_dtype)

    want = mg_t.clone()
    idx = torch.from_numpy(ids)
    g = (torch.zeros(n, hidden) + grad_t.float()).to(wl.TORCH_DTYPE[grad_dtype]).float()
    want[idx] = (want[idx].float() + g).to(wl.TORCH_DTYPE[mg_dtype])
    assert np.array_equal(got, wl.to_numpy_bits(want))


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
def test_integer_grads_exact_vs_float64(grad_dtype):
    """Small integers: every fp32 add is exact (all partial sums < 2^24), so
    the result equals the float64 scatter-add (numpy.add.at) rounded once to the
    grad dtype and added to main_grad. Any dropped, doubled or misplaced row
    shows up here, independent of summation order."""
    rng = np.random.default_rng(12)
    n, vocab, hidden = 3073, 50, 17
    ids = rng.integers(0, vocab, size=n).astype(np.int32)
    gvals = rng.integers(-8, 9, size=(n, hidden)).astype(np.float32)
    if grad_dtype == "bf16":
        gvals[:, :] = np.clip(gvals, -8, 8)   # small integers are exact in bf16
    mvals = rng.integers(-1000, 1000, size=(vocab, hidden)).astype(np.float32)
    s = np.zeros((vocab, hidden), dtype=np.float64)
    np.add.at(s, ids, gvals.astype(np.float64))
    s32 = s.astype(np.float32)
    assert np.array_equal(s32.astype(np.float64), s)       # exact in fp32
    if grad_dtype == "bf16":
        s32 = torch.from_numpy(s32).to(torch.bfloat16).float().numpy()
    touched = np.zeros(vocab, dtype=bool)
    touched[ids] = True
    want = mvals.copy()
    want[touched] = (mvals[touched].astype(np.float64) + s32[touched]).astype(np.float32)
    got = mvals.copy()
    oracle.accumulate_embedding_wgrad(ids, encode(gvals, grad_dtype), got, grad_dtype, "fp32")
    assert np.array_equal(bits32(got), bits32(want))


# --------------------------------------------------------------------------
# Untouched rows: left bit-for-bit as they were, -0.0 and NaN payloads
# included (the sentence after the two bullets).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mg_dtype", ["bf16", "fp32"])
def test_untouched_rows_bit_identical(mg_dtype):
    rng = np.random.default_rng(13)
    n, vocab, hidden = 200, 64, 9
    ids = rng.integers(0, vocab // 2, size=n).astype(np.int32) * 2   # only even ids
    grad = wl.to_numpy_bits(wl.normal_tensor(rng, (n, hidden), 1.0, "bf16"))
    mg = wl.to_numpy_bits(wl.normal_tensor(rng, (vocab, hidden), 1.0, mg_dtype)).copy()
    specials = {"fp32": [0x80000000, 0x7FC01234, 0xFFA00001, 0x7F800000],
                "bf16": [0x8000, 0x7FC1, 0xFFA1, 0x7F80]}[mg_dtype]
    view = mg.view(np.uint32 if mg_dtype == "fp32" else np.uint16)
    for k, v in enumerate(specials):
        view[2 * k + 1, :] = v                     # odd rows: never touched
    before = mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, mg, "bf16", mg_dtype)
    odd = np.arange(1, vocab, 2)
    assert np.array_equal(mg[odd].view(np.uint8), before[odd].view(np.uint8))
    touched = np.unique(ids)
    assert not np.array_equal(mg[touched], before[touched])


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------

def test_relabeling_permutes_rows():
    rng = np.random.default_rng(14)
    n, vocab, hidden = 3073, 40, 12
    ids, grad, mg = random_problem(rng, n, vocab, hidden, "bf16", "fp32")
    perm = rng.permutation(vocab)
    a = mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, a, "bf16", "fp32")
    b = np.empty_like(mg)
    b[perm] = mg
    oracle.accumulate_embedding_wgrad(perm[ids].astype(np.int32), grad, b, "bf16", "fp32")
    assert np.array_equal(bits32(b[perm]), bits32(a))


def test_column_slices_are_independent():
    rng = np.random.default_rng(15)
    n, vocab, hidden = 3073, 30, 40
    ids, grad, mg = random_problem(rng, n, vocab, hidden, "fp32", "bf16")
    full = mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, full, "fp32", "bf16")
    for lo, hi in [(0, 7), (7, 8), (8, 40)]:
        part = np.ascontiguousarray(mg[:, lo:hi])
        oracle.accumulate_embedding_wgrad(ids, np.ascontiguousarray(grad[:, lo:hi]), part,
                                          "fp32", "bf16")
        assert np.array_equal(part, full[:, lo:hi])


@pytest.mark.parametrize("grad_dtype,mg_dtype", [("bf16", "fp32"), ("fp32", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("hidden,threads", [(7, 8), (40, 3), (100, 8), (257, 5), (64, 1)])
def test_column_blocks_equal_serial(grad_dtype, mg_dtype, hidden, threads):
    """The threaded timing entry (column blocks, one call of the C routine each, run at
    once) gives the serial call's bits, for ragged widths and more threads than columns."""
    rng = np.random.default_rng(18 + hidden)
    ids, grad, mg = random_problem(rng, 3100, 50, hidden, grad_dtype, mg_dtype)
    serial, blocked = mg.copy(), mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, serial, grad_dtype, mg_dtype)
    blocks = oracle.accumulate_embedding_wgrad_column_blocks(ids, grad, blocked, grad_dtype,
                                                             mg_dtype, threads)
    assert 1 <= blocks <= min(threads, hidden)
    assert np.array_equal(blocked.view(np.uint8), serial.view(np.uint8))


def test_row_strides_and_int64_ids():
    rng = np.random.default_rng(16)
    n, vocab, hidden = 500, 20, 10
    ids, grad, mg = random_problem(rng, n, vocab, hidden, "bf16", "fp32")
    a = mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, a, "bf16", "fp32")
    gpad = np.zeros((n, hidden + 6), dtype=grad.dtype)
    gpad[:, :hidden] = grad
    mpad = np.zeros((vocab, hidden + 3), dtype=mg.dtype)
    mpad[:, :hidden] = mg
    mpad[:, hidden:] = 99.0
    oracle.accumulate_embedding_wgrad(ids.astype(np.int64), gpad[:, :hidden],
                                      mpad[:, :hidden], "bf16", "fp32")
    assert np.array_equal(bits32(mpad[:, :hidden]), bits32(a))
    assert np.all(mpad[:, hidden:] == 99.0)


def test_repeatable():
    rng = np.random.default_rng(17)
    ids, grad, mg = random_problem(rng, 4096, 300, 16, "bf16", "bf16")
    a, b = mg.copy(), mg.copy()
    oracle.accumulate_embedding_wgrad(ids, grad, a, "bf16", "bf16")
    oracle.accumulate_embedding_wgrad(ids, grad, b, "bf16", "bf16")
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# fp64 agreement: the result is within the rounding-error bound of the exact
# sum. Per element, with S = sum of the run's grad values (fp64), L = run
# length, u = 2^-24, gamma = (L-1)u/(1-(L-1)u), A = |S| + gamma*sum|g|,
# u_G = 2^-8 for bf16 grad (0 for fp32), u_M = 2^-8 for a bf16 main_grad
# (2^-24 for fp32):
#   |out - (mg + S)| <= 1.01 [gamma*sum|g| + u_G*A + 2u_M(|mg| + A)] + 2^-126
# (summation error of any order of L-1 fp32 adds, one rounding to the grad
# dtype, the fp32 add and the rounding to main_grad's dtype).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["uniform3073_v512_h128", "longrun_small", "zipf_bf16mg_small"])
def test_fp64_error_bound(name):
    if name == "uniform3073_v512_h128":
        w = wl.WORKLOADS[name]
    elif name == "longrun_small":
        w = wl.Workload(name, (8192,), 129280, 24, "longrun", 0.0, "fp32", 1.0, "fp32", 1e-3, 4)
    else:
        w = wl.Workload(name, (4, 2048), 129280, 24, "zipf", 1.3, "bf16", 0.01, "bf16", 1e-3, 5)
    ids = wl.make_ids(w).reshape(-1)
    grad = wl.to_numpy_bits(wl.make_grad(w).reshape(w.num_tokens, w.hidden))
    rows = np.unique(ids)
    compact = np.searchsorted(rows, ids).astype(np.int32)    # order-preserving relabel
    mg_t = wl.normal_tensor(np.random.default_rng(w.seed), (rows.size, w.hidden),
                            w.main_grad_sigma, w.main_grad_dtype)
    mg = wl.to_numpy_bits(mg_t).copy()
    before = widen(mg, w.main_grad_dtype).astype(np.float64)
    oracle.accumulate_embedding_wgrad(compact, grad, mg, w.grad_dtype, w.main_grad_dtype)
    out = widen(mg, w.main_grad_dtype).astype(np.float64)

    g64 = widen(grad, w.grad_dtype).astype(np.float64)
    S = np.zeros_like(before)
    absum = np.zeros_like(before)
    np.add.at(S, compact, g64)
    np.add.at(absum, compact, np.abs(g64))
    L = np.bincount(compact, minlength=rows.size).astype(np.float64)[:, None]
    u = 2.0 ** -24
    gamma = (L - 1) * u / (1 - (L - 1) * u)
    uG = 2.0 ** -8 if w.grad_dtype == "bf16" else 0.0
    uM = 2.0 ** -8 if w.main_grad_dtype == "bf16" else u
    A = np.abs(S) + gamma * absum
    bound = 1.01 * (gamma * absum + uG * A + 2 * uM * (np.abs(before) + A)) + 2.0 ** -126
    err = np.abs(out - (before + S))
    assert np.all(err <= bound), float(np.max(err / bound))
    # and the bound is not vacuous: the error uses a fair part of it somewhere
    assert np.max(err / bound) > 1e-3
