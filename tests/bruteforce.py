"""Sort-free brute force of the embedding weight-gradient accumulation, for tiny inputs.

Test-side pin of the oracle; it shares no code with it. Where the oracle sorts
(id, position) pairs, this scans the vocabulary: for every id it walks the
positions 0..N-1 and collects the matches, which are in position order by
construction. Sums are numpy float32 element-wise adds (one IEEE binary32 add
each); rounding to bf16 is torch's CPU conversion, not the oracle's routine.

Arithmetic followed: Megatron-Core API docs, "core.fusions.fused_embedding_wgrad",
introduction (each id's rows by ascending position, cut into fp32-summed
chunks of ten or fewer; the chunk sums folded left to right from +0 and
converted once to the grad dtype; an fp32 update of main_grad converted back
to its dtype) and the _partial_sums_kernel
docstring (a run of at most 10 rows is one chunk).
"""
import numpy as np
import torch

NROWS = 10


def _to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 -> fp32 through torch (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def occurrences(ids: np.ndarray, vocab: int):
    """{id: [positions in ascending order]} for every id that occurs."""
    flat = ids.reshape(-1)
    out = {}
    for v in range(vocab):
        hits = [p for p in range(flat.size) if int(flat[p]) == v]
        if hits:
            out[v] = hits
    return out


def sort_tables(ids: np.ndarray, vocab: int) -> dict:
    """The sort step's tables, rebuilt from per-id occurrence lists."""
    occ = occurrences(ids, vocab)
    sorted_ids, positions, run_first, run_last, long_runs, chunk_first = [], [], [], [], [], []
    for v in sorted(occ):
        first = len(sorted_ids)
        plist = occ[v]
        for k, p in enumerate(plist):
            sorted_ids.append(v)
            positions.append(p)
            run_first.append(first)
            run_last.append(first + len(plist) - 1)
            if k % NROWS == 0:
                chunk_first.append(first + k)
        if len(plist) > NROWS:
            long_runs.append(first)
    return {k: np.array(v, dtype=np.int64) for k, v in dict(
        sorted_ids=sorted_ids, positions=positions, run_first=run_first, run_last=run_last,
        long_runs=long_runs, chunk_first=chunk_first).items()}


def accumulate(ids: np.ndarray, grad_f32: np.ndarray, main_grad_f32: np.ndarray,
               grad_dtype: str, main_grad_dtype: str) -> np.ndarray:
    """Return a new main_grad (as float32 values) after the accumulation.

    grad_f32 / main_grad_f32 hold the values already widened to fp32 (bf16
    inputs are exactly representable). The result for a bf16 main_grad is
    returned widened to fp32.
    """
    vocab, hidden = main_grad_f32.shape
    out = main_grad_f32.astype(np.float32, copy=True)
    for v, plist in occurrences(ids, vocab).items():
        total = np.zeros(hidden, dtype=np.float32)
        for c in range(0, len(plist), NROWS):
            part = np.zeros(hidden, dtype=np.float32)
            for p in plist[c:c + NROWS]:
                part = part + grad_f32[p].astype(np.float32)
            total = total + part
        g = _to_bf16_f32(total) if grad_dtype == "bf16" else total
        s = out[v] + g
        out[v] = _to_bf16_f32(s) if main_grad_dtype == "bf16" else s
    return out
