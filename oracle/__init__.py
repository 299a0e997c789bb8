"""CPU oracle for main_grad += embedding_dense_backward(grad, ids), touched rows only.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import this package. It shares no code with the HIP
library in sparse_embedding_weight_amd/, and the library never calls it.

The arithmetic lives in embedding_wgrad_oracle.c (Megatron-Core API docs,
"core.fusions.fused_embedding_wgrad", introduction and the three kernel
docstrings); this module only marshals numpy arrays into it. bf16 arrays are
passed as numpy uint16 holding the raw bits.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute force, hand-computed chunk orders, closed forms, invariants, an
exhaustive check of the rounding, an fp64 error bound). Not pinned: the bit
pattern of a NaN after rounding (any quiet NaN is accepted).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        lib = ctypes.CDLL(_build.LIBRARY)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_uint32]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_bf16_array.argtypes = [vp, vp, i64]
        lib.oracle_round_bf16_array.restype = None
        lib.oracle_sort_tokens.argtypes = [vp, ci, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_sort_tokens.restype = ci
        lib.oracle_accumulate_embedding_wgrad.argtypes = [vp, ci, i64, vp, ci, i64, vp, ci, i64, i64]
        lib.oracle_accumulate_embedding_wgrad.restype = ci
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ids_flag(ids: np.ndarray) -> int:
    if ids.dtype == np.int64:
        return 1
    if ids.dtype == np.int32:
        return 0
    raise TypeError(f"ids must be int32 or int64, got {ids.dtype}")


def _float_flag(a: np.ndarray, dtype: str, what: str) -> int:
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError(f"{what}: bf16 data is passed as raw uint16 bits, got {a.dtype}")
        return 1
    if dtype == "fp32":
        if a.dtype != np.float32:
            raise TypeError(f"{what}: expected float32, got {a.dtype}")
        return 0
    raise ValueError(f"{what}: dtype must be 'bf16' or 'fp32', got {dtype!r}")


def _row_stride(a: np.ndarray, what: str) -> int:
    if a.ndim != 2 or a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        raise ValueError(f"{what}: need a 2-D array with unit column stride")
    return a.strides[0] // a.itemsize


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(_ptr(bits), _ptr(out), bits.size)
    return out


def round_bf16_bits(bits: np.ndarray, out: np.ndarray = None) -> np.ndarray:
    """Same as round_bf16 but takes raw uint32 bit patterns (any values, NaNs included)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    if out is None:
        out = np.empty(bits.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(_ptr(bits), _ptr(out), bits.size)
    return out


def sort_tokens(ids: np.ndarray) -> dict:
    """The tables of the sort step for flat `ids` (see oracle_sort_tokens in the C file)."""
    ids = np.ascontiguousarray(ids.reshape(-1))
    n = ids.size
    out = {k: np.zeros(n, dtype=np.int64) for k in ("sorted_ids", "positions", "run_first", "run_last")}
    long_runs = np.zeros(n + 1, dtype=np.int64)
    chunk_first = np.zeros(n + 1, dtype=np.int64)
    rc = _load().oracle_sort_tokens(_ptr(ids), _ids_flag(ids), n, _ptr(out["sorted_ids"]),
                                    _ptr(out["positions"]), _ptr(out["run_first"]),
                                    _ptr(out["run_last"]), _ptr(long_runs), _ptr(chunk_first))
    if rc != 0:
        raise MemoryError("oracle_sort_tokens ran out of memory")
    out["long_runs"] = long_runs[1:1 + long_runs[0]].copy()
    out["chunk_first"] = chunk_first[1:1 + chunk_first[0]].copy()
    return out


def accumulate_embedding_wgrad(ids: np.ndarray, grad: np.ndarray, main_grad: np.ndarray,
                               grad_dtype: str, main_grad_dtype: str) -> None:
    """main_grad[rows of ids] += wgrad, in place, with the page's arithmetic.

    ids: any shape, int32/int64, flattened row-major into positions.
    grad: [num_tokens, hidden] (unit column stride; row stride free).
    main_grad: [num_embeddings, hidden] (unit column stride; row stride free).
    """
    ids = np.ascontiguousarray(ids.reshape(-1))
    n = ids.size
    if grad.ndim != 2 or grad.shape[0] != n:
        raise ValueError(f"grad must be [{n}, hidden], got {grad.shape}")
    if main_grad.ndim != 2 or main_grad.shape[1] != grad.shape[1]:
        raise ValueError("main_grad must be [num_embeddings, hidden] with grad's hidden")
    if not main_grad.flags.writeable:
        raise ValueError("main_grad must be writeable")
    if n and (ids.min() < 0 or ids.max() >= main_grad.shape[0]):
        raise ValueError("ids must lie in [0, num_embeddings)")
    g_flag = _float_flag(grad, grad_dtype, "grad")
    m_flag = _float_flag(main_grad, main_grad_dtype, "main_grad")
    rc = _load().oracle_accumulate_embedding_wgrad(
        _ptr(ids), _ids_flag(ids), n, _ptr(grad), g_flag, _row_stride(grad, "grad"),
        _ptr(main_grad), m_flag, _row_stride(main_grad, "main_grad"), grad.shape[1])
    if rc != 0:
        raise MemoryError("oracle_accumulate_embedding_wgrad ran out of memory")


def accumulate_embedding_wgrad_column_blocks(ids: np.ndarray, grad: np.ndarray,
                                             main_grad: np.ndarray, grad_dtype: str,
                                             main_grad_dtype: str, threads: int) -> int:
    """accumulate_embedding_wgrad with the columns cut into `threads` blocks, each
    block one call of the same C routine on column views of grad and main_grad,
    the calls running at once on threads (ctypes drops the GIL during a call).

    Every sum of the page's arithmetic runs down one column (one element of the
    hidden dimension), so a block's columns see exactly the operations, in
    exactly the order, of the whole call: the result is the serial one bit for
    bit (pinned in tests/test_oracle_pins.py). Returns the number of blocks."""
    from concurrent.futures import ThreadPoolExecutor

    hidden = grad.shape[1]
    threads = max(1, min(int(threads), hidden))
    # block edges on multiples of 16 columns (64 bytes of fp32) where the width allows
    step = -(-hidden // threads)
    step = -(-step // 16) * 16 if hidden >= 16 * threads else step
    edges = list(range(0, hidden, step)) + [hidden]
    blocks = list(zip(edges[:-1], edges[1:]))
    with ThreadPoolExecutor(max_workers=len(blocks)) as pool:
        futures = [pool.submit(accumulate_embedding_wgrad, ids, grad[:, a:b], main_grad[:, a:b],
                               grad_dtype, main_grad_dtype) for a, b in blocks]
        for f in futures:
            f.result()
    return len(blocks)
