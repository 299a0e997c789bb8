"""Helpers of the GPU parity tests: the oracle's result for the touched rows of
main_grad, and the bit-for-bit comparison of a call's result with it."""
import numpy as np
import torch

import oracle
import workloads as wl


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _is_nan_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a & 0x7FFF) > 0x7F80
    b = a.view(np.uint32)
    return (b & 0x7FFFFFFF) > 0x7F800000


def oracle_rows(ids: torch.Tensor, grad: torch.Tensor, rows: torch.Tensor,
                before_rows: torch.Tensor) -> np.ndarray:
    """Oracle result for the touched rows: ids relabelled to their index in the
    sorted list of touched rows (an order-preserving relabel)."""
    g_dt = "bf16" if grad.dtype == torch.bfloat16 else "fp32"
    m_dt = "bf16" if before_rows.dtype == torch.bfloat16 else "fp32"
    ids_np = ids.reshape(-1).cpu().numpy()
    compact = np.searchsorted(rows.cpu().numpy(), ids_np).astype(ids_np.dtype)
    grad_np = wl.to_numpy_bits(grad.reshape(ids_np.size, grad.shape[-1]).cpu())
    mg_np = wl.to_numpy_bits(before_rows.cpu()).copy()
    oracle.accumulate_embedding_wgrad(compact, grad_np, mg_np, g_dt, m_dt)
    return mg_np


def assert_rows_match(ids: torch.Tensor, grad: torch.Tensor, main_grad: torch.Tensor,
                      before: torch.Tensor, rows: torch.Tensor, before_rows: torch.Tensor):
    """main_grad (after a call) against the oracle on its touched rows `rows`
    (before_rows: their values before the call), bit for bit with NaNs compared
    as a class; every other row bit-identical to `before`."""
    m_dt = "bf16" if main_grad.dtype == torch.bfloat16 else "fp32"
    got = wl.to_numpy_bits(main_grad[rows].cpu())
    want = oracle_rows(ids, grad, rows, before_rows)
    nan_g, nan_w = _is_nan_bits(got, m_dt), _is_nan_bits(want, m_dt)
    assert np.array_equal(nan_g, nan_w), "NaN positions differ"
    gv = got.view(np.uint16 if m_dt == "bf16" else np.uint32)
    wv = want.view(np.uint16 if m_dt == "bf16" else np.uint32)
    mism = (gv != wv) & ~nan_g
    if mism.any():
        r, c = np.argwhere(mism)[0]
        bad_rows = np.flatnonzero(mism.any(axis=1))
        counts = np.bincount(ids.reshape(-1).long().cpu().numpy())
        detail = "; ".join(
            f"id {int(rows[b])} ({int(counts[int(rows[b])])} rows): {int(mism[b].sum())} cols "
            f"in [{int(np.flatnonzero(mism[b])[0])}, {int(np.flatnonzero(mism[b])[-1])}]"
            for b in bad_rows[:12])
        raise AssertionError(f"{int(mism.sum())} mismatching elements in {bad_rows.size} rows; first "
                             f"at touched row {r} (id {int(rows[r])}), column {c}: got {gv[r, c]:#x} "
                             f"want {wv[r, c]:#x}; {detail}")

    # untouched rows: bit-identical to the copy taken before the call
    changed = (_bits(main_grad) != _bits(before)).any(dim=1)
    touched = torch.zeros(main_grad.shape[0], dtype=torch.bool, device=main_grad.device)
    touched[rows] = True
    assert not (changed & ~touched).any(), "a row whose id does not occur was written"
