"""ctypes binding of libembedding_wgrad.so (include/embedding_wgrad.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library. PyTorch supplies device memory and the current
stream. Importing this module loads the library and fails loudly if it has
not been built.
"""
import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libembedding_wgrad.so")

if not os.path.exists(LIBRARY):
    raise ImportError(
        f"{LIBRARY} is missing: build it with `python sparse_embedding_weight_amd/build.py` "
        "(or __graft_entry__.build()). There is no fallback path.")

lib = ctypes.CDLL(LIBRARY)

# ---- constants and codes (include/embedding_wgrad.h) ----------------------
MIN_TOKENS = 3073
MAX_TOKENS = 8192
NROWS = 10
MANY_MAX_TOKENS = 131072          # EWG_MANY_MAX_TOKENS
MANY_MAX_EMBEDDINGS = 262144      # EWG_MANY_MAX_EMBEDDINGS

EWG_INT32, EWG_INT64, EWG_BF16, EWG_FP32 = 0, 1, 2, 3
(EWG_OK, EWG_UNSUPPORTED, EWG_INVALID_ARGUMENT, EWG_WORKSPACE_TOO_SMALL, EWG_HIP_ERROR,
 EWG_SCRATCH_TOO_SMALL) = range(6)
NO_ALLOC_SCRATCH_BYTES = 256 << 10  # EWG_NO_ALLOC_SCRATCH_BYTES

DTYPE_CODE = {torch.int32: EWG_INT32, torch.int64: EWG_INT64,
              torch.bfloat16: EWG_BF16, torch.float32: EWG_FP32}

# every function include/embedding_wgrad.h declares
EXPORTS = (
    "ewg_position_bits",
    "can_accumulate_embedding_wgrad",
    "accumulate_embedding_wgrad_workspace_bytes",
    "accumulate_embedding_wgrad",
    "accumulate_embedding_wgrad_timed",
    "accumulate_embedding_wgrad_no_alloc",
    "can_accumulate_embedding_wgrad_vocab_shard",
    "accumulate_embedding_wgrad_vocab_shard",
    "accumulate_embedding_wgrad_sort_tokens",
    "can_accumulate_embedding_wgrad_many_tokens",
    "accumulate_embedding_wgrad_many_tokens_workspace_bytes",
    "accumulate_embedding_wgrad_many_tokens",
    "accumulate_embedding_wgrad_many_tokens_timed",
    "ewg_status_string",
    # include/embedding_wgrad_test.h (test-only)
    "ewg_test_accumulate_embedding_wgrad",
)

_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t

lib.ewg_position_bits.argtypes = [_i64]
lib.ewg_position_bits.restype = _int
lib.can_accumulate_embedding_wgrad.argtypes = [_i64, _i64, _i64, _int, _int, _int]
lib.can_accumulate_embedding_wgrad.restype = _int
lib.accumulate_embedding_wgrad_workspace_bytes.argtypes = [_i64, _i64]
lib.accumulate_embedding_wgrad_workspace_bytes.restype = _sz
_ACC_ARGS = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _vp, _sz, _vp]
lib.accumulate_embedding_wgrad.argtypes = _ACC_ARGS
lib.accumulate_embedding_wgrad.restype = _int
lib.accumulate_embedding_wgrad_timed.argtypes = _ACC_ARGS + [_vp]
lib.accumulate_embedding_wgrad_timed.restype = _int
lib.accumulate_embedding_wgrad_no_alloc.argtypes = _ACC_ARGS[:11] + [_vp]
lib.accumulate_embedding_wgrad_no_alloc.restype = _int
lib.can_accumulate_embedding_wgrad_vocab_shard.argtypes = [_i64, _i64, _i64, _i64, _int, _int, _int]
lib.can_accumulate_embedding_wgrad_vocab_shard.restype = _int
lib.accumulate_embedding_wgrad_vocab_shard.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                                       _i64, _int, _int, _int, _vp, _sz, _vp]
lib.accumulate_embedding_wgrad_vocab_shard.restype = _int
lib.accumulate_embedding_wgrad_sort_tokens.argtypes = [_vp, _i64, _i64, _int] + [_vp] * 6 + [_vp, _sz, _vp]
lib.accumulate_embedding_wgrad_sort_tokens.restype = _int
lib.can_accumulate_embedding_wgrad_many_tokens.argtypes = [_i64, _i64, _i64, _int, _int, _int]
lib.can_accumulate_embedding_wgrad_many_tokens.restype = _int
lib.accumulate_embedding_wgrad_many_tokens_workspace_bytes.argtypes = [_i64, _i64]
lib.accumulate_embedding_wgrad_many_tokens_workspace_bytes.restype = _sz
lib.accumulate_embedding_wgrad_many_tokens.argtypes = _ACC_ARGS
lib.accumulate_embedding_wgrad_many_tokens.restype = _int
lib.accumulate_embedding_wgrad_many_tokens_timed.argtypes = _ACC_ARGS + [_vp]
lib.accumulate_embedding_wgrad_many_tokens_timed.restype = _int
lib.ewg_status_string.argtypes = [_int]
lib.ewg_status_string.restype = ctypes.c_char_p
lib.ewg_test_accumulate_embedding_wgrad.argtypes = _ACC_ARGS[:-1] + [_int, _int, _vp]
lib.ewg_test_accumulate_embedding_wgrad.restype = _int


class EmbeddingWgradError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.ewg_status_string(status).decode()} (status {status})")


class WaitGaveUpError(RuntimeError):
    """A bounded wait inside the kernel gave up: the call's main_grad is wrong."""


def position_bits(num_tokens: int) -> int:
    """bit_length(num_tokens - 1): low key bits that hold a position."""
    return lib.ewg_position_bits(num_tokens)


def workspace_bytes(num_tokens: int, hidden: int) -> int:
    return lib.accumulate_embedding_wgrad_workspace_bytes(num_tokens, hidden)


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _same_gpu(*tensors) -> bool:
    dev = tensors[0].device
    return dev.type == "cuda" and all(t.device == dev for t in tensors)


def can_accumulate_embedding_wgrad(ids: torch.Tensor, grad: torch.Tensor,
                                   main_grad: torch.Tensor) -> bool:
    """Whether accumulate_embedding_wgrad supports these tensors: MIN_TOKENS..MAX_TOKENS
    tokens, bf16 or fp32 grad and main_grad on one GPU, int32/int64 ids, grad of
    shape [*ids.shape, hidden], main_grad [num_embeddings, hidden] with unit column
    stride, and an id and position that pack into 31 bits."""
    if not (isinstance(ids, torch.Tensor) and isinstance(grad, torch.Tensor)
            and isinstance(main_grad, torch.Tensor)):
        return False
    if not _same_gpu(ids, grad, main_grad):
        return False
    if ids.dtype not in (torch.int32, torch.int64):
        return False
    if grad.dtype not in (torch.bfloat16, torch.float32) or main_grad.dtype not in (torch.bfloat16, torch.float32):
        return False
    if grad.dim() != ids.dim() + 1 or tuple(grad.shape[:-1]) != tuple(ids.shape):
        return False
    if main_grad.dim() != 2 or main_grad.shape[1] != grad.shape[-1] or main_grad.stride(1) != 1:
        return False
    return bool(lib.can_accumulate_embedding_wgrad(
        ids.numel(), grad.shape[-1], main_grad.shape[0], DTYPE_CODE[ids.dtype],
        DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad.dtype]))


def _flat_inputs(ids: torch.Tensor, grad: torch.Tensor):
    n, hidden = ids.numel(), grad.shape[-1]
    ids_flat = ids.reshape(-1)
    if not ids_flat.is_contiguous():
        ids_flat = ids_flat.contiguous()
    grad2 = grad.reshape(n, hidden)
    if grad2.stride(1) != 1:
        grad2 = grad2.contiguous()
    return ids_flat, grad2


# one zero-filled workspace per (device, stream), grown on demand; calls leave
# its flag word zero again, so it is reused without clearing
_WORKSPACES = {}


def new_workspace(num_tokens: int, hidden: int, device) -> torch.Tensor:
    """A zero-filled workspace for calls with these sizes (zero-filled before first use)."""
    return torch.zeros(workspace_bytes(num_tokens, hidden), dtype=torch.uint8, device=device)


def _workspace(n: int, hidden: int, device, workspace):
    need = workspace_bytes(n, hidden)
    if workspace is None:
        key = (device.index, torch.cuda.current_stream(device).cuda_stream)
        workspace = _WORKSPACES.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=device)
            _WORKSPACES[key] = workspace
    if workspace.dtype != torch.uint8 or workspace.device != device or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {device}")
    return workspace


def accumulate_embedding_wgrad(ids: torch.Tensor, grad: torch.Tensor, main_grad: torch.Tensor,
                               workspace: torch.Tensor = None, checked: bool = False) -> None:
    """main_grad += embedding_dense_backward(grad, ids), touching only the rows of ids.

    ids: token ids, num_tokens elements (any shape, flattened row-major).
    grad: [*ids.shape, hidden], gradient of the lookup's output.
    main_grad: [num_embeddings, hidden], updated in place.
    workspace: optional uint8 device tensor of >= workspace_bytes(num_tokens, hidden),
        zero-filled before its first use (new_workspace() makes one); by default a
        cached workspace per device and stream is used.
    checked: synchronise after the call and raise WaitGaveUpError if a bounded wait
        inside the kernel gave up during it (its result is then wrong). Off by
        default: the unchecked call never synchronises.
    Requires can_accumulate_embedding_wgrad(ids, grad, main_grad); raises ValueError
    otherwise. Enqueued on the current stream of main_grad's device; no sync.
    """
    if not can_accumulate_embedding_wgrad(ids, grad, main_grad):
        raise ValueError("accumulate_embedding_wgrad: unsupported inputs "
                         "(see can_accumulate_embedding_wgrad)")
    n, hidden = ids.numel(), grad.shape[-1]
    ids_flat, grad2 = _flat_inputs(ids, grad)
    ws = _workspace(n, hidden, main_grad.device, workspace)
    before = wait_timeouts(ws) if checked else 0
    with torch.cuda.device(main_grad.device):
        st = lib.accumulate_embedding_wgrad(
            ids_flat.data_ptr(), grad2.data_ptr(), main_grad.data_ptr(), n, hidden,
            main_grad.shape[0], grad2.stride(0), main_grad.stride(0), DTYPE_CODE[ids.dtype],
            DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad.dtype], ws.data_ptr(), ws.numel(),
            _stream_handle(main_grad.device))
    if st != EWG_OK:
        raise EmbeddingWgradError(st, "accumulate_embedding_wgrad")
    if checked:
        raise_if_waits_gave_up(ws, before, "accumulate_embedding_wgrad")


def accumulate_embedding_wgrad_no_alloc(ids: torch.Tensor, grad: torch.Tensor,
                                        main_grad: torch.Tensor) -> None:
    """accumulate_embedding_wgrad without a workspace and without allocating: the
    library's static per-device scratch serves as the workspace (calls that overlap
    on one device race). Nothing is copied either, so ids must be contiguous and
    grad viewable as [num_tokens, hidden] with unit column stride; raises ValueError
    otherwise, and EmbeddingWgradError (EWG_SCRATCH_TOO_SMALL) for sizes whose
    workspace exceeds NO_ALLOC_SCRATCH_BYTES. Enqueued on the current stream."""
    if not can_accumulate_embedding_wgrad(ids, grad, main_grad):
        raise ValueError("accumulate_embedding_wgrad_no_alloc: unsupported inputs "
                         "(see can_accumulate_embedding_wgrad)")
    n, hidden = ids.numel(), grad.shape[-1]
    if not ids.is_contiguous():
        raise ValueError("accumulate_embedding_wgrad_no_alloc: ids must be contiguous")
    try:
        grad2 = grad.view(n, hidden)
    except RuntimeError:
        raise ValueError("accumulate_embedding_wgrad_no_alloc: grad must be viewable as "
                         "[num_tokens, hidden]") from None
    if grad2.stride(1) != 1:
        raise ValueError("accumulate_embedding_wgrad_no_alloc: grad needs unit column stride")
    with torch.cuda.device(main_grad.device):
        st = lib.accumulate_embedding_wgrad_no_alloc(
            ids.data_ptr(), grad2.data_ptr(), main_grad.data_ptr(), n, hidden,
            main_grad.shape[0], grad2.stride(0), main_grad.stride(0), DTYPE_CODE[ids.dtype],
            DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad.dtype], _stream_handle(main_grad.device))
    if st != EWG_OK:
        raise EmbeddingWgradError(st, "accumulate_embedding_wgrad_no_alloc")


def accumulate_with_grid_for_tests(ids: torch.Tensor, grad: torch.Tensor, main_grad: torch.Tensor,
                                   workspace: torch.Tensor, grid: int,
                                   odd_skip_long: bool = False) -> None:
    """Tests only (include/embedding_wgrad_test.h): accumulate_embedding_wgrad launched
    with `grid` workgroups; with odd_skip_long the odd-numbered workgroups take no
    column block of a long run. Same result as accumulate_embedding_wgrad."""
    if not can_accumulate_embedding_wgrad(ids, grad, main_grad):
        raise ValueError("accumulate_with_grid_for_tests: unsupported inputs")
    n, hidden = ids.numel(), grad.shape[-1]
    ids_flat, grad2 = _flat_inputs(ids, grad)
    ws = _workspace(n, hidden, main_grad.device, workspace)
    with torch.cuda.device(main_grad.device):
        st = lib.ewg_test_accumulate_embedding_wgrad(
            ids_flat.data_ptr(), grad2.data_ptr(), main_grad.data_ptr(), n, hidden,
            main_grad.shape[0], grad2.stride(0), main_grad.stride(0), DTYPE_CODE[ids.dtype],
            DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad.dtype], ws.data_ptr(), ws.numel(),
            int(grid), 1 if odd_skip_long else 0, _stream_handle(main_grad.device))
    if st != EWG_OK:
        raise EmbeddingWgradError(st, "ewg_test_accumulate_embedding_wgrad")


def _same_layout(ids, grad, main_grad) -> bool:
    if not (isinstance(ids, torch.Tensor) and isinstance(grad, torch.Tensor)
            and isinstance(main_grad, torch.Tensor)):
        return False
    if not _same_gpu(ids, grad, main_grad):
        return False
    if ids.dtype not in (torch.int32, torch.int64):
        return False
    if grad.dtype not in (torch.bfloat16, torch.float32) or main_grad.dtype not in (torch.bfloat16, torch.float32):
        return False
    if grad.dim() != ids.dim() + 1 or tuple(grad.shape[:-1]) != tuple(ids.shape):
        return False
    return main_grad.dim() == 2 and main_grad.shape[1] == grad.shape[-1] and main_grad.stride(1) == 1


def can_accumulate_embedding_wgrad_vocab_shard(ids: torch.Tensor, grad: torch.Tensor,
                                               main_grad_shard: torch.Tensor,
                                               vocab_start: int) -> bool:
    """Whether accumulate_embedding_wgrad_vocab_shard supports these tensors: as
    can_accumulate_embedding_wgrad with main_grad_shard's rows standing for ids
    [vocab_start, vocab_start + rows), vocab_start >= 0, and one more id bit in the
    31-bit packing test."""
    if not _same_layout(ids, grad, main_grad_shard) or int(vocab_start) < 0:
        return False
    return bool(lib.can_accumulate_embedding_wgrad_vocab_shard(
        ids.numel(), grad.shape[-1], int(vocab_start), main_grad_shard.shape[0],
        DTYPE_CODE[ids.dtype], DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad_shard.dtype]))


def accumulate_embedding_wgrad_vocab_shard(ids: torch.Tensor, grad: torch.Tensor,
                                           main_grad_shard: torch.Tensor, vocab_start: int,
                                           workspace: torch.Tensor = None) -> None:
    """The rows of one vocabulary shard: main_grad_shard[v] (id vocab_start + v) +=
    the embedding weight gradient of that id; ids outside the shard are left out.
    Same arithmetic, bit for bit, as accumulate_embedding_wgrad on the full table.
    Other arguments and behaviour as for accumulate_embedding_wgrad."""
    if not can_accumulate_embedding_wgrad_vocab_shard(ids, grad, main_grad_shard, vocab_start):
        raise ValueError("accumulate_embedding_wgrad_vocab_shard: unsupported inputs "
                         "(see can_accumulate_embedding_wgrad_vocab_shard)")
    n, hidden = ids.numel(), grad.shape[-1]
    ids_flat, grad2 = _flat_inputs(ids, grad)
    ws = _workspace(n, hidden, main_grad_shard.device, workspace)
    with torch.cuda.device(main_grad_shard.device):
        st = lib.accumulate_embedding_wgrad_vocab_shard(
            ids_flat.data_ptr(), grad2.data_ptr(), main_grad_shard.data_ptr(), n, hidden,
            int(vocab_start), main_grad_shard.shape[0], grad2.stride(0), main_grad_shard.stride(0),
            DTYPE_CODE[ids.dtype], DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad_shard.dtype],
            ws.data_ptr(), ws.numel(), _stream_handle(main_grad_shard.device))
    if st != EWG_OK:
        raise EmbeddingWgradError(st, "accumulate_embedding_wgrad_vocab_shard")


def many_tokens_workspace_bytes(num_tokens: int, hidden: int) -> int:
    return lib.accumulate_embedding_wgrad_many_tokens_workspace_bytes(num_tokens, hidden)


def can_accumulate_embedding_wgrad_many_tokens(ids: torch.Tensor, grad: torch.Tensor,
                                               main_grad: torch.Tensor) -> bool:
    """Whether accumulate_embedding_wgrad_many_tokens supports these tensors: as
    can_accumulate_embedding_wgrad, but MIN_TOKENS..MANY_MAX_TOKENS tokens and at
    most MANY_MAX_EMBEDDINGS rows of main_grad (no position packing)."""
    if not _same_layout(ids, grad, main_grad):
        return False
    return bool(lib.can_accumulate_embedding_wgrad_many_tokens(
        ids.numel(), grad.shape[-1], main_grad.shape[0], DTYPE_CODE[ids.dtype],
        DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad.dtype]))


def new_many_tokens_workspace(num_tokens: int, hidden: int, device) -> torch.Tensor:
    """A workspace for many-token calls with these sizes (needs no clearing)."""
    return torch.empty(many_tokens_workspace_bytes(num_tokens, hidden), dtype=torch.uint8,
                       device=device)


_MANY_WORKSPACES = {}


def accumulate_embedding_wgrad_many_tokens(ids: torch.Tensor, grad: torch.Tensor,
                                           main_grad: torch.Tensor,
                                           workspace: torch.Tensor = None) -> None:
    """accumulate_embedding_wgrad for more than MAX_TOKENS tokens (up to
    MANY_MAX_TOKENS): the same arithmetic, bit for bit. workspace: optional uint8
    device tensor of >= many_tokens_workspace_bytes(num_tokens, hidden) bytes
    (new_many_tokens_workspace() makes one); by default a cached one per device and
    stream. Requires can_accumulate_embedding_wgrad_many_tokens; raises ValueError
    otherwise. Enqueued on the current stream of main_grad's device; no sync."""
    if not can_accumulate_embedding_wgrad_many_tokens(ids, grad, main_grad):
        raise ValueError("accumulate_embedding_wgrad_many_tokens: unsupported inputs "
                         "(see can_accumulate_embedding_wgrad_many_tokens)")
    n, hidden = ids.numel(), grad.shape[-1]
    ids_flat, grad2 = _flat_inputs(ids, grad)
    device = main_grad.device
    need = many_tokens_workspace_bytes(n, hidden)
    if workspace is None:
        key = (device.index, torch.cuda.current_stream(device).cuda_stream)
        workspace = _MANY_WORKSPACES.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
            _MANY_WORKSPACES[key] = workspace
    if workspace.dtype != torch.uint8 or workspace.device != device or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {device}")
    with torch.cuda.device(device):
        st = lib.accumulate_embedding_wgrad_many_tokens(
            ids_flat.data_ptr(), grad2.data_ptr(), main_grad.data_ptr(), n, hidden,
            main_grad.shape[0], grad2.stride(0), main_grad.stride(0), DTYPE_CODE[ids.dtype],
            DTYPE_CODE[grad.dtype], DTYPE_CODE[main_grad.dtype], workspace.data_ptr(),
            workspace.numel(), _stream_handle(device))
    if st != EWG_OK:
        raise EmbeddingWgradError(st, "accumulate_embedding_wgrad_many_tokens")


def sort_tokens(ids: torch.Tensor, num_embeddings: int, workspace: torch.Tensor = None) -> dict:
    """Run only the sort step and return its tables (device int32 tensors):
    sorted_ids, positions, run_first, run_last (per sorted slot), long_runs (first
    slots of the runs longer than NROWS) and chunk_first (first slot of every chunk)."""
    if ids.device.type != "cuda" or ids.dtype not in (torch.int32, torch.int64):
        raise ValueError("ids must be an int32/int64 GPU tensor")
    n = ids.numel()
    ids_flat = ids.reshape(-1).contiguous()
    dev = ids.device
    out = {k: torch.empty(n, dtype=torch.int32, device=dev)
           for k in ("sorted_ids", "positions", "run_first", "run_last")}
    long_runs = torch.zeros(n + 1, dtype=torch.int32, device=dev)
    chunk_first = torch.zeros(n + 1, dtype=torch.int32, device=dev)
    ws = _workspace(n, 1, dev, workspace)
    with torch.cuda.device(dev):
        st = lib.accumulate_embedding_wgrad_sort_tokens(
            ids_flat.data_ptr(), n, num_embeddings, DTYPE_CODE[ids.dtype],
            out["sorted_ids"].data_ptr(), out["positions"].data_ptr(), out["run_first"].data_ptr(),
            out["run_last"].data_ptr(), long_runs.data_ptr(), chunk_first.data_ptr(),
            ws.data_ptr(), ws.numel(), _stream_handle(dev))
    if st != EWG_OK:
        raise EmbeddingWgradError(st, "accumulate_embedding_wgrad_sort_tokens")
    out["long_runs"] = long_runs[1:1 + int(long_runs[0].item())]
    out["chunk_first"] = chunk_first[1:1 + int(chunk_first[0].item())]
    return out


def invalid_id_count(workspace: torch.Tensor) -> int:
    """Ids outside [0, num_embeddings) seen by the last call that used `workspace`
    (reads the documented first int32 of the workspace; synchronises)."""
    return int(workspace[:4].view(torch.int32).item())


WS_WAIT_TIMEOUTS_OFFSET = 144   # EWG_WS_WAIT_TIMEOUTS_OFFSET
WS_CHECK_FAILURES_OFFSET = 148  # EWG_WS_CHECK_FAILURES_OFFSET (0 unless built with device checks)


def wait_timeouts(workspace: torch.Tensor) -> int:
    """Bounded waits inside the kernel that gave up since `workspace` was
    zero-filled (the documented diagnostic word; synchronises). Never expected."""
    o = WS_WAIT_TIMEOUTS_OFFSET
    return int(workspace[o:o + 4].view(torch.int32).item())


def raise_if_waits_gave_up(workspace: torch.Tensor, before: int, what: str = "call") -> None:
    """Raise WaitGaveUpError if the workspace's wait-timeout word grew past `before`
    (its value read before the call): a wait that gave up skipped work, so the
    call's result is wrong. Synchronises with the workspace's device."""
    after = wait_timeouts(workspace)
    if after != before:
        raise WaitGaveUpError(
            f"{what}: {after - before} bounded wait(s) inside the kernel gave up; "
            "main_grad is wrong for this call")
