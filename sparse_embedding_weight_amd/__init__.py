"""MI355X (gfx950) embedding weight-gradient accumulation.

    main_grad += embedding_dense_backward(grad, ids), touching only the rows of ids

with the arithmetic of PyTorch's sort-based embedding backward followed by
main_grad.add_ (Megatron-Core API docs, "core.fusions.fused_embedding_wgrad").
The work runs in hand-written HIP kernels behind the C ABI of
include/embedding_wgrad.h; this package is a thin binding to it.
"""
from ._binding import (  # noqa: F401
    MANY_MAX_EMBEDDINGS,
    MANY_MAX_TOKENS,
    MAX_TOKENS,
    MIN_TOKENS,
    NO_ALLOC_SCRATCH_BYTES,
    NROWS,
    EmbeddingWgradError,
    WaitGaveUpError,
    accumulate_embedding_wgrad,
    accumulate_embedding_wgrad_many_tokens,
    accumulate_embedding_wgrad_no_alloc,
    accumulate_embedding_wgrad_vocab_shard,
    can_accumulate_embedding_wgrad,
    can_accumulate_embedding_wgrad_many_tokens,
    can_accumulate_embedding_wgrad_vocab_shard,
    invalid_id_count,
    many_tokens_workspace_bytes,
    new_many_tokens_workspace,
    new_workspace,
    position_bits,
    raise_if_waits_gave_up,
    sort_tokens,
    wait_timeouts,
    workspace_bytes,
)
from ._binding import LIBRARY as library_path  # noqa: F401
