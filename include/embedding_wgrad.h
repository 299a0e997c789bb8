/*
 * embedding_wgrad.h -- C ABI of the MI355X (gfx950) embedding weight-gradient
 * accumulation library, libembedding_wgrad.so.
 *
 * Operation (Megatron-Core API docs, "core.fusions.fused_embedding_wgrad",
 * accumulate_embedding_wgrad and the introduction):
 *
 *     main_grad += embedding_dense_backward(grad, ids)
 *
 * touching only the rows of main_grad whose id occurs in ids, with the
 * arithmetic of the sort-based dense backward (introduction, first bullet)
 * followed by main_grad.add_ (second bullet):
 *   - the rows of one id are taken by ascending position;
 *   - they are cut into chunks of ten rows (the last chunk may be shorter),
 *     counted from the id's first row, and each chunk is summed in fp32;
 *   - the chunk sums are folded left to right from +0 and the total is
 *     converted once (round to nearest even) to grad's dtype;
 *   - that value is added to the main_grad row in fp32 and the sum rounded to
 *     main_grad's dtype.
 * Rows of ids that do not occur are neither read nor written (the sentence
 * after the two bullets). For given inputs every output bit is fixed: two
 * calls on the same inputs give identical main_grad bits.
 *
 * Conventions for every entry point below:
 *   - pointers named ids, grad, main_grad, workspace and the sort tables are
 *     DEVICE pointers on the device that `stream` belongs to, owned by the
 *     caller; the library keeps no pointer after the call returns;
 *   - all work is enqueued on `stream` (NULL = the legacy default stream);
 *     no entry point synchronises the stream or allocates device memory;
 *   - arguments are checked on the host before anything is enqueued; on any
 *     non-zero return nothing was enqueued and main_grad is untouched
 *     (except EWG_HIP_ERROR, which reports a failed launch);
 *   - the functions are thread-safe; concurrent calls must not share a
 *     workspace unless ordered by their streams;
 *   - the accumulate entry points enqueue kernels only (no memset, no copy,
 *     no allocation), so a call can be captured in a HIP graph and the graph
 *     replayed: each replay adds the gradient again, exactly as a new call
 *     with the same arguments would.
 */
#ifndef EMBEDDING_WGRAD_H
#define EMBEDDING_WGRAD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Envelope (page, Data: MIN_TOKENS, MAX_TOKENS, _NROWS). MIN_TOKENS is the
 * smallest token count that takes PyTorch's sort-based path (page,
 * introduction: 3072 tokens or fewer take another path). */
#define EWG_MIN_TOKENS 3073
#define EWG_MAX_TOKENS 8192
#define EWG_NROWS 10

/* Element types. ids: EWG_INT32 or EWG_INT64. grad, main_grad: EWG_BF16 or EWG_FP32. */
typedef enum ewg_dtype {
    EWG_INT32 = 0,
    EWG_INT64 = 1,
    EWG_BF16 = 2,
    EWG_FP32 = 3
} ewg_dtype;

typedef enum ewg_status {
    EWG_OK = 0,
    EWG_UNSUPPORTED = 1,          /* outside the envelope (can_accumulate... is 0) */
    EWG_INVALID_ARGUMENT = 2,     /* null pointer, bad stride, bad dtype code */
    EWG_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below ..._workspace_bytes() */
    EWG_HIP_ERROR = 4,            /* a kernel launch failed */
    EWG_SCRATCH_TOO_SMALL = 5     /* ..._no_alloc: sizes beyond EWG_NO_ALLOC_SCRATCH_BYTES */
} ewg_status;

/*
 * Number of low key bits that hold a token's position, for num_tokens tokens
 * (page, _position_bits): the fewest bits that represent every position
 * 0 .. num_tokens-1, i.e. bit_length(num_tokens - 1); 0 for num_tokens <= 1.
 * Host only.
 */
int ewg_position_bits(int64_t num_tokens);

/*
 * Whether accumulate_embedding_wgrad supports these sizes and types (page,
 * can_accumulate_embedding_wgrad): 1 or 0, host only, reads no memory.
 * True iff
 *   EWG_MIN_TOKENS <= num_tokens <= EWG_MAX_TOKENS (both bounds included),
 *   hidden >= 1, num_embeddings >= 1,
 *   ids_dtype is EWG_INT32 or EWG_INT64,
 *   grad_dtype and main_grad_dtype are EWG_BF16 or EWG_FP32, and
 *   the largest id and position pack into 31 bits:
 *     ((num_embeddings - 1) << ewg_position_bits(num_tokens)) | (num_tokens - 1) < 2^31.
 * (The page's "on the GPU" condition is the caller's: the pointers passed to
 * accumulate_embedding_wgrad must be device memory.)
 */
int can_accumulate_embedding_wgrad(int64_t num_tokens, int64_t hidden, int64_t num_embeddings,
                                   int ids_dtype, int grad_dtype, int main_grad_dtype);

/*
 * Bytes of device workspace accumulate_embedding_wgrad and
 * accumulate_embedding_wgrad_sort_tokens need for these sizes (host only).
 * The workspace holds the records of the runs longer than EWG_NROWS rows
 * (positions and rows of their chunks) and the flag and counters the
 * kernel's workgroups share: about 61 KB for 8192 tokens, whatever hidden is.
 * Its content between calls is not part of the interface except for two
 * int32 words: the first 4 bytes (see below), and the one at byte offset
 * EWG_WS_WAIT_TIMEOUTS_OFFSET, which counts the bounded waits inside the
 * kernel that gave up (and the long-run records found not to belong to the
 * call) since the workspace was zero-filled.
 *
 * A wait that gives up is an ERROR of the call, not a diagnostic: the work
 * behind it was skipped and that call's main_grad is wrong. Every wait is
 * bounded (seconds) so that a launch always ends; none is expected to give up.
 * A caller that must know reads the word before the call and after it has
 * finished on its stream, and treats any growth as a failed call (the Python
 * binding's checked mode does this and raises).
 * 0 if the sizes are out of range.
 */
#define EWG_WS_WAIT_TIMEOUTS_OFFSET 144

/*
 * Byte offset of a third int32 word of the workspace: the device-side bounds
 * checks that failed since the workspace was zero-filled. It stays 0 in the
 * default build. A build with -DEWG_DEVICE_CHECKS=1 (a debugging aid) checks
 * the data-derived indices of the one-kernel path (LDS tables, staged chunk
 * sums, positions and rows of long-run chunks) against their bounds; an index
 * out of bounds is counted here and replaced by the last valid one, so that
 * such a build never accesses memory out of bounds.
 */
#define EWG_WS_CHECK_FAILURES_OFFSET 148

size_t accumulate_embedding_wgrad_workspace_bytes(int64_t num_tokens, int64_t hidden);

/*
 * main_grad[ids[p], :] += the weight gradient, touching only occurring rows
 * (page, accumulate_embedding_wgrad).
 *
 *   ids        num_tokens ids (ids_dtype), the flattened (row-major) id tensor;
 *              position p of a token is its index here. Each id must lie in
 *              [0, num_embeddings). If any does not, the call changes nothing
 *              in main_grad and stores the number of such ids as an int32 in
 *              the first 4 bytes of the workspace (0 after a valid call).
 *   grad       num_tokens rows of `hidden` values (grad_dtype); row p starts at
 *              element p * grad_row_stride; unit column stride.
 *   main_grad  num_embeddings rows of `hidden` values (main_grad_dtype); row v
 *              starts at element v * main_grad_row_stride; unit column stride.
 *              Updated in place; must not overlap grad, ids or the workspace.
 *   grad_row_stride, main_grad_row_stride
 *              in elements, each >= hidden.
 *   workspace  device scratch of at least
 *              accumulate_embedding_wgrad_workspace_bytes(num_tokens, hidden)
 *              bytes, 256-byte aligned, zero-filled before its first use; every
 *              call leaves its synchronisation word zero again, so it is reused
 *              without clearing. It must not be used by another call until this
 *              one has finished on `stream`.
 *
 * Returns EWG_OK after enqueueing one kernel on `stream`. It launches one
 * 1024-thread workgroup per compute unit. Workgroup 0 sorts the keys in LDS
 * and publishes the chunks of runs longer than EWG_NROWS rows; meanwhile the
 * other workgroups finish every run of at most EWG_NROWS rows; then all of
 * them take column blocks of the long runs from a shared ticket, each block
 * summed, folded in chunk order and finished inside one workgroup. The only
 * wait between workgroups is for workgroup 0's flag, and workgroup 0 waits
 * for nothing, so the call needs no particular number of workgroups running
 * at once. The wait is bounded; one that gives up is counted in the
 * workspace's int32 at EWG_WS_WAIT_TIMEOUTS_OFFSET and its work is skipped.
 * Any alignment is accepted; 16-byte aligned rows take the vector path.
 *
 * The workspace carries counters from one call to the next: a call that did
 * not run to completion (for example a device fault) leaves it unusable
 * until it is zero-filled again.
 */
int accumulate_embedding_wgrad(const void *ids, const void *grad, void *main_grad,
                               int64_t num_tokens, int64_t hidden, int64_t num_embeddings,
                               int64_t grad_row_stride, int64_t main_grad_row_stride,
                               int ids_dtype, int grad_dtype, int main_grad_dtype,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * accumulate_embedding_wgrad (same arguments less the workspace, same checks,
 * arithmetic and result) with the workspace in a static device array of
 * EWG_NO_ALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends (its address is looked up once per device,
 * on that device's first call). The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine. It enqueues on `stream` a small
 * kernel that zeroes the array's header, then the accumulate kernel.
 *
 * Every call on one device shares that device's array and leaves its contents
 * there: calls that overlap on one device (on different streams, or from
 * different threads without ordering) race and give wrong results. Sizes
 * whose workspace (accumulate_embedding_wgrad_workspace_bytes) exceeds
 * EWG_NO_ALLOC_SCRATCH_BYTES would return EWG_SCRATCH_TOO_SMALL before
 * anything is enqueued; 256 KiB holds every size of the envelope (about 61 KB
 * for 8192 tokens, whatever hidden is), so that check is a guard. A bounded
 * wait that gives up is not reported by this entry point (use
 * accumulate_embedding_wgrad with a workspace to read the count).
 */
#define EWG_NO_ALLOC_SCRATCH_BYTES (256 << 10)
int accumulate_embedding_wgrad_no_alloc(const void *ids, const void *grad, void *main_grad,
                                        int64_t num_tokens, int64_t hidden,
                                        int64_t num_embeddings, int64_t grad_row_stride,
                                        int64_t main_grad_row_stride, int ids_dtype,
                                        int grad_dtype, int main_grad_dtype, hipStream_t stream);

/*
 * accumulate_embedding_wgrad with timing markers: `events` points to 4
 * caller-created hipEvent_t (timing enabled). events[0] and events[1] are
 * recorded on `stream` right before and right after the call's work;
 * events[2] and events[3] are attached to the kernel's own dispatch
 * (hipExtLaunchKernelGGL), so that they span the kernel's execution alone.
 * events[2] and events[3] may both be NULL: the kernel is then dispatched as
 * in accumulate_embedding_wgrad (such a dispatch costs less time around the
 * kernel than one that takes events). Same arguments, results and errors
 * otherwise; meant for benchmarks.
 */
int accumulate_embedding_wgrad_timed(const void *ids, const void *grad, void *main_grad,
                                     int64_t num_tokens, int64_t hidden, int64_t num_embeddings,
                                     int64_t grad_row_stride, int64_t main_grad_row_stride,
                                     int ids_dtype, int grad_dtype, int main_grad_dtype,
                                     void *workspace, size_t workspace_bytes,
                                     hipStream_t stream, hipEvent_t *events);

/*
 * Vocabulary-sharded form (the embedding table split by rows over devices):
 * main_grad holds only the shard_rows rows of ids [vocab_start, vocab_start +
 * shard_rows) of the full table, row v for id vocab_start + v. ids and grad
 * are the whole batch (num_tokens positions, as in accumulate_embedding_wgrad).
 * Ids outside the shard are left out: their grad rows are not read and no
 * row is touched for them; an id in the shard is accumulated with exactly the
 * arithmetic of accumulate_embedding_wgrad (its run, chunks and their order
 * depend only on its own positions), so the shards of any partition of the
 * vocabulary together give, bit for bit, the rows of one unsharded call.
 *
 * can_accumulate_embedding_wgrad_vocab_shard: as can_accumulate_embedding_wgrad
 * with num_embeddings replaced by shard_rows, plus vocab_start >= 0; the
 * packing test takes one more id bit: (shard_rows << position_bits) |
 * (num_tokens - 1) < 2^31. No id is invalid here, so the workspace's
 * invalid-id count stays 0. Workspace, stream, errors: as for
 * accumulate_embedding_wgrad.
 */
int can_accumulate_embedding_wgrad_vocab_shard(int64_t num_tokens, int64_t hidden,
                                               int64_t vocab_start, int64_t shard_rows,
                                               int ids_dtype, int grad_dtype, int main_grad_dtype);

int accumulate_embedding_wgrad_vocab_shard(const void *ids, const void *grad, void *main_grad,
                                           int64_t num_tokens, int64_t hidden,
                                           int64_t vocab_start, int64_t shard_rows,
                                           int64_t grad_row_stride, int64_t main_grad_row_stride,
                                           int ids_dtype, int grad_dtype, int main_grad_dtype,
                                           void *workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/*
 * Only the sort step, with its tables written out for inspection (page,
 * _sort_tokens_kernel: sort the (token, position) pairs, give every sorted
 * slot the first and last slot of its token's run, list the runs longer than
 * NROWS with their count first). Device int32 outputs, s = sorted slot:
 *   sorted_ids[s], positions[s]   num_tokens entries each
 *   run_first[s], run_last[s]     first and last (inclusive) slot of the run
 *   long_runs                     num_tokens + 1 entries: [0] = number of runs
 *                                 longer than EWG_NROWS, [1..] their first
 *                                 slots in ascending order
 *   chunk_first                   num_tokens + 1 entries: [0] = number of
 *                                 chunks, [1..] the first slot of every chunk
 *                                 (chunks of EWG_NROWS rows counted from the
 *                                 start of each run), ascending
 * Entries past the counts are left as they were. Same envelope, id rule and
 * workspace as accumulate_embedding_wgrad (with invalid ids both counts are 0).
 */
int accumulate_embedding_wgrad_sort_tokens(const void *ids, int64_t num_tokens,
                                           int64_t num_embeddings, int ids_dtype,
                                           int32_t *sorted_ids, int32_t *positions,
                                           int32_t *run_first, int32_t *run_last,
                                           int32_t *long_runs, int32_t *chunk_first,
                                           void *workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/*
 * Calls of more tokens than the page's MAX_TOKENS. That bound comes from the
 * page's one-program sort of at most 8192 keys, not from the arithmetic
 * (introduction; _sort_tokens_kernel sorts one block of keys): this form
 * gives exactly the result the arithmetic above defines, bit for bit, for
 * EWG_MIN_TOKENS <= num_tokens <= EWG_MANY_MAX_TOKENS (and the same bits as
 * accumulate_embedding_wgrad where both apply).
 *
 * The batch is cut into tiles of 8192 positions, each sorted in LDS by one
 * workgroup, and the sorted tiles are merged by rank (a position of tile t
 * precedes every position of tile t + 1). Five kernels on `stream`; none
 * waits for another workgroup, so any number of them may run at once.
 *
 * can_accumulate_embedding_wgrad_many_tokens: 1 iff
 *   EWG_MIN_TOKENS <= num_tokens <= EWG_MANY_MAX_TOKENS,
 *   1 <= num_embeddings <= EWG_MANY_MAX_EMBEDDINGS (a tile key packs the id
 *   above 13 position bits into 31 bits), hidden >= 1, and the dtypes of
 *   can_accumulate_embedding_wgrad. Host only.
 * accumulate_embedding_wgrad_many_tokens_workspace_bytes: bytes of workspace
 *   for these sizes (0 if out of range). The workspace needs no clearing:
 *   a call writes every part of it before reading it. Its first int32 is the
 *   invalid-id count, as for accumulate_embedding_wgrad. A many-token call
 *   writes nothing in bytes 128..1023, where accumulate_embedding_wgrad keeps
 *   its flags and counters, so one buffer (large enough for both) may be
 *   passed to either entry point in turn.
 * accumulate_embedding_wgrad_many_tokens: arguments, layouts, the id rule
 *   (an id outside [0, num_embeddings) makes the call change nothing in
 *   main_grad and stores the number of such ids in the first int32 of the
 *   workspace), errors and alignment as for accumulate_embedding_wgrad.
 * ..._timed: with 2 caller-created events recorded on `stream` before the
 *   first and after the last kernel (benchmarks).
 */
#define EWG_MANY_MAX_TOKENS 131072
#define EWG_MANY_MAX_EMBEDDINGS 262144

int can_accumulate_embedding_wgrad_many_tokens(int64_t num_tokens, int64_t hidden,
                                               int64_t num_embeddings, int ids_dtype,
                                               int grad_dtype, int main_grad_dtype);

size_t accumulate_embedding_wgrad_many_tokens_workspace_bytes(int64_t num_tokens, int64_t hidden);

int accumulate_embedding_wgrad_many_tokens(const void *ids, const void *grad, void *main_grad,
                                           int64_t num_tokens, int64_t hidden,
                                           int64_t num_embeddings, int64_t grad_row_stride,
                                           int64_t main_grad_row_stride, int ids_dtype,
                                           int grad_dtype, int main_grad_dtype, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream);

int accumulate_embedding_wgrad_many_tokens_timed(const void *ids, const void *grad,
                                                 void *main_grad, int64_t num_tokens,
                                                 int64_t hidden, int64_t num_embeddings,
                                                 int64_t grad_row_stride,
                                                 int64_t main_grad_row_stride, int ids_dtype,
                                                 int grad_dtype, int main_grad_dtype,
                                                 void *workspace, size_t workspace_bytes,
                                                 hipStream_t stream, hipEvent_t *events);

/* Static English text for a status code (never NULL). */
const char *ewg_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EMBEDDING_WGRAD_H */
