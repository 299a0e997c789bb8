// Internal layout shared by the kernels and the host entry points of
// libembedding_wgrad.so. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ewg {

constexpr int kNRows = 10;           // rows per partial sum (NROWS_PER_THREAD)
constexpr int kMaxTokens = 8192;     // keys one LDS sort holds
constexpr int kSortThreads = 1024;   // sort workgroup: 16 waves of 64
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = kMaxTokens / kSortThreads;   // keys per thread
constexpr int kMaxDigitBits = 10;    // radix digit of one sort pass

// Workspace header, at offset 0. invalid_ids is the documented first int32.
struct WsHeader {
    int32_t invalid_ids;      // ids outside [0, num_embeddings) seen by the last call
    int32_t num_chunks;       // chunks of all runs
    int32_t num_long_runs;    // runs longer than kNRows rows
    int32_t num_long_chunks;  // chunks of those runs = rows of the partial buffer in use
    int32_t num_runs;         // distinct ids
    uint32_t cost_total;      // sum of the per-tile costs of all chunks
    int32_t pad0[10];
    // 64-byte aligned: set to the call's epoch (nonzero) by the sorting
    // workgroup once the tables are published, back to 0 by the combine kernel
    // that ends every call
    uint32_t ready;
    int32_t wait_timeouts;    // workgroups that gave up waiting (never expected)
    int32_t pad1[46];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

// One run longer than kNRows rows: its chunks' partial sums are rows
// first_partial .. first_partial + nchunks - 1 of the partial buffer.
struct alignas(16) LongRunDesc {
    int32_t row;
    int32_t first_partial;
    int32_t nchunks;
    int32_t unused;
};
static_assert(sizeof(LongRunDesc) == 16, "long-run descriptor is 16 bytes");

// Optional outputs of the sort step (all null in the accumulate path).
struct SortTables {
    int32_t *sorted_ids;
    int32_t *positions;
    int32_t *run_first;
    int32_t *run_last;
    int32_t *long_runs;
    int32_t *chunk_first;
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte offsets inside the workspace for num_tokens tokens and `hidden` columns.
struct WsLayout {
    size_t keys;             // uint32[kMaxTokens]: sorted keys (published by the sorter)
    size_t info;             // uint32[kMaxTokens]: chunk table
    size_t cost;             // uint32[kMaxTokens + 1]: exclusive prefix of chunk costs
    size_t long_runs;        // LongRunDesc[num_tokens / 11 + 1]
    size_t partial;          // float[max_long_chunks][partial_stride]
    size_t total;
    int64_t partial_stride;  // floats per partial row
    int64_t max_long_chunks; // a run of L > 10 rows has ceil(L/10) <= 2L/11 chunks
};

inline WsLayout ws_layout(int64_t num_tokens, int64_t hidden) {
    WsLayout l;
    l.keys = sizeof(WsHeader);
    l.info = l.keys + sizeof(uint32_t) * kMaxTokens;
    l.cost = l.info + sizeof(uint32_t) * kMaxTokens;
    l.long_runs = round_up(l.cost + sizeof(uint32_t) * (kMaxTokens + 1), 256);
    l.partial = round_up(l.long_runs + sizeof(LongRunDesc) * (size_t)(num_tokens / 11 + 1), 256);
    l.partial_stride = (int64_t)round_up((size_t)hidden, 64);
    l.max_long_chunks = 2 * num_tokens / 11;
    l.total = round_up(l.partial + sizeof(float) * (size_t)l.partial_stride *
                                       (size_t)l.max_long_chunks, 256);
    return l;
}

// ---- launchers (one per kernel family; defined next to the kernels) --------

// Sort + run marking with the tables written out. One workgroup.
hipError_t launch_sort_tokens(const void *ids, bool ids_int64, int n, int num_embeddings,
                              int pos_bits, int id_bits, void *workspace, const WsLayout &l,
                              const SortTables &tables, hipStream_t stream);

// Fused sort + chunk sums over the grad rows; finishes single-chunk runs and
// writes the long-run list for the combine. One workgroup per compute unit.
// grad_bf16 / mg_bf16 select the element types; vec selects 16-byte rows.
hipError_t launch_accumulate(bool ids_int64, bool grad_bf16, bool mg_bf16, bool vec,
                             const void *ids, int n, int num_embeddings, int pos_bits, int id_bits,
                             const void *grad, int64_t grad_stride, void *main_grad,
                             int64_t mg_stride, int hidden, void *workspace, const WsLayout &l,
                             int num_cus, uint32_t epoch, hipStream_t stream);

// Ordered combine of the chunk sums of long runs; finishes them and clears
// the ready flag for the next call.
hipError_t launch_long_run_sums(bool grad_bf16, bool mg_bf16, bool vec, void *main_grad,
                                int64_t mg_stride, int hidden, void *workspace,
                                const WsLayout &l, int max_long_runs, int num_cus,
                                hipStream_t stream);

}  // namespace ewg
