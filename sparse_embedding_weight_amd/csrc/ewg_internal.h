// Internal layout shared by the three kernels and the host entry points of
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
    int32_t invalid_ids;     // ids outside [0, num_embeddings) seen by the last call
    int32_t num_chunks;      // chunks of all runs
    int32_t num_long_runs;   // runs longer than kNRows rows
    int32_t num_long_chunks; // chunks of those runs = rows of the partial buffer in use
    int32_t num_runs;        // distinct ids
    int32_t pad[59];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

// One chunk: up to kNRows grad rows of one id, in position order.
struct alignas(16) ChunkDesc {
    int32_t row;        // id = main_grad row
    int32_t dest;       // -1: the run is this one chunk, finish into main_grad;
                        // else the partial-buffer row of this chunk's fp32 sum
    int32_t nrows;      // 1..kNRows
    int32_t unused;
    int32_t pos[12];    // grad rows (positions), pos[0..nrows)
};
static_assert(sizeof(ChunkDesc) == 64, "chunk descriptor is 64 bytes");

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
    size_t chunks;           // ChunkDesc[num_tokens]
    size_t long_runs;        // LongRunDesc[num_tokens / 11 + 1]
    size_t partial;          // float[max_long_chunks][partial_stride]
    size_t total;
    int64_t partial_stride;  // floats per partial row
    int64_t max_long_chunks; // a run of L > 10 rows has ceil(L/10) <= 2L/11 chunks
};

inline WsLayout ws_layout(int64_t num_tokens, int64_t hidden) {
    WsLayout l;
    l.chunks = sizeof(WsHeader);
    l.long_runs = round_up(l.chunks + sizeof(ChunkDesc) * (size_t)num_tokens, 256);
    l.partial = round_up(l.long_runs + sizeof(LongRunDesc) * (size_t)(num_tokens / 11 + 1), 256);
    l.partial_stride = (int64_t)round_up((size_t)hidden, 64);
    l.max_long_chunks = 2 * num_tokens / 11;
    l.total = round_up(l.partial + sizeof(float) * (size_t)l.partial_stride *
                                       (size_t)l.max_long_chunks, 256);
    return l;
}

// ---- launchers (one per kernel family; defined next to the kernels) --------

// Sort + run marking + work lists. One workgroup.
hipError_t launch_sort_tokens(const void *ids, bool ids_int64, int n, int num_embeddings,
                              int pos_bits, int id_bits, void *workspace, const WsLayout &l,
                              const SortTables &tables, hipStream_t stream);

// Chunk sums over grad rows; finishes single-chunk runs.
// grad_bf16 / mg_bf16 select the element types; vec selects 16-byte rows.
hipError_t launch_partial_sums(bool grad_bf16, bool mg_bf16, bool vec, const void *grad,
                               int64_t grad_stride, void *main_grad, int64_t mg_stride,
                               int hidden, void *workspace, const WsLayout &l,
                               int max_chunks, int num_cus, hipStream_t stream);

// Ordered combine of the chunk sums of long runs; finishes them.
hipError_t launch_long_run_sums(bool grad_bf16, bool mg_bf16, bool vec, void *main_grad,
                                int64_t mg_stride, int hidden, void *workspace,
                                const WsLayout &l, int max_long_runs, int num_cus,
                                hipStream_t stream);

}  // namespace ewg
