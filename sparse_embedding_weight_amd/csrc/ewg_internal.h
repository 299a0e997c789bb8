// Internal layout shared by the kernels and the host entry points of
// libembedding_wgrad.so. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "embedding_wgrad.h"

namespace ewg {

constexpr int kNRows = 10;           // rows per partial sum (NROWS_PER_THREAD)
constexpr int kMaxTokens = 8192;     // keys one LDS sort holds
constexpr int kSortThreads = 1024;   // sort workgroup: 16 waves of 64
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = kMaxTokens / kSortThreads;   // keys per thread
constexpr int kMaxDigitBits = 10;    // radix digit of one sort pass

// Workspace header, at offset 0: eight 128-byte cache lines. invalid_ids is
// the documented first int32. Line 0 is written with plain stores by the sort
// step and read only by the host; the other lines are only accessed with
// device-coherent loads, stores and atomics. Device-scope atomics on one
// address are serialised (about 11 ns each on MI355X), so every counter that
// many workgroups update has a line of its own and is touched once per
// workgroup, not once per wave.
constexpr int kExitGroups = 8;       // exit counters: one per group of workgroups (XCD)

struct WsHeader {
    // line 0
    int32_t invalid_ids;      // ids outside [0, num_embeddings) seen by the last call
    int32_t num_chunks;       // chunks of all runs
    int32_t num_long_runs;    // runs longer than kNRows rows
    int32_t num_long_chunks;  // chunks of those runs
    int32_t num_runs;         // distinct ids
    int32_t pad0[27];
    // line 1: published by the sorting workgroup, then `ready` is set to the
    // call's epoch (nonzero); the last workgroup to finish sets it back to 0
    // (ready and the three counts form one 16-byte word, read by one load)
    uint32_t ready;
    uint32_t pub_blocks;      // column blocks of long runs in this call
    uint32_t pub_long_chunks; // long chunks of this call
    uint32_t pub_long_runs;   // long runs of this call
    int32_t wait_timeouts;    // bounded waits that gave up, and records that did not
                              // belong to the call (never expected)
    int32_t check_failures;   // device-side bounds checks that failed (checked builds only)
    int32_t pad1[26];
    // line 2: next column block of a long run to hand out
    uint32_t block_ticket;
    int32_t pad2[31];
    // line 3: groups of workgroups that have finished
    uint32_t exit_top;
    int32_t pad3[31];
    // lines 4-7: workgroups of each group that have finished, 64 bytes apart
    uint32_t exit_group[kExitGroups][16];
};
static_assert(sizeof(WsHeader) == 1024, "header is eight 128-byte lines");
static_assert(offsetof(WsHeader, wait_timeouts) == EWG_WS_WAIT_TIMEOUTS_OFFSET,
              "documented diagnostic word");
static_assert(offsetof(WsHeader, check_failures) == EWG_WS_CHECK_FAILURES_OFFSET,
              "documented diagnostic word");

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

constexpr int kMaxGrid = 4095;       // workgroups of one launch, at most

// Byte offsets inside the workspace for num_tokens tokens and `hidden` columns.
// The header has a fixed place; everything after it depends on the sizes and
// is written by a call before that call reads it.
struct WsLayout {
    size_t units;            // 32-byte record per long chunk (positions, rows, run)
    size_t runs;             // 16-byte record per long run (row, first chunk, chunks and
                             // block width, first block)
    size_t total;
    int64_t max_long_chunks; // a run of L > 10 rows has ceil(L/10) <= 2L/11 chunks
    int64_t max_long_runs;   // a long run has at least 11 rows
};

constexpr size_t kUnitRecordBytes = 32;
constexpr size_t kRunRecordBytes = 16;

// The workspace holds the header and the records of the long runs only: the
// chunk sums of a long run never leave the compute unit that folds them, so
// its size does not depend on hidden (the argument stays for the interface).
inline WsLayout ws_layout(int64_t num_tokens, int64_t hidden) {
    (void)hidden;
    WsLayout l;
    l.max_long_chunks = 2 * num_tokens / 11;
    l.max_long_runs = num_tokens / 11;
    l.units = sizeof(WsHeader);
    l.runs = round_up(l.units + kUnitRecordBytes * (size_t)(l.max_long_chunks + 1), 256);
    l.total = round_up(l.runs + kRunRecordBytes * (size_t)(l.max_long_runs + 1), 256);
    return l;
}

// ---- calls of more than kMaxTokens tokens (many_tokens.hip) ------------------

constexpr int kManyMaxTokens = EWG_MANY_MAX_TOKENS;
static_assert(kManyMaxTokens % 8192 == 0, "whole tiles");
constexpr int kManyMaxTiles = kManyMaxTokens / kMaxTokens;  // tiles of one LDS sort each

// First bytes of the workspace of a many-token call. The first int32 is the
// invalid-id count, as in the one-kernel workspace; the rest is written by
// every call before it is read. It lies in line 0 of WsHeader (host-read
// counts only), and the many-token arrays start after the whole WsHeader, so
// a many-token call never touches the one-kernel path's flags and counters
// (lines 1-7) and one buffer may serve both paths in turn.
struct ManyHeader {
    int32_t invalid_ids;
    uint32_t n_chunks, n_long_runs, n_long_chunks, n_tasks;
    int32_t tile_bad[kManyMaxTiles];   // invalid ids per tile
};
static_assert(sizeof(ManyHeader) <= 128, "many-token header fits line 0 of WsHeader");

struct ManyLayout {
    size_t tkeys;            // uint32 per position: each tile's keys, sorted
    size_t gpos, gid, cw, glen;  // per global rank: position, id, chunk-head word, run length
    size_t chunks;           // 16-byte record per chunk (first rank, rows, row, partial row)
    size_t runs;             // 16-byte record per long run (row, first partial row, chunks, first task)
    size_t partial;          // float[max_long_chunks][partial_stride]
    size_t total;
    int64_t partial_stride;
    int64_t max_long_chunks;
    int64_t max_long_runs;
};

inline ManyLayout many_layout(int64_t num_tokens, int64_t hidden) {
    ManyLayout l;
    const size_t n = (size_t)num_tokens;
    const size_t tiles = (n + kMaxTokens - 1) / kMaxTokens;
    l.max_long_chunks = 2 * num_tokens / 11;
    l.max_long_runs = num_tokens / 11;
    l.tkeys = sizeof(WsHeader);
    l.gpos = round_up(l.tkeys + 4 * tiles * kMaxTokens, 256);
    l.gid = round_up(l.gpos + 4 * n, 256);
    l.cw = round_up(l.gid + 4 * n, 256);
    l.glen = round_up(l.cw + 4 * n, 256);
    l.chunks = round_up(l.glen + 4 * n, 256);
    l.runs = round_up(l.chunks + 16 * n, 256);
    l.partial = round_up(l.runs + 16 * (size_t)(l.max_long_runs + 1), 256);
    l.partial_stride = (int64_t)round_up((size_t)hidden, 64);
    l.total = round_up(l.partial + sizeof(float) * (size_t)l.partial_stride *
                                       (size_t)l.max_long_chunks, 256);
    return l;
}

// ---- launchers (one per kernel family; defined next to the kernels) --------

// Sort + run marking with the tables written out. One workgroup.
hipError_t launch_sort_tokens(const void *ids, bool ids_int64, int n, int num_embeddings,
                              int pos_bits, int id_bits, void *workspace, const WsLayout &l,
                              const SortTables &tables, hipStream_t stream);

// The whole accumulation in one kernel: sort, chunk sums over the grad rows,
// single-chunk runs finished, ordered combine of long runs. One workgroup per
// compute unit. grad_bf16 / mg_bf16 select the element types; vec selects
// 16-byte rows. Row v of main_grad belongs to id id_base + v, for v below
// num_embeddings; with skip_outside other ids are left out, else they are
// invalid (the call then touches nothing and reports them). odd_skip_long
// (tests only): odd-numbered workgroups take no column block of a long run.
// Calls of kMaxTokens < n <= kManyMaxTokens tokens (any n >= 1 works): five
// kernels (tile sort, ranks, chunk lists, chunk sums, ordered combine), same
// arithmetic as launch_accumulate. Ids must lie in [0, num_embeddings) with
// num_embeddings <= 2^18; otherwise the call touches nothing and reports them.
hipError_t launch_many_tokens(bool ids_int64, bool grad_bf16, bool mg_bf16, bool vec,
                              const void *ids, int n, int num_embeddings, int id_bits,
                              const void *grad, int64_t grad_stride, void *main_grad,
                              int64_t mg_stride, int hidden, void *workspace,
                              const ManyLayout &l, int num_cus, hipStream_t stream);

hipError_t launch_accumulate(bool ids_int64, bool grad_bf16, bool mg_bf16, bool vec,
                             const void *ids, int n, int num_embeddings, int64_t id_base,
                             bool skip_outside, int pos_bits, int id_bits,
                             const void *grad, int64_t grad_stride, void *main_grad,
                             int64_t mg_stride, int hidden, void *workspace, const WsLayout &l,
                             int num_cus, uint32_t epoch, int odd_skip_long,
                             hipEvent_t kstart, hipEvent_t kstop, hipStream_t stream);

}  // namespace ewg
