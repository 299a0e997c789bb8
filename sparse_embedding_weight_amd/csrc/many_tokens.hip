// Calls of more than 8192 tokens (up to kManyMaxTokens), with the same
// arithmetic as the one-kernel path: the batch is cut into tiles of 8192
// positions, each sorted in LDS by one workgroup, and the sorted tiles are
// merged by rank instead of re-sorted. Five kernels on one stream; each
// depends only on the ones before it, so no workgroup waits for another.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad": the
// introduction (equal ids ordered by ascending position; fp32 chunk sums of
// ten consecutive rows or fewer, the chunks counted from an id's first row;
// those sums folded left to right from +0 and converted once to grad's dtype;
// the main_grad update done in fp32), _sort_tokens_kernel,
// _partial_sums_kernel and _long_run_sums_kernel. The one-program sort of at
// most 8192 keys is what bounds MAX_TOKENS there; nothing in the arithmetic
// depends on that bound.
//
//   1. tile_sort_kernel (one workgroup per tile): keys (id << 13 | position
//      in the tile) radix-sorted in LDS (sort_lds.h), written out sorted.
//   2. rank_kernel (one workgroup per 256 sorted keys of a tile, four
//      threads per key, each searching one of four tiles staged together): every
//      position of tile t precedes every position of tile t + 1, so the
//      global (id, position) rank of a key is its index in its own sorted
//      tile plus, in every earlier tile, the keys with id <= its id and, in
//      every later tile, the keys with id < its id (binary searches). The
//      same searches give its run: first rank (keys with a smaller id) and
//      length (keys with its id). Writes per rank: position, id, and a word
//      that marks the first row of every chunk (chunks of 10 counted from the
//      run's first rank) with its row count and whether the run is long.
//   3. chunk_list_kernel (one workgroup per 2048 ranks): prefix counts of the
//      marked ranks give every chunk its record (first rank, rows, main_grad
//      row, partial row for a chunk of a long run) and every long run its
//      record (row, first partial row, chunk count, first combine task).
//   4. chunk_sums_kernel: (chunk, 4 column tiles) units dealt round-robin to
//      the waves of a grid several times larger than fits at once; a chunk
//      of a run of at most 10 rows is finished into main_grad, a chunk of a
//      longer run stored as a partial row.
//   5. combine_kernel: one (long run, block of columns) task per workgroup
//      at a time: partial rows added in chunk order from +0, rounded,
//      added to main_grad (chunk_sums.h combine_block).
#include "chunk_sums.h"
#include "ewg_device.h"
#include "ewg_internal.h"
#include "sort_lds.h"

namespace ewg {
namespace {

constexpr int kTileBits = 13;              // positions inside a tile
constexpr int kTileKeys = 1 << kTileBits;  // keys one workgroup sorts
static_assert(kTileKeys == kMaxTokens, "a tile is one LDS sort");
constexpr int kRankGroup = 4;              // tiles staged and searched at once by rank_kernel
constexpr int kRankSlice = kSortThreads / kRankGroup;   // sorted keys per rank_kernel workgroup
constexpr int kListItems = 2;              // ranks per thread of chunk_list_kernel
constexpr int kListBlock = kSortThreads * kListItems;   // ranks per chunk_list_kernel workgroup
constexpr int kSumThreads = 256;           // chunk_sums_kernel workgroup
constexpr int kSumTilesPerUnit = 4;        // column tiles of one chunk per chunk-sum unit
constexpr int kSumGroupsPerCu = 64;        // chunk_sums_kernel workgroups per compute unit
// combine staging: 128 KiB, one workgroup per CU. (32 KiB, four per CU,
// measured slower: a deep run's task then needs several staging round trips
// in a row.)
constexpr int kManyStage = kStageFloats;
constexpr int kCombineGroupsPerCu = 4;     // combine_kernel workgroups per compute unit (one fits)

// Word per sorted rank: 0, or the first row of a chunk: bit 0 set, rows - 1
// in bits 1..4, bit 5 if the run has more than 10 rows, bit 6 if the chunk is
// the run's first; the first chunk of a long run carries the run's number of
// combine tasks from bit 8 (at most ceil(hidden / 128) <= 2^17).
constexpr uint32_t kHeadChunk = 1u, kHeadLong = 1u << 5, kHeadRun = 1u << 6;
constexpr int kTasksShift = 8;
constexpr uint32_t kHeadLongRun = kHeadChunk | kHeadLong | kHeadRun;

__device__ __forceinline__ bool any_bad(const ManyHeader *hdr, int tiles, int32_t *sum) {
    int32_t s = 0;
    for (int k = 0; k < tiles; ++k) s += hdr->tile_bad[k];
    *sum = s;
    return s != 0;
}

// ---- 1. tile sort ----------------------------------------------------------

template <typename IdT>
__global__ __launch_bounds__(kSortThreads) void tile_sort_kernel(const IdT *__restrict__ ids, int n,
                                                                 int num_embeddings, int id_bits,
                                                                 ManyHeader *__restrict__ hdr,
                                                                 uint32_t *__restrict__ tkeys) {
    __shared__ SortSmem sm;
    const int t = blockIdx.x, base = t * kTileKeys;
    const int nt = n - base < kTileKeys ? n - base : kTileKeys;
    const int bad = load_keys<IdT>(sm, ids + base, nt, num_embeddings, kTileBits, 0, false);
    const int cur = radix_sort_ids(sm, kTileBits, id_bits, nt);
    for (int i = threadIdx.x; i < nt; i += kSortThreads) tkeys[base + i] = sm.keys[cur][i];
    if (threadIdx.x == 0) hdr->tile_bad[t] = bad;
}

// ---- 2. global ranks -------------------------------------------------------

// Keys of `a[0, nk)` (sorted) below `key`: branch-free binary search in LDS.
__device__ __forceinline__ uint32_t lds_count_below(const uint32_t *a, uint32_t nk, uint32_t key) {
    uint32_t below = 0u;
#pragma unroll
    for (int b = kTileBits; b >= 0; --b) {
        const uint32_t c = below + (1u << b);
        if (c <= nk && a[c - 1] < key) below = c;
    }
    return below;
}

// Combine tasks of a long run of `len` rows: blocks of combine_width columns.
__device__ __forceinline__ uint32_t run_tasks(uint32_t len, int hidden) {
    const int chunks = (int)((len + kNRows - 1) / kNRows);
    const int w = combine_width<kManyStage>(chunks, hidden);
    return (uint32_t)((hidden + w - 1) / w);
}

__global__ __launch_bounds__(kSortThreads) void rank_kernel(int n, int tiles, int hidden,
                                                            const ManyHeader *__restrict__ hdr,
                                                            const uint32_t *__restrict__ tkeys,
                                                            int32_t *__restrict__ gpos,
                                                            uint32_t *__restrict__ gid,
                                                            uint32_t *__restrict__ cw,
                                                            uint32_t *__restrict__ glen) {
    __shared__ uint32_t s_tile[kRankGroup][kTileKeys];         // a group of tiles, all searched at once
    __shared__ uint32_t s_part[kRankGroup][3][kRankSlice];     // per tile lane: before, start, length
    __shared__ uint32_t s_res[3][kRankSlice];   // per id of the slice: before, run start, run length
    __shared__ uint64_t s_scan[kSortWaves + 1];
    int32_t bad;
    if (any_bad(hdr, tiles, &bad)) return;   // uniform: nothing is accumulated
    const int tid = threadIdx.x;
    // thread = (key of the slice kl, tile lane ts): the kRankGroup threads of
    // a key search one tile each of every group of tiles
    const int kl = tid % kRankSlice, ts = tid / kRankSlice;
    const int t = blockIdx.x / (kTileKeys / kRankSlice);
    const int i = (blockIdx.x % (kTileKeys / kRankSlice)) * kRankSlice + kl;   // index in the sorted tile
    const int nt = n - t * kTileKeys < kTileKeys ? n - t * kTileKeys : kTileKeys;
    const bool valid = i < nt;
    const uint32_t key = valid ? tkeys[t * kTileKeys + i] : 0xffffffffu;
    const uint32_t x = key >> kTileBits;
    const bool head = valid && (kl == 0 || (tkeys[t * kTileKeys + i - 1] >> kTileBits) != x);
    uint64_t heads;
    const uint32_t excl =
        (uint32_t)block_exclusive_scan(head && ts == 0 ? 1u : 0u, s_scan, &heads);
    const uint32_t ord = head ? excl : excl - 1u;   // for ts == 0: the slice's id groups in order

    // Each id group of the slice counts, in every tile k, the keys below x
    // and below x + 1 (ids < x, ids <= x): tiles are staged kRankGroup at a
    // time (thread j moves keys [8j, 8j + 8) of each), and the group's head
    // key is searched in tile k by its thread of lane k % kRankGroup.
    const uint32_t key_a = x << kTileBits, key_b = (x + 1u) << kTileBits;
    uint32_t before = 0u, start = 0u, len = 0u;
    for (int g0 = 0; g0 < tiles; g0 += kRankGroup) {
        uint4 r[kRankGroup][2];
#pragma unroll
        for (int q = 0; q < kRankGroup; ++q) {
            const int k = g0 + q;
            const int nk = k < tiles ? (n - k * kTileKeys < kTileKeys ? n - k * kTileKeys : kTileKeys) : 0;
            const uint4 *src = reinterpret_cast<const uint4 *>(tkeys + (size_t)k * kTileKeys);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = tid * kSortItems + 4 * h;   // first key of this piece
                r[q][h] = e < nk ? src[e / 4]
                                 : uint4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
            }
        }
        if (g0 > 0) __syncthreads();   // the previous group's searches are done
#pragma unroll
        for (int q = 0; q < kRankGroup; ++q) {
            uint4 *dst = reinterpret_cast<uint4 *>(s_tile[q]);
            dst[2 * tid] = r[q][0];
            dst[2 * tid + 1] = r[q][1];
        }
        __syncthreads();
        const int k = g0 + ts;
        if (head && k < tiles) {
            const uint32_t nk = (uint32_t)(n - k * kTileKeys < kTileKeys ? n - k * kTileKeys : kTileKeys);
            const uint32_t lo = lds_count_below(s_tile[ts], nk, key_a);
            const uint32_t hi = lds_count_below(s_tile[ts], nk, key_b);
            start += lo;
            len += hi - lo;
            if (k < t) before += hi;       // earlier positions of this id and smaller ids
            else if (k > t) before += lo;  // smaller ids only
        }
    }
    if (head) {
        s_part[ts][0][kl] = before;
        s_part[ts][1][kl] = start;
        s_part[ts][2][kl] = len;
    }
    __syncthreads();
    if (head && ts == 0) {   // the key's lane 0 adds up its lanes' counts
        before = start = len = 0u;
#pragma unroll
        for (int q = 0; q < kRankGroup; ++q) {
            before += s_part[q][0][kl];
            start += s_part[q][1][kl];
            len += s_part[q][2][kl];
        }
        s_res[0][ord] = before;
        s_res[1][ord] = start;
        s_res[2][ord] = len;
    }
    __syncthreads();
    if (ts != 0 || !valid) return;   // the rest is per key, in lane 0
    const uint32_t rank = s_res[0][ord] + (uint32_t)i;
    const uint32_t run0 = s_res[1][ord], rlen = s_res[2][ord];
    if (rank >= (uint32_t)n) return;   // never: the ranks of the n keys are 0 .. n-1
    const uint32_t off = rank - run0;
    gpos[rank] = t * kTileKeys + (int32_t)(key & (kTileKeys - 1));
    gid[rank] = x;
    uint32_t w = 0u;
    if (off % kNRows == 0) {
        const uint32_t rows = rlen - off < (uint32_t)kNRows ? rlen - off : (uint32_t)kNRows;
        w = kHeadChunk | ((rows - 1u) << 1) | (rlen > (uint32_t)kNRows ? kHeadLong : 0u);
        if (off == 0) {
            w |= kHeadRun;
            if (rlen > (uint32_t)kNRows) w |= run_tasks(rlen, hidden) << kTasksShift;
        }
    }
    cw[rank] = w;
    if (off == 0) glen[rank] = rlen;
}

// ---- 3. chunk and long-run lists -------------------------------------------

// counters packed in 21-bit fields: chunks, long runs, long chunks
__device__ __forceinline__ uint64_t head_counts(uint32_t w) {
    if (!(w & kHeadChunk)) return 0;
    const bool lng = (w & kHeadLong) != 0;
    return 1ull | ((uint64_t)(lng && (w & kHeadRun)) << 21) | ((uint64_t)lng << 42);
}

constexpr uint64_t kField = (1ull << 21) - 1;

// Four 64-bit values per thread in one pass over the workgroup: the sums
// of a and b over all threads, the exclusive prefixes of c and d in thread
// order, and the sums of c and d. Every thread must call it.
__device__ __forceinline__ void block_scan4(uint64_t a, uint64_t b, uint64_t c, uint64_t d,
                                            uint64_t (*s)[kSortWaves + 1], uint64_t *sum_a,
                                            uint64_t *sum_b, uint64_t *pre_c, uint64_t *pre_d,
                                            uint64_t *sum_c, uint64_t *sum_d) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t v[4] = {a, b, c, d};
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = wave_inclusive_scan(v[k], lane);
    if (lane == 63) {
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k][wave] = v[k];
    }
    __syncthreads();
    if (wave < 4) {   // wave k scans the wave totals of value k
        const uint64_t t = lane < kSortWaves ? s[wave][lane] : 0;
        const uint64_t ti = wave_inclusive_scan(t, lane);
        if (lane < kSortWaves) s[wave][lane] = ti - t;
        if (lane == kSortWaves - 1) s[wave][kSortWaves] = ti;
    }
    __syncthreads();
    *sum_a = s[0][kSortWaves];
    *sum_b = s[1][kSortWaves];
    *pre_c = s[2][wave] + v[2] - c;
    *pre_d = s[3][wave] + v[3] - d;
    *sum_c = s[2][kSortWaves];
    *sum_d = s[3][kSortWaves];
}

__global__ __launch_bounds__(kSortThreads) void chunk_list_kernel(int n, int tiles,
                                                                  uint32_t max_long_runs,
                                                                  uint32_t max_long_chunks,
                                                                  ManyHeader *__restrict__ hdr,
                                                                  const uint32_t *__restrict__ gid,
                                                                  const uint32_t *__restrict__ cw,
                                                                  const uint32_t *__restrict__ glen,
                                                                  u32x4 *__restrict__ chunks,
                                                                  u32x4 *__restrict__ runs) {
    __shared__ uint64_t s_scan4[4][kSortWaves + 1];
    const int tid = threadIdx.x;
    int32_t bad;
    if (any_bad(hdr, tiles, &bad)) {   // uniform
        if (blockIdx.x == 0 && tid == 0) {
            hdr->invalid_ids = bad;
            hdr->n_chunks = hdr->n_long_runs = hdr->n_long_chunks = hdr->n_tasks = 0u;
        }
        return;
    }
    const int r0 = blockIdx.x * kListBlock;
    // this block's ranks: thread j owns [r0 + 2j, r0 + 2j + 2); 8-byte loads
    // of the thread's words of each array, issued first so that they are in
    // flight with the prefix counts below (a piece past n reads workspace
    // that follows the array: its words are masked)
    static_assert(kListItems == 2, "8-byte loads of two ranks");
    const int s0 = r0 + tid * kListItems;
    uint32_t w[kListItems] = {0u, 0u}, ids8[kListItems] = {0u, 0u}, len8[kListItems] = {0u, 0u};
    if (s0 < n) {
        const uint2 a = *reinterpret_cast<const uint2 *>(cw + s0);
        const uint2 b = *reinterpret_cast<const uint2 *>(gid + s0);
        const uint2 c = *reinterpret_cast<const uint2 *>(glen + s0);
        w[0] = a.x; w[1] = a.y;
        ids8[0] = b.x; ids8[1] = b.y;
        len8[0] = c.x; len8[1] = c.y;
    }
    // counts over the ranks of earlier blocks (each block recounts them: no
    // block waits for another); 16-byte loads, 4 per thread in flight
    // together (r0 is a multiple of 4)
    uint64_t pre = 0, pre_tasks = 0;
    for (int r = tid * 4; r < r0; r += kSortThreads * 16) {
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rq = r + q * kSortThreads * 4;
            v[q] = rq < r0 ? *reinterpret_cast<const uint4 *>(cw + rq) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pre += head_counts(w4[j]);
                if ((w4[j] & kHeadLongRun) == kHeadLongRun) pre_tasks += w4[j] >> kTasksShift;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kListItems; ++j) {
        if (s0 + j >= n) w[j] = ids8[j] = len8[j] = 0u;
    }
    uint64_t mine = 0, mine_tasks = 0;
#pragma unroll
    for (int j = 0; j < kListItems; ++j) {
        mine += head_counts(w[j]);
        if ((w[j] & kHeadLongRun) == kHeadLongRun) mine_tasks += w[j] >> kTasksShift;
    }
    // one pass: totals of the earlier blocks' counts, exclusive prefixes of
    // this block's
    uint64_t base, base_tasks, all, all_tasks, idx, task;
    block_scan4(pre, pre_tasks, mine, mine_tasks, s_scan4, &base, &base_tasks, &idx, &task, &all,
                &all_tasks);
    idx += base;
    task += base_tasks;
#pragma unroll
    for (int j = 0; j < kListItems; ++j) {
        if (w[j] & kHeadChunk) {
            const uint32_t s = (uint32_t)(s0 + j);
            const uint32_t c = (uint32_t)(idx & kField);
            const uint32_t lr = (uint32_t)((idx >> 21) & kField);
            const uint32_t lc = (uint32_t)((idx >> 42) & kField);
            const bool lng = (w[j] & kHeadLong) != 0;
            const uint32_t rows = ((w[j] >> 1) & 15u) + 1u;
            const uint32_t row = ids8[j];
            // (the bounds hold by construction: at most n chunks, n / 11 long
            // runs, 2n / 11 long-run chunks)
            if (c < (uint32_t)n && (!lng || lc < max_long_chunks))
                chunks[c] = u32x4{s, rows, row, lng ? lc : 0xffffffffu};
            if (lng && (w[j] & kHeadRun) && lr < max_long_runs) {
                const uint32_t len = len8[j];
                runs[lr] = u32x4{row, lc, (len + kNRows - 1) / kNRows, (uint32_t)task};
                task += w[j] >> kTasksShift;
            }
            idx += head_counts(w[j]);
        }
    }
    if (blockIdx.x == gridDim.x - 1 && tid == 0) {
        const uint64_t tot = base + all;
        hdr->invalid_ids = 0;
        hdr->n_chunks = (uint32_t)(tot & kField);
        hdr->n_long_runs = (uint32_t)((tot >> 21) & kField);
        hdr->n_long_chunks = (uint32_t)((tot >> 42) & kField);
        hdr->n_tasks = (uint32_t)(base_tasks + all_tasks);
    }
}

// ---- 4. chunk sums ---------------------------------------------------------

// Units are (chunk, group of kSumTilesPerUnit column tiles), chunk-major;
// wave w of W takes units w, w + W, ... The grid holds several times more
// workgroups than fit at once, so the hardware hands each compute unit a new
// workgroup as one finishes: units of unequal cost even out without any
// counter.
template <typename G, typename M, int VEC>
__global__ __launch_bounds__(kSumThreads) void chunk_sums_kernel(
    int n, int num_embeddings, const ManyHeader *__restrict__ hdr,
    const u32x4 *__restrict__ chunks, const int32_t *__restrict__ gpos,
    const typename G::T *__restrict__ grad, int64_t grad_stride,
    typename M::T *__restrict__ main_grad, int64_t mg_stride, float *__restrict__ partial,
    int64_t partial_stride, uint32_t max_long_chunks, int hidden, int tiles) {
    const uint32_t n_chunks = min(hdr->n_chunks, (uint32_t)n);
    const uint32_t groups = (uint32_t)((tiles + kSumTilesPerUnit - 1) / kSumTilesPerUnit);
    const uint32_t units = n_chunks * groups;
    const int full_tiles = hidden / (64 * VEC);
    const uint32_t waves = gridDim.x * (kSumThreads / 64);
    for (uint32_t u = blockIdx.x * (kSumThreads / 64) + (threadIdx.x >> 6); u < units; u += waves) {
        const uint32_t c = u / groups, g = u - c * groups;
        const u32x4 rec = chunks[c];
        const uint32_t s = __builtin_amdgcn_readfirstlane(rec.x);
        const uint32_t row = __builtin_amdgcn_readfirstlane(rec.z);
        const uint32_t dest = __builtin_amdgcn_readfirstlane(rec.w);
        int rows = (int)__builtin_amdgcn_readfirstlane(rec.y);
        rows = rows < 1 ? 1 : (rows > kNRows ? kNRows : rows);
        // a record outside this call's ranges (never expected) is skipped
        if (row >= (uint32_t)num_embeddings || s + (uint32_t)rows > (uint32_t)n ||
            (dest != 0xffffffffu && dest >= max_long_chunks))
            continue;
        int32_t pos[kNRows];
#pragma unroll
        for (int r = 0; r < kNRows; ++r) {
            const int32_t p = r < rows ? gpos[s + r] : 0;
            pos[r] = __builtin_amdgcn_readfirstlane(p >= 0 && p < n ? p : 0);   // inside grad
        }
        const int t0 = (int)g * kSumTilesPerUnit;
        const int t_end = t0 + kSumTilesPerUnit < tiles ? t0 + kSumTilesPerUnit : tiles;
        // plain stores: only the combine kernel, launched after this one, reads the sums
        chunk_tiles_any<G, M, VEC, 0>(pos, rows, (int)row, dest == 0xffffffffu ? -1 : (int)dest,
                                   grad, grad_stride, main_grad, mg_stride, partial,
                                   partial_stride, hidden, t0, t_end, full_tiles);
    }
}

// ---- 5. ordered combine ----------------------------------------------------

template <typename G, typename M>
__global__ __launch_bounds__(kSortThreads) void combine_kernel(
    int num_embeddings, const ManyHeader *__restrict__ hdr, const u32x4 *__restrict__ runs,
    const float *__restrict__ partial, int64_t partial_stride, typename M::T *__restrict__ main_grad,
    int64_t mg_stride, uint32_t max_long_chunks, uint32_t max_long_runs, int hidden) {
    __shared__ float stage[kManyStage];
    __shared__ uint32_t s_run;
    const uint32_t n_tasks = hdr->n_tasks;
    const int n_lr = (int)min(hdr->n_long_runs, max_long_runs);
    for (uint32_t t = blockIdx.x; t < n_tasks; t += gridDim.x) {
        // the run: the last one whose first task is at or before t (first
        // tasks never decrease). The first wave probes 64 records at once,
        // narrowing the range 64-fold per round trip.
        if (threadIdx.x < 64) {
            const uint32_t lane = threadIdx.x;
            uint32_t lo = 0u, hi = n_lr > 0 ? (uint32_t)n_lr : 1u;
            while (hi - lo > 1u) {
                const uint32_t step = (hi - lo + 63u) / 64u;
                const uint32_t idx = lo + lane * step;
                const uint32_t v = idx < hi ? runs[idx].w : 0xffffffffu;
                const uint64_t m = __ballot(v <= t);   // lanes 0 .. k: a prefix
                const uint32_t k = m ? 63u - (uint32_t)__clzll((long long)m) : 0u;
                lo += k * step;
                hi = min(hi, lo + step);
            }
            if (lane == 0) s_run = lo;
        }
        __syncthreads();
        const u32x4 rec = runs[s_run];
        const uint32_t row = rec.x, first = rec.y, chunks = rec.z;
        const int wdt = combine_width<kManyStage>((int)chunks, hidden);
        const int64_t col0 = (int64_t)(t - rec.w) * wdt;
        // a record that does not describe this call's work (never expected) is skipped
        const bool valid = n_lr >= 1 && rec.w <= t && row < (uint32_t)num_embeddings &&
                           chunks >= 1 && first < max_long_chunks &&
                           chunks <= max_long_chunks - first && col0 < hidden;
        if (valid)   // uniform
            // 16 LDS reads in flight per group of adds (measured: 8 on the one-kernel path)
            combine_block<G, M, kManyStage, 0, 16>(stage, row, first, chunks, col0, wdt, partial,
                                            partial_stride, main_grad, mg_stride, hidden);
        __syncthreads();   // stage and s_run are free for the next task
    }
}

// ---- launch ----------------------------------------------------------------

template <typename IdT, typename G, typename M, int VEC>
hipError_t launch(const void *ids, int n, int num_embeddings, int id_bits, const void *grad,
                  int64_t grad_stride, void *main_grad, int64_t mg_stride, int hidden,
                  void *workspace, const ManyLayout &l, int num_cus, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    ManyHeader *hdr = reinterpret_cast<ManyHeader *>(ws);
    uint32_t *tkeys = reinterpret_cast<uint32_t *>(ws + l.tkeys);
    int32_t *gpos = reinterpret_cast<int32_t *>(ws + l.gpos);
    uint32_t *gid = reinterpret_cast<uint32_t *>(ws + l.gid);
    uint32_t *cw = reinterpret_cast<uint32_t *>(ws + l.cw);
    uint32_t *glen = reinterpret_cast<uint32_t *>(ws + l.glen);
    u32x4 *chunks = reinterpret_cast<u32x4 *>(ws + l.chunks);
    u32x4 *runs = reinterpret_cast<u32x4 *>(ws + l.runs);
    float *partial = reinterpret_cast<float *>(ws + l.partial);
    const int tiles = (n + kTileKeys - 1) / kTileKeys;
    const int col_tiles = (hidden + 64 * VEC - 1) / (64 * VEC);

    tile_sort_kernel<IdT><<<tiles, kSortThreads, 0, stream>>>(
        static_cast<const IdT *>(ids), n, num_embeddings, id_bits, hdr, tkeys);
    rank_kernel<<<tiles * (kTileKeys / kRankSlice), kSortThreads, 0, stream>>>(
        n, tiles, hidden, hdr, tkeys, gpos, gid, cw, glen);
    chunk_list_kernel<<<(n + kListBlock - 1) / kListBlock, kSortThreads, 0, stream>>>(
        n, tiles, (uint32_t)l.max_long_runs, (uint32_t)l.max_long_chunks, hdr, gid, cw, glen,
        chunks, runs);
    chunk_sums_kernel<G, M, VEC><<<num_cus * kSumGroupsPerCu, kSumThreads, 0, stream>>>(
        n, num_embeddings, hdr, chunks, gpos, static_cast<const typename G::T *>(grad),
        grad_stride, static_cast<typename M::T *>(main_grad), mg_stride, partial, l.partial_stride,
        (uint32_t)l.max_long_chunks, hidden, col_tiles);
    combine_kernel<G, M><<<num_cus * kCombineGroupsPerCu, kSortThreads, 0, stream>>>(
        num_embeddings, hdr, runs, partial, l.partial_stride,
        static_cast<typename M::T *>(main_grad), mg_stride, (uint32_t)l.max_long_chunks,
        (uint32_t)l.max_long_runs, hidden);
    return hipGetLastError();
}

template <typename IdT>
hipError_t dispatch_types(bool grad_bf16, bool mg_bf16, bool vec, const void *ids, int n,
                          int num_embeddings, int id_bits, const void *grad, int64_t grad_stride,
                          void *main_grad, int64_t mg_stride, int hidden, void *workspace,
                          const ManyLayout &l, int num_cus, hipStream_t stream) {
#define EWG_MANY(G, M, V)                                                                       \
    launch<IdT, G, M, V>(ids, n, num_embeddings, id_bits, grad, grad_stride, main_grad, mg_stride, \
                         hidden, workspace, l, num_cus, stream)
    if (grad_bf16) {
        if (mg_bf16) return vec ? EWG_MANY(BF16, BF16, 8) : EWG_MANY(BF16, BF16, 1);
        return vec ? EWG_MANY(BF16, F32, 8) : EWG_MANY(BF16, F32, 1);
    }
    if (mg_bf16) return vec ? EWG_MANY(F32, BF16, 4) : EWG_MANY(F32, BF16, 1);
    return vec ? EWG_MANY(F32, F32, 4) : EWG_MANY(F32, F32, 1);
#undef EWG_MANY
}

}  // namespace

hipError_t launch_many_tokens(bool ids_int64, bool grad_bf16, bool mg_bf16, bool vec,
                              const void *ids, int n, int num_embeddings, int id_bits,
                              const void *grad, int64_t grad_stride, void *main_grad,
                              int64_t mg_stride, int hidden, void *workspace,
                              const ManyLayout &l, int num_cus, hipStream_t stream) {
    if (ids_int64)
        return dispatch_types<int64_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, id_bits,
                                       grad, grad_stride, main_grad, mg_stride, hidden, workspace,
                                       l, num_cus, stream);
    return dispatch_types<int32_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, id_bits, grad,
                                   grad_stride, main_grad, mg_stride, hidden, workspace, l,
                                   num_cus, stream);
}

}  // namespace ewg
