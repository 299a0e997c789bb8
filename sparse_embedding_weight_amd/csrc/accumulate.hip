// The whole accumulation in one kernel: sort, chunk sums, single-chunk runs
// finished in place, and the ordered combine of long runs. One 1024-thread
// workgroup per compute unit (at least two workgroups).
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad": the
// introduction's two bullets (sort the ids with their positions, sum each
// token's rows in position order into fp32 partial sums of up to 10 rows, add
// the partial sums in order from 0, round once to the gradient dtype, add in
// fp32 into main_grad and round to its dtype), _sort_tokens_kernel,
// _partial_sums_kernel (a run of at most NROWS rows is finished there) and
// _long_run_sums_kernel (the partial sums of a longer run added in order).
//
// Phases of one launch:
//   1. Workgroup 0 (dispatched first, it never waits for anyone) radix-sorts
//      the packed keys in LDS (sort_lds.h) and writes, with device-coherent
//      stores, one record per chunk of a run longer than 10 rows (its row
//      positions and run), one per such run (main_grad row, first chunk, chunk
//      count, first combine task). Once every store has completed it sets
//      the ready flag to the call's epoch (a nonzero number per call).
//   2. Meanwhile every other workgroup builds an LDS hash table of the ids
//      and finishes its equal-cost share of the runs of at most 10 rows (a run
//      of at most 10 rows is one chunk: it needs its rows in position order,
//      not a global sort).
//   3. The first wave of a workgroup to be done with its short runs waits
//      for the flag, claims the workgroup's fixed share of the (long chunk,
//      column tile) units and stages its records in LDS; every wave takes
//      units as soon as it is done with its short runs and that is staged
//      (no barrier in between), stores their fp32 chunk sums in the partial
//      buffer with device-coherent stores and, once all have completed, the
//      workgroup adds its count of each run's units to that run's counter for
//      its group of workgroups.
//   4. Then whole workgroups take combine tasks (one long run, one block of
//      columns) from a ticket counter: wait until the run's units are all
//      counted, stage its chunk sums in LDS, add them in chunk order from +0,
//      round, add to main_grad, round.
//   5. The last workgroup to finish clears the ticket, the exit counters and
//      the flag for the next call. (These live in the workspace header, whose
//      place does not depend on the sizes of a call; the per-run counters do,
//      so workgroup 0 zeroes them before it raises the flag.)
// Device-scope atomics on one address are serialised, and a wave's atomic
// that returns a value also holds back its later loads (the vector memory
// counter drains in order), so the kernel claims fine-grained work through
// LDS counters and touches every shared counter about once per workgroup.
// The flag is raised by workgroup 0, which waits for nothing before it; a
// combine task waits only for the long units of the shares of other
// workgroups, which wait for nothing but the flag. If such a wait lasts long
// (200 us: some workgroups of the launch have not started, because more were
// launched than fit or other work holds compute units), the waiting workgroup
// claims the run's unclaimed shares and sums them itself, so every wait ends
// whatever number of workgroups runs at once. Every wait is bounded; a wait
// that gives up is counted in the workspace header and its work skipped.
//
// A column tile is 64 lanes x VEC columns (8 for bf16 grad, 4 for fp32), laid
// out in lane-contiguous pieces (piece_cols in ewg_device.h).
#include <hip/hip_ext.h>

#include "chunk_sums.h"
#include "ewg_device.h"
#include "ewg_internal.h"
#include "sort_lds.h"

namespace ewg {
namespace {

constexpr int64_t kWaitLimit = 1 << 22;  // polls before a wait gives up (seconds)
constexpr uint64_t kStealAfterTicks = 20000;   // 200 us of the 100 MHz clock: a combine task
                                               // then takes the run's unclaimed long shares
constexpr int kHashSlots = 16384;        // > 2 x kMaxTokens: linear probing always ends
constexpr int kHashBits = 14;
constexpr int kOwnedMax = 256;           // short runs gathered per round by one follower
constexpr uint32_t kNoSlot = 0xffffu;    // slot of a position whose id is left out
constexpr int kMaxLongRuns = kMaxTokens / 11;
constexpr int kMaxLongChunks = 2 * kMaxTokens / 11;

struct FollowerSmem {
    uint32_t key[kHashSlots];               // (id + 1) | first position << (32 - position bits); 0 = empty
    uint32_t cnt[kHashSlots];               // occurrences (saturating at 11) | (round-local run + 1) << 16
    uint16_t slot_of_pos[kMaxTokens];
    uint16_t run_pos[kOwnedMax][kNRows];
    uint32_t run_len[kOwnedMax];
    uint32_t run_id[kOwnedMax];
    uint32_t run_slot[kOwnedMax];
    uint64_t scan[kSortWaves + 1];
    uint32_t scan32[kSortWaves + 1];
    int bad;
    uint32_t first_rank;   // number of this follower's first run
    uint32_t n_mine;       // runs in this follower's share
    uint32_t next_unit;    // next (run, tile group) unit of the round to claim
};

struct CombineSmem {
    float stage[kStageFloats];              // chunk sums of one task, [chunk][column]
    u32x4 runs[kMaxLongRuns + 1];           // run records: row, first chunk, chunks, first task
};

struct LongSmem {
    u32x4 rec[2 * kMaxLongChunks];      // unit records of this workgroup's chunks, two halves each
    uint32_t run_cnt[kMaxLongRuns];     // units of each long run this workgroup has finished
    uint32_t claim;                     // next unit of this workgroup's share to claim
};
// A wave may stage a long share while its siblings still take short-run units
// of their last round, which read only the run tables after the hash table:
// the long share's LDS must lie inside the (then unused) hash keys.
static_assert(sizeof(LongSmem) <= sizeof(uint32_t) * kHashSlots, "long share overlaps live LDS");
// a take-over between two combine tasks keeps the run records staged for them
static_assert(sizeof(LongSmem) <= offsetof(CombineSmem, runs), "long share overlaps the run records");
static_assert(offsetof(FollowerSmem, key) == 0, "hash keys first");

union AccSmem {
    SortSmem sort;
    FollowerSmem fol;
    LongSmem lng;
    CombineSmem comb;
};

__device__ __forceinline__ uint32_t hash_home(uint32_t id) {
    return (id * 0x9E3779B1u) >> (32 - kHashBits);
}

// Follower part 1: the runs of at most 10 rows in this follower's share.
// Every follower inserts all ids into its LDS hash table (occurrences and the
// first position per id, the slot of every position). The first position
// shares the key word with the id: id + 1 fills the low 32 - pos_bits bits
// (the 31-bit key packing bounds id + 1 by 2^(31 - pos_bits)), the position
// the bits above, so that an atomic minimum over the words of one id keeps
// its smallest position. Walking the positions
// in order, the first occurrence of every id with at most 10 occurrences
// carries the byte cost of its run; follower `me` takes the runs whose cost
// prefix starts in [me, me + 1) * total / followers. That order and those
// costs depend only on the ids, so all followers agree without talking. The
// positions of the taken runs are gathered in rounds of up to kOwnedMax runs,
// put in order, and the runs finished in main_grad.
template <typename IdT, typename G, typename M, int VEC>
__device__ __forceinline__ void follower_short_runs(FollowerSmem &fs, const IdT *__restrict__ ids,
                                                    int n, int num_embeddings, int64_t id_base,
                                                    bool skip_outside, int pos_bits,
                                                    const typename G::T *__restrict__ grad,
                                                    int64_t grad_stride,
                                                    typename M::T *__restrict__ main_grad,
                                                    int64_t mg_stride, int hidden, int tiles,
                                                    int me, int followers) {
    const int tid = threadIdx.x;
    constexpr int kSlotsPerThread = kHashSlots / kSortThreads;
    const int id_shift = 32 - pos_bits;
    const uint32_t id_mask = (1u << id_shift) - 1u;

    // load the ids (all 8 loads in flight) while the table is cleared
    int64_t id[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int p = i * kSortThreads + tid;
        id[i] = (int64_t)ids[p < n ? p : n - 1];
    }
#pragma unroll
    for (int k = 0; k < kSlotsPerThread / 4; ++k) {   // 16-byte stores
        reinterpret_cast<u32x4 *>(fs.key)[k * kSortThreads + tid] = u32x4{0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4 *>(fs.cnt)[k * kSortThreads + tid] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid == 0) fs.bad = 0;
    __syncthreads();

    // insert: occurrences per id, slot per position (kNoSlot for a position
    // whose id is left out)
    int bad = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int p = i * kSortThreads + tid;
        if (p >= n) continue;
        const int64_t v = id[i] - id_base;
        if (v < 0 || v >= num_embeddings) {
            if (!skip_outside) ++bad;
            fs.slot_of_pos[p] = (uint16_t)kNoSlot;
            continue;
        }
        const uint32_t k1 = (uint32_t)v + 1u;
        const uint32_t kp = k1 | ((uint32_t)p << id_shift);
        uint32_t h = hash_home((uint32_t)v);
        for (;;) {
            uint32_t cur = fs.key[h];
            if (cur == 0u) {
                cur = atomicCAS(&fs.key[h], 0u, kp);
                if (cur == 0u) break;   // a new id, with this first position
            }
            if ((cur & id_mask) == k1) {   // the id is here: keep the smaller position
                if ((cur >> id_shift) > (uint32_t)p) atomicMin(&fs.key[h], kp);
                break;
            }
            h = (h + 1u) & (kHashSlots - 1);
        }
        // counts saturate just above kNRows (only "at most 10 rows" matters), so
        // a frequent id stops taking atomics on its slot once it is known to be long
        if (fs.cnt[h] <= (uint32_t)kNRows) atomicAdd(&fs.cnt[h], 1u);
        fs.slot_of_pos[p] = (uint16_t)h;
    }
    if (bad) atomicAdd(&fs.bad, bad);
    __syncthreads();
    if (fs.bad) return;   // uniform: the sorting workgroup reports it, nothing is touched

    // per-tile byte cost of a run of c rows, in 16-byte lane loads; an item's
    // scanned word is its cost | 1 << kCostBits (one run), so that the scan
    // sums costs below bit kCostBits and counts runs above
    constexpr uint32_t row_cost = (uint32_t)(VEC * sizeof(typename G::T) + 15) / 16;
    constexpr uint32_t end_cost = 2u * (uint32_t)(VEC * sizeof(typename M::T) + 15) / 16;
    constexpr int kCostBits = 17;
    constexpr uint32_t kCostMask = (1u << kCostBits) - 1u;
    static_assert((uint64_t)kMaxTokens * (kNRows * row_cost + end_cost) <= kCostMask &&
                      kMaxTokens < (1u << (32 - kCostBits)),
                  "costs and run counts share one 32-bit word");
    const int full_tiles = hidden / (64 * VEC);
    const int groups = (tiles + kTilesPerUnit - 1) / kTilesPerUnit;

    for (int r0 = 0;; r0 += kOwnedMax) {
        if (tid == 0) {
            fs.first_rank = 0xffffffffu;
            fs.n_mine = 0u;
            fs.next_unit = 0u;
        }
        // positions in blocked order: thread t owns [8t, 8t + 8), whose slots
        // it reads with one 16-byte load
        const int p0 = tid * kSortItems;
        static_assert(kSortItems == 8, "eight 16-bit slots per thread");
        const u32x4 sw = reinterpret_cast<const u32x4 *>(fs.slot_of_pos)[tid];
        const uint32_t sw4[4] = {sw.x, sw.y, sw.z, sw.w};
        uint32_t v[kSortItems];
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const int p = p0 + j;
            v[j] = 0;
            const uint32_t h = p < n ? (sw4[j >> 1] >> (16 * (j & 1))) & 0xffffu : kNoSlot;
            if (h != kNoSlot) {
                const uint32_t c = fs.cnt[h] & 0xffffu;
                if ((fs.key[h] >> id_shift) == (uint32_t)p && c <= (uint32_t)kNRows)
                    v[j] = (c * row_cost + end_cost) | (1u << kCostBits);
            }
            sum += v[j];
        }
        uint32_t total;
        const uint32_t run = block_exclusive_scan32(sum, fs.scan32, &total);
        const uint64_t cost_all = total & kCostMask;
        const uint64_t lo = cost_all * (uint64_t)me / (uint64_t)followers;
        const uint64_t hi = cost_all * (uint64_t)(me + 1) / (uint64_t)followers;
        // runs are numbered in position order; this follower's (cost start in
        // [lo, hi)) are a contiguous range of numbers
        {
            uint32_t x = run;
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < kSortItems; ++j) {
                const uint64_t start = x & kCostMask;
                if (v[j] && start >= lo && start < hi) {
                    atomicMin(&fs.first_rank, x >> kCostBits);
                    ++mine;
                }
                x += v[j];
            }
            if (mine) atomicAdd(&fs.n_mine, mine);
        }
        __syncthreads();
        const uint32_t first = fs.first_rank;
        const int total_mine = (int)fs.n_mine;
        {
            uint32_t x = run;
#pragma unroll
            for (int j = 0; j < kSortItems; ++j) {
                const uint64_t start = x & kCostMask;
                if (v[j] && start >= lo && start < hi) {
                    const int li = (int)((x >> kCostBits) - first) - r0;
                    if (li >= 0 && li < kOwnedMax) {
                        const uint32_t h = fs.slot_of_pos[p0 + j];
                        fs.run_id[li] = (fs.key[h] & id_mask) - 1u;
                        fs.run_len[li] = 0u;
                        fs.run_slot[li] = h;
                        fs.cnt[h] |= (uint32_t)(li + 1) << 16;
                    }
                }
                x += v[j];
            }
        }
        __syncthreads();
        const int n_round = total_mine - r0 < kOwnedMax ? total_mine - r0 : kOwnedMax;
        if (n_round <= 0) break;
        const bool last_round = total_mine - r0 <= kOwnedMax;

        // gather the positions of the round's runs, then put each run in order
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            const int p = i * kSortThreads + tid;
            if (p >= n || fs.slot_of_pos[p] == kNoSlot) continue;
            const uint32_t m = fs.cnt[fs.slot_of_pos[p]] >> 16;
            if (m) {
                const uint32_t k = atomicAdd(&fs.run_len[m - 1u], 1u);
                fs.run_pos[m - 1u][k] = (uint16_t)p;
            }
        }
        __syncthreads();
        if (tid < n_round) {
            const int len = (int)fs.run_len[tid];
            uint16_t q[kNRows];
#pragma unroll
            for (int r = 0; r < kNRows; ++r) q[r] = r < len ? fs.run_pos[tid][r] : (uint16_t)0xffff;
#pragma unroll
            for (int a = 1; a < kNRows; ++a)   // insertion sort, fixed network of compares
#pragma unroll
                for (int b = a; b > 0; --b)
                    if (q[b] < q[b - 1]) {
                        const uint16_t x = q[b];
                        q[b] = q[b - 1];
                        q[b - 1] = x;
                    }
#pragma unroll
            for (int r = 0; r < kNRows; ++r) fs.run_pos[tid][r] = q[r];
        }
        __syncthreads();

        // (run, group of kTilesPerUnit tiles) units, claimed by the waves as they come free
        const int units = n_round * groups;
        for (;;) {
            uint32_t claim = 0;
            if ((tid & 63) == 0) claim = atomicAdd(&fs.next_unit, 1u);
            const int u = (int)__builtin_amdgcn_readfirstlane(claim);
            if (u >= units) break;
            const int li = u / groups, g = u - li * groups;
            const int nrows = (int)__builtin_amdgcn_readfirstlane(fs.run_len[li]);
            const int row = (int)__builtin_amdgcn_readfirstlane(fs.run_id[li]);
            int32_t pos[kNRows];
#pragma unroll
            for (int r = 0; r < kNRows; ++r)
                pos[r] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)fs.run_pos[li][r]);
            const int t0 = g * kTilesPerUnit;
            const int t_end = t0 + kTilesPerUnit < tiles ? t0 + kTilesPerUnit : tiles;
            chunk_tiles_any<G, M, VEC>(pos, nrows, row, -1, grad, grad_stride, main_grad, mg_stride,
                                       nullptr, 0, hidden, t0, t_end, full_tiles);
        }
        // after the last round every wave goes on by itself
        if (last_round) break;
        __syncthreads();
        if (tid < n_round) fs.cnt[fs.run_slot[tid]] &= 0xffffu;
        __syncthreads();
    }
}


// ---- phase 1: the sorting workgroup -------------------------------------------

constexpr int kQuickCheckKeys = kMaxTokens / 4;   // kept positions the quick check takes

// True if some id occurs on more than kNRows of the kept keys (at most
// kQuickCheckKeys, left-out and missing positions hold all ones): a count
// table of the kept ids with linear probing over kMaxTokens / 2 (id + 1,
// count) pairs in the sort's second key buffer, at most half full. Every
// thread must call it; it returns the same value in every thread.
__device__ __forceinline__ bool kept_id_exceeds_rows(SortSmem &ss, int pos_bits) {
    constexpr int kSlots = kMaxTokens / 2;
    static_assert(2 * kQuickCheckKeys <= kSlots, "the table stays at most half full");
    const int tid = threadIdx.x;
    uint32_t *tab = ss.keys[1];
    for (int i = tid; i < 2 * kSlots; i += kSortThreads) tab[i] = 0u;
    if (tid == 0) ss.long_seen = 0;
    __syncthreads();
    int seen = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t key = ss.keys[0][i * kSortThreads + tid];
        if (key == 0xffffffffu) continue;
        const uint32_t k1 = (key >> pos_bits) + 1u;
        uint32_t h = (k1 * 0x9E3779B1u) >> (32 - 12);
        static_assert(kSlots == 1 << 12, "12-bit slot numbers");
        for (;;) {
            const uint32_t old = atomicCAS(&tab[2 * h], 0u, k1);
            if (old == 0u || old == k1) break;
            h = (h + 1u) & (kSlots - 1);
        }
        if (atomicAdd(&tab[2 * h + 1], 1u) >= (uint32_t)kNRows) seen = 1;
    }
    if (seen) atomicOr(&ss.long_seen, 1);
    __syncthreads();
    return ss.long_seen != 0;
}

// Sort, mark runs, write the unit and run records, zero the runs' unit counts
// and the tickets, publish the counts and raise the flag. With an id out of
// range there is nothing to do: all counts are 0.
template <typename IdT>
__device__ __forceinline__ void leader_publish(SortSmem &ss, const IdT *__restrict__ ids, int n,
                                               int num_embeddings, int64_t id_base,
                                               bool skip_outside, int pos_bits, int id_bits,
                                               int hidden, WsHeader *__restrict__ hdr,
                                               __amdgpu_buffer_rsrc_t units_rs,
                                               __amdgpu_buffer_rsrc_t runs_rs,
                                               uint32_t *__restrict__ done,
                                               uint32_t *__restrict__ shares, uint32_t epoch) {
    const int tid = threadIdx.x;
    uint32_t n_lc = 0, n_lr = 0, n_tasks = 0;
    const SortOutputs out0 = {{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr}, hdr,
                              nullptr, nullptr};
    const int bad = load_keys<IdT>(ss, ids, n, num_embeddings, pos_bits, id_base, skip_outside);
    // A vocabulary shard that keeps few positions often has no id on more than
    // 10 of them, and then no long run: the flag goes up without the sort.
    const bool few = !bad && ss.n_keys <= kQuickCheckKeys;   // uniform
    if (bad) {
        report_invalid(out0, bad);
    } else if (few && !kept_id_exceeds_rows(ss, pos_bits)) {
        if (tid == 0) {
            hdr->invalid_ids = 0;
            hdr->num_long_runs = 0;
            hdr->num_long_chunks = 0;
        }
    } else {
        const int cur = radix_sort_ids(ss, pos_bits, id_bits);
        // after the sort, aux holds: the run of every long chunk, the long-run
        // list (4 words each) and the chunk word of every long chunk
        uint32_t *lc_run = ss.aux;
        uint32_t *lr = ss.aux + 2048;
        uint32_t *lc_info = ss.aux + 8192;
        static_assert(kMaxLongChunks <= 2048 && 2048 + 4 * kMaxLongRuns <= 8192 &&
                          8192 + kMaxLongChunks <= (kSortWaves << kMaxDigitBits),
                      "long-run tables fit the sort's counter space");
        const SortOutputs out = {{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr}, hdr,
                                 lc_run, lr};
        const SortResult res = mark_runs(ss, cur, ss.n_keys, pos_bits, out);
        for (int c = tid; c < res.n_chunks; c += kSortThreads) {
            const uint32_t x = res.chunk_info[c];
            if (x & kInfoLong) lc_info[info_long_chunk(x)] = x;
        }
        __syncthreads();
        n_lc = (uint32_t)res.n_long_chunks;
        n_lr = (uint32_t)res.n_long;

        // unit records: positions of the chunk's rows (16 bits each), rows | run << 16,
        // chunk number, epoch
        const uint32_t pos_mask = (1u << pos_bits) - 1u;
        for (int c = tid; c < (int)n_lc; c += kSortThreads) {
            const uint32_t x = lc_info[c];
            const int f = info_first(x), rows = info_rows(x);
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const uint32_t a = 2 * i < rows ? res.keys[f + 2 * i] & pos_mask : 0u;
                const uint32_t b = 2 * i + 1 < rows ? res.keys[f + 2 * i + 1] & pos_mask : 0u;
                w[i] = a | (b << 16);
            }
            w[5] = (uint32_t)rows | (lc_run[c] << 16);
            w[6] = (uint32_t)c;
            w[7] = epoch;
            store_coherent16(units_rs, (uint32_t)c * kUnitRecordBytes, u32x4{w[0], w[1], w[2], w[3]});
            store_coherent16(units_rs, (uint32_t)c * kUnitRecordBytes + 16, u32x4{w[4], w[5], w[6], w[7]});
        }
        // run records, with the exclusive prefix of their combine tasks; unit counts to 0
        uint32_t tasks = 0, chunks = 0;
        if (tid < (int)n_lr) {
            chunks = lr[4 * tid + 2];
            const uint32_t wdt = (uint32_t)combine_width((int)chunks, hidden);
            tasks = ((uint32_t)hidden + wdt - 1) / wdt;
        }
        uint64_t total;
        const uint32_t first_task = (uint32_t)block_exclusive_scan(tasks, ss.scan, &total);
        if (tid < (int)n_lr)
            store_coherent16(runs_rs, (uint32_t)tid * kRunRecordBytes,
                             u32x4{lr[4 * tid], lr[4 * tid + 1], chunks, first_task});
        for (int i = tid; i < (int)n_lr * kDoneGroups; i += kSortThreads)
            store_coherent(&done[(size_t)i * kDoneStride], 0u);
        n_tasks = (uint32_t)total;

    }
    // every share of long units unclaimed (they are claimed only after the flag)
    for (int i = tid; i < (int)gridDim.x; i += kSortThreads) store_coherent(&shares[(size_t)i * kDoneStride], 0u);
    if (tid == 0) {
        store_coherent(&hdr->pub_long_chunks, n_lc);
        store_coherent(&hdr->pub_long_runs, n_lr);
        store_coherent(&hdr->pub_tasks, n_tasks);
        store_coherent(reinterpret_cast<uint32_t *>(&hdr->stolen_shares), 0u);
        store_coherent(&hdr->task_ticket, 0u);
    }
    // every store of every wave has completed, then the flag goes up
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) store_coherent(&hdr->ready, epoch);
}

// ---- phase 3: chunks of long runs ---------------------------------------------

// Wave-level wait for this call's flag; false if the wait gave up. The flag
// and the published counts (combine tasks, long chunks, long runs) are read by
// one 16-byte load: the counts had completed before the flag was stored, so
// the load that sees the flag returns them too.
__device__ __forceinline__ bool wave_wait_ready(WsHeader *__restrict__ hdr, uint32_t epoch,
                                                uint32_t *n_tasks, uint32_t *n_lc, uint32_t *n_lr) {
    static_assert(offsetof(WsHeader, ready) % 16 == 0 &&
                      offsetof(WsHeader, pub_tasks) == offsetof(WsHeader, ready) + 4 &&
                      offsetof(WsHeader, pub_long_chunks) == offsetof(WsHeader, ready) + 8 &&
                      offsetof(WsHeader, pub_long_runs) == offsetof(WsHeader, ready) + 12,
                  "flag and counts in one 16-byte word");
    const __amdgpu_buffer_rsrc_t h = buffer_range(hdr, (uint32_t)sizeof(WsHeader));
    int64_t spins = 0;
    for (;;) {
        const u32x4 v = load_coherent16(h, (uint32_t)offsetof(WsHeader, ready));
        if ((uint32_t)__builtin_amdgcn_readfirstlane(v.x) == epoch) {
            *n_tasks = __builtin_amdgcn_readfirstlane(v.y);
            *n_lc = __builtin_amdgcn_readfirstlane(v.z);
            *n_lr = __builtin_amdgcn_readfirstlane(v.w);
            return true;
        }
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kWaitLimit) {
            if ((threadIdx.x & 63) == 0) fetch_add_coherent(reinterpret_cast<uint32_t *>(&hdr->wait_timeouts), 1u);
            return false;
        }
    }
}

// First long unit of share w of the launch's gridDim.x shares of `total`.
__device__ __forceinline__ uint32_t share_begin(uint32_t total, uint32_t w) {
    return (uint32_t)((uint64_t)total * w / gridDim.x);
}

// The share that holds unit u (< total).
__device__ __forceinline__ uint32_t share_of(uint32_t total, uint32_t u) {
    uint32_t w = (uint32_t)(((uint64_t)u * gridDim.x) / total);
    while (w + 1 < gridDim.x && share_begin(total, w + 1) <= u) ++w;
    while (w > 0 && share_begin(total, w) > u) --w;
    return w;
}

// Share w's slot (128 bytes apart, zeroed by workgroup 0 before the flag) goes
// from 0 to `mark` once: 1 when its own workgroup takes it, 2 when a waiting
// combine task does. True if this call made that change.
__device__ __forceinline__ bool claim_share(uint32_t *__restrict__ shares, uint32_t w, uint32_t mark) {
    uint32_t expected = 0u;
    return __hip_atomic_compare_exchange_strong(&shares[(size_t)w * kDoneStride], &expected, mark,
                                                __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}

// Words of the long-unit hand-off, outside the LDS union: kLongElect holds
// the number of the last long_units call whose staging wave was elected;
// kLongState = call number << 2 | kStateNoFlag | kStateNoShare, published by
// the staging wave; kLongChunks / kLongRuns / kLongTasks the published counts.
constexpr int kLongElect = 0, kLongState = 1, kLongChunks = 2, kLongRuns = 3, kLongTasks = 4;
constexpr int kLongWords = 5;
constexpr uint32_t kStateNoFlag = 1u, kStateNoShare = 2u;

// Long units (chunk c, column tile k) = c * tiles + k. Workgroup w of W
// takes units [w * U / W, (w + 1) * U / W) of the U = chunks * tiles units:
// the shares are fixed by the published chunk count alone, so no device-wide
// counter is touched while the units run (a device-scope atomic in a wave
// also holds back that wave's next loads until it returns).
//
// The waves enter one by one (after their short runs, on the first call) and
// the first to enter stages the share for all: on the first call it waits for
// the flag and loads the published counts; it claims the share's slot (mark 1
// for the workgroup's own share, 2 for a take-over, 0 to leave the share
// alone), copies the records of the share's chunks to LDS while the claim is
// in flight, and publishes the outcome in `s_long`. The other waves wait for
// that on LDS, not at a barrier, so a wave that is done with its short runs
// starts long units while its siblings still finish theirs. The waves then
// claim units one at a time with an LDS counter; each unit's fp32 chunk sums
// go to its partial row with device-coherent stores. The finished units are
// counted per run in LDS and added to the run's counter of this workgroup's
// group once, after all stores of the workgroup have completed. `call` is the
// number of this call in the workgroup (1, 2, ...; the same in every wave).
template <typename G, typename M, int VEC>
__device__ __forceinline__ bool long_units(LongSmem &ls, uint32_t *s_long, uint32_t call,
                                           bool first_call, uint32_t share, uint32_t mark,
                                           uint32_t *__restrict__ shares, WsHeader *__restrict__ hdr,
                                           __amdgpu_buffer_rsrc_t units_rs,
                                           uint32_t *__restrict__ done, uint32_t n_lc_in,
                                           uint32_t n_lr_in, uint32_t n_lc_max, uint32_t n_lr_max,
                                           int n, const typename G::T *__restrict__ grad,
                                           int64_t grad_stride, float *__restrict__ partial,
                                           int64_t partial_stride, int hidden, int tiles,
                                           uint32_t epoch) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int full_tiles = hidden / (64 * VEC);
    // every branch below is on a wave-uniform value; the single-lane LDS
    // updates are whole-wave atomics in which only lane 0 changes anything
    const uint32_t one = lane == 0 ? 1u : 0u;
    const uint32_t prev = call - 1u;
    const bool stager = (uint32_t)__builtin_amdgcn_readfirstlane(
                            atomicCAS(&s_long[kLongElect], prev, lane == 0 ? call : prev)) == prev;
    if (stager) {
        bool ok = true;
        uint32_t lc = n_lc_in, lr = n_lr_in, nt = 0u;
        if (first_call) {
            ok = wave_wait_ready(hdr, epoch, &nt, &lc, &lr);
            lc = min(lc, n_lc_max);
            lr = min(lr, n_lr_max);
            if (lane == 0) s_long[kLongTasks] = nt;
        }
        lc = __builtin_amdgcn_readfirstlane(lc);
        lr = __builtin_amdgcn_readfirstlane(lr);
        bool won = false;
        if (ok && mark != 0u) {
            const uint32_t total = lc * (uint32_t)tiles;
            const uint32_t lo = share_begin(total, share), hi = share_begin(total, share + 1);
            const uint32_t c_lo = lo / (uint32_t)tiles;
            const uint32_t c_hi = hi > lo ? (hi - 1) / (uint32_t)tiles + 1 : c_lo;
            // the claim is in flight together with the loads of the records
            uint32_t w = 0u;
            if (lane == 0) w = claim_share(shares, share, mark) ? 1u : 0u;
            for (uint32_t i = (uint32_t)lane; i < 2 * (c_hi - c_lo); i += 64)
                ls.rec[i] = load_coherent16(units_rs, (2 * c_lo + i) * 16u);
            for (uint32_t r = (uint32_t)lane; r < lr; r += 64) ls.run_cnt[r] = 0u;
            if (lane == 0) ls.claim = 0u;
            won = __builtin_amdgcn_readfirstlane(w) != 0u;
        }
        if (lane == 0) {
            s_long[kLongChunks] = lc;
            s_long[kLongRuns] = lr;
        }
        const uint32_t state = call << 2 | (ok ? 0u : kStateNoFlag) | (won ? 0u : kStateNoShare);
        // the records, counters and counts above are visible before the state
        __hip_atomic_store(&s_long[kLongState], state, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    uint32_t state;
    int64_t spins = 0;
    for (;;) {
        state = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&s_long[kLongState], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if ((state >> 2) == call) break;
        // the staging wave waits at most kWaitLimit polls of the flag and a few loads
        if (++spins > 16 * kWaitLimit) {
            if (lane == 0) fetch_add_coherent(reinterpret_cast<uint32_t *>(&hdr->wait_timeouts), 1u);
            state = call << 2 | kStateNoFlag;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    if (state & (kStateNoFlag | kStateNoShare)) return false;   // uniform over the workgroup

    const uint32_t n_lc = s_long[kLongChunks], n_lr = s_long[kLongRuns];
    const uint32_t total = n_lc * (uint32_t)tiles;
    const uint32_t lo = share_begin(total, share);
    const uint32_t hi = share_begin(total, share + 1);
    const uint32_t c_lo = lo / (uint32_t)tiles;
    for (;;) {
        const uint32_t u = lo + __builtin_amdgcn_readfirstlane(atomicAdd(&ls.claim, one));
        if (u >= hi) break;
        const uint32_t c = u / (uint32_t)tiles;
        const int tile = (int)(u - c * (uint32_t)tiles);
        const u32x4 ra = ls.rec[2 * (c - c_lo)], rb = ls.rec[2 * (c - c_lo) + 1];
        uint32_t w[6] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y};
#pragma unroll
        for (int q = 0; q < 6; ++q) w[q] = __builtin_amdgcn_readfirstlane(w[q]);
        int rows = (int)(w[5] & 0xffffu);
        rows = rows < 1 ? 1 : (rows > kNRows ? kNRows : rows);
        int32_t pos[kNRows];
#pragma unroll
        for (int r = 0; r < kNRows; ++r) {
            const uint32_t q = (w[r >> 1] >> (16 * (r & 1))) & 0xffffu;
            pos[r] = q < (uint32_t)n ? (int32_t)q : 0;   // every row inside grad
        }
        const uint32_t run = w[5] >> 16;
        // a record of another call (never expected) is counted and its unit skipped
        if ((uint32_t)__builtin_amdgcn_readfirstlane(rb.w) == epoch && run < n_lr) {
            chunk_tiles_any<G, M, VEC>(pos, rows, 0, (int)c, grad, grad_stride, nullptr, 0,
                                       partial, partial_stride, hidden, tile, tile + 1,
                                       full_tiles);
            atomicAdd(&ls.run_cnt[run], one);
        } else {
            fetch_add_coherent(reinterpret_cast<uint32_t *>(&hdr->wait_timeouts), one);
        }
    }
    // the chunk sums of every wave have completed before they are counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const size_t grp = blockIdx.x % kDoneGroups;
    for (uint32_t r = (uint32_t)tid; r < n_lr; r += kSortThreads) {
        const uint32_t m = ls.run_cnt[r];
        if (m) fetch_add_coherent(&done[((size_t)r * kDoneGroups + grp) * kDoneStride], m);
    }
    return true;
}

// ---- phase 4: ordered combine of long runs -------------------------------------

// Where a workgroup stands in its combine tasks between two calls of
// combine_tasks (the values are the same in every thread).
struct CombineCursor {
    uint32_t task;        // the task being waited for, if have_task
    bool have_task;
    int64_t spins;        // polls spent on that task's wait
    uint32_t n_lc, n_lr, n_tasks;   // the published counts, as the flag's load returned them
    bool runs_loaded;     // the run records are in LDS (nothing else writes that part later)
};

// Returns false once no combine task is left. Returns true, with the task
// kept in the cursor, when the current task's run still needs the shares
// [*w_lo, *w_hi) that no workgroup has taken: the caller takes and processes
// them (long_units, which reuses this LDS) and calls again to resume the task.
template <typename G, typename M, int VEC>
__device__ __forceinline__ bool combine_tasks(AccSmem &sm, uint32_t *s_word, CombineCursor &cur,
                                              uint32_t *w_lo, uint32_t *w_hi,
                                              WsHeader *__restrict__ hdr,
                                              __amdgpu_buffer_rsrc_t runs_rs,
                                              uint32_t *__restrict__ done, bool flag_seen,
                                              float *__restrict__ partial,
                                              int64_t partial_stride,
                                              typename M::T *__restrict__ main_grad,
                                              int64_t mg_stride, int hidden, int tiles,
                                              int num_embeddings, uint32_t n_lc_max,
                                              uint32_t n_lr_max) {
    CombineSmem &cs = sm.comb;
    const int tid = threadIdx.x;
    // The counts are those the flag's load returned (without the flag, which
    // never fails to come, there is no task to take). The run records are
    // loaded once, before the first ticket (taking the ticket first and the
    // records only with a task cost 2 us on small calls, no time on large).
    if (!flag_seen) return false;
    const int n_lr = (int)min(cur.n_lr, n_lr_max);
    const uint32_t n_tasks = cur.n_tasks;
    if (n_lr == 0 || n_tasks == 0) return false;   // uniform
    const uint32_t n_lc = min(cur.n_lc, n_lc_max);
    const uint32_t total = n_lc * (uint32_t)tiles;
    if (!cur.runs_loaded) {   // uniform
        for (int r = tid; r < n_lr; r += kSortThreads)
            cs.runs[r] = load_coherent16(runs_rs, (uint32_t)r * kRunRecordBytes);
        __syncthreads();
        cur.runs_loaded = true;
    }

    for (;;) {
        if (!cur.have_task) {   // uniform
            if (tid == 0) {
                // a cheap look first: most late workgroups find the tasks gone
                // without a serialised atomic
                uint32_t t = load_coherent(&hdr->task_ticket);
                if (t < n_tasks) t = fetch_add_coherent(&hdr->task_ticket, 1u);
                s_word[2] = t;
            }
            __syncthreads();
            cur.task = s_word[2];
            cur.have_task = true;
            cur.spins = 0;
        }
        const uint32_t t = cur.task;
        if (t >= n_tasks) return false;   // uniform
        // the run: the last one whose first task is at or before t
        int lo = 0, hi = n_lr;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cs.runs[mid].w <= t) lo = mid; else hi = mid;
        }
        const u32x4 rec = cs.runs[lo];
        const uint32_t row = rec.x, first = rec.y, chunks = rec.z;
        const int wdt = combine_width((int)chunks, hidden);
        const int64_t col0 = (int64_t)(t - rec.w) * wdt;
        // a record that does not describe this call's work is skipped
        const bool valid = rec.w <= t && row < (uint32_t)num_embeddings && chunks >= 1 &&
                           first < n_lc_max && chunks <= n_lc_max - first && col0 < hidden;
        // Wait until the run's units are all counted. If that takes long, some
        // workgroups of the launch are not running (more were launched than fit,
        // or other work holds compute units): then the caller processes the
        // run's shares that nobody has taken yet, and the wait resumes.
        // Stealing needs the run's units inside this call's unit list.
        const bool can_steal = flag_seen && valid && first + chunks <= n_lc;
        if (tid == 0) {
            uint32_t status = valid ? 0u : 3u;   // 0 waiting, 1 done, 2 steal, 3 give up
            const uint32_t target = chunks * (uint32_t)tiles;
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            int64_t spins = cur.spins;
            while (status == 0u) {
                uint32_t sum = 0;
                for (int g = 0; g < kDoneGroups; ++g)
                    sum += load_coherent(&done[((size_t)lo * kDoneGroups + g) * kDoneStride]);
                if (sum >= target) {
                    status = 1u;
                } else if (++spins > kWaitLimit) {
                    fetch_add_coherent(reinterpret_cast<uint32_t *>(&hdr->wait_timeouts), 1u);
                    status = 3u;
                } else if (can_steal && __builtin_amdgcn_s_memrealtime() - t0 > kStealAfterTicks) {
                    status = 2u;
                } else {
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            s_word[3] = status;
            s_word[0] = (uint32_t)(spins < kWaitLimit ? spins : kWaitLimit);   // free since the run list loaded
        }
        __syncthreads();
        const uint32_t status = s_word[3];
        cur.spins = (int64_t)s_word[0];
        if (status == 2u) {   // uniform
            // the run's units are [first * tiles, (first + chunks) * tiles)
            *w_lo = share_of(total, first * (uint32_t)tiles);
            *w_hi = share_of(total, (first + chunks) * (uint32_t)tiles - 1u) + 1u;   // <= gridDim.x
            __syncthreads();   // every thread has read s_word before the caller reuses it
            return true;
        }
        const bool task_ok = status == 1u;
        cur.have_task = false;
        __syncthreads();
        if (task_ok) {   // uniform
            combine_block<G, M>(cs.stage, row, first, chunks, col0, wdt, partial, partial_stride,
                                main_grad, mg_stride, hidden);
        }
        __syncthreads();
    }
}

template <typename IdT, typename G, typename M, int VEC>
__global__ __launch_bounds__(kSortThreads) void accumulate_kernel(
    const IdT *__restrict__ ids, int n, int num_embeddings, int64_t id_base, int skip_outside,
    int pos_bits, int id_bits,
    const typename G::T *__restrict__ grad, int64_t grad_stride,
    typename M::T *__restrict__ main_grad, int64_t mg_stride, int hidden, int tiles,
    WsHeader *__restrict__ hdr, uint8_t *__restrict__ units,
    uint8_t *__restrict__ runs, uint32_t *__restrict__ done, uint32_t *__restrict__ shares,
    float *__restrict__ partial, int64_t partial_stride, uint32_t epoch, int defer_odd_shares) {
    __shared__ AccSmem sm;
    __shared__ uint32_t s_word[4];   // LDS broadcasts between phases
    __shared__ uint32_t s_long[kLongWords];   // long-share hand-off (kLongElect ...)
    const int tid = threadIdx.x;
    const uint32_t n_lc_max = (uint32_t)(2 * n / 11), n_lr_max = (uint32_t)(n / 11);
    const __amdgpu_buffer_rsrc_t units_rs = buffer_range(units, n_lc_max * (uint32_t)kUnitRecordBytes);
    const __amdgpu_buffer_rsrc_t runs_rs = buffer_range(runs, n_lr_max * (uint32_t)kRunRecordBytes);
    if (tid == 0) {   // read after the barriers of either first phase
        s_long[kLongElect] = 0u;
        s_long[kLongState] = 0u;
        s_long[kLongTasks] = 0u;
    }

    if (blockIdx.x == 0) {
        leader_publish<IdT>(sm.sort, ids, n, num_embeddings, id_base, skip_outside != 0, pos_bits,
                            id_bits, hidden, hdr,
                            units_rs, runs_rs, done, shares, epoch);
    } else {
        // the waves leave this one by one, as their short-run units run out
        follower_short_runs<IdT, G, M, VEC>(sm.fol, ids, n, num_embeddings, id_base,
                                            skip_outside != 0, pos_bits, grad, grad_stride,
                                            main_grad, mg_stride, hidden, tiles,
                                            (int)blockIdx.x - 1, (int)gridDim.x - 1);
    }
    // Phases 3 and 4: the workgroup's own share (claimed with mark 1, unless a
    // waiting combine task took it already; a test setting leaves every other
    // share to the combine tasks: mark 0), then combine tasks. A combine task
    // that waits long hands back the shares [w, w_end) its run still needs,
    // taken over here with mark 2 (one copy of the long-unit code serves both).
    uint32_t w = blockIdx.x, w_end = blockIdx.x + 1u;
    uint32_t mark = defer_odd_shares && (blockIdx.x & 1u) ? 0u : 1u;
    uint32_t call = 0u;
    bool flag_seen = false;
    CombineCursor cur;
    cur.have_task = false;
    cur.task = 0u;
    cur.spins = 0;
    cur.n_lc = cur.n_lr = cur.n_tasks = 0u;
    cur.runs_loaded = false;
    for (;;) {
        for (; w < w_end; ++w) {
            ++call;
            const bool took = long_units<G, M, VEC>(sm.lng, s_long, call, call == 1u, w, mark,
                                                    shares, hdr, units_rs, done, cur.n_lc,
                                                    cur.n_lr, n_lc_max, n_lr_max, n, grad,
                                                    grad_stride, partial, partial_stride, hidden,
                                                    tiles, epoch);
            if (call == 1u) {   // the flag and the counts, as the staging wave saw them
                flag_seen = (s_long[kLongState] & kStateNoFlag) == 0u;
                cur.n_lc = s_long[kLongChunks];
                cur.n_lr = s_long[kLongRuns];
                cur.n_tasks = s_long[kLongTasks];
            }
            if (took && mark == 2u && tid == 0)
                fetch_add_coherent(reinterpret_cast<uint32_t *>(&hdr->stolen_shares), 1u);
            __syncthreads();
        }
        if (!combine_tasks<G, M, VEC>(sm, s_word, cur, &w, &w_end, hdr, runs_rs, done, flag_seen,
                                      partial, partial_stride, main_grad, mg_stride, hidden,
                                      tiles, num_embeddings, n_lc_max, n_lr_max))
            break;
        mark = 2u;
    }

    // ---- phase 5: the last workgroup out resets the call's shared state ----
    // two levels of counters, so that no address takes more than ~32 atomics
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t grp = blockIdx.x % kExitGroups;
        const uint32_t members = (gridDim.x - grp + kExitGroups - 1) / kExitGroups;
        uint32_t last = 0;
        if (fetch_add_coherent(&hdr->exit_group[grp][0], 1u) == members - 1) {
            const uint32_t used = gridDim.x < kExitGroups ? gridDim.x : kExitGroups;
            last = fetch_add_coherent(&hdr->exit_top, 1u) == used - 1 ? 1u : 0u;
        }
        if (last) {
            for (int g = 0; g < kExitGroups; ++g) store_coherent(&hdr->exit_group[g][0], 0u);
            store_coherent(&hdr->exit_top, 0u);
            store_coherent(&hdr->task_ticket, 0u);
            store_coherent(&hdr->ready, 0u);
        }
    }
}

template <typename IdT, typename G, typename M, int VEC>
hipError_t launch(const void *ids, int n, int num_embeddings, int64_t id_base, int skip_outside,
                  int pos_bits, int id_bits,
                  const void *grad, int64_t grad_stride, void *main_grad, int64_t mg_stride,
                  int hidden, void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                  int defer_odd_shares, hipEvent_t kstart, hipEvent_t kstop, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    const int tiles = (hidden + 64 * VEC - 1) / (64 * VEC);
    const int grid = num_cus < 2 ? 2 : (num_cus > kMaxGrid ? kMaxGrid : num_cus);
    auto kernel = accumulate_kernel<IdT, G, M, VEC>;
    const IdT *ids_t = static_cast<const IdT *>(ids);
    const typename G::T *grad_t = static_cast<const typename G::T *>(grad);
    typename M::T *mg_t = static_cast<typename M::T *>(main_grad);
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws);
    uint8_t *units = reinterpret_cast<uint8_t *>(ws + l.units);
    uint8_t *runs = reinterpret_cast<uint8_t *>(ws + l.runs);
    uint32_t *done = reinterpret_cast<uint32_t *>(ws + l.done);
    uint32_t *shares = reinterpret_cast<uint32_t *>(ws + l.shares);
    float *partial = reinterpret_cast<float *>(ws + l.partial);
    if (kstart && kstop)   // events taken by the dispatch itself: the kernel's own duration
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kSortThreads), 0, stream, kstart, kstop, 0,
                              ids_t, n, num_embeddings, id_base, skip_outside, pos_bits, id_bits,
                              grad_t, grad_stride, mg_t, mg_stride, hidden, tiles, hdr, units, runs,
                              done, shares, partial, l.partial_stride, epoch, defer_odd_shares);
    else
        kernel<<<grid, kSortThreads, 0, stream>>>(ids_t, n, num_embeddings, id_base, skip_outside,
                                                  pos_bits, id_bits, grad_t, grad_stride, mg_t,
                                                  mg_stride, hidden, tiles, hdr, units, runs, done,
                                                  shares, partial, l.partial_stride, epoch,
                                                  defer_odd_shares);
    return hipGetLastError();
}

template <typename IdT>
hipError_t dispatch_types(bool grad_bf16, bool mg_bf16, bool vec, const void *ids, int n,
                          int num_embeddings, int64_t id_base, int skip_outside, int pos_bits,
                          int id_bits, const void *grad,
                          int64_t grad_stride, void *main_grad, int64_t mg_stride, int hidden,
                          void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                          int defer_odd_shares, hipEvent_t kstart, hipEvent_t kstop,
                          hipStream_t stream) {
#define EWG_ACC(G, M, V)                                                                        \
    launch<IdT, G, M, V>(ids, n, num_embeddings, id_base, skip_outside, pos_bits, id_bits, grad,   \
                         grad_stride, main_grad, mg_stride, hidden, workspace, l, num_cus, epoch, \
                         defer_odd_shares, kstart, kstop, stream)
    if (grad_bf16) {
        if (mg_bf16) return vec ? EWG_ACC(BF16, BF16, 8) : EWG_ACC(BF16, BF16, 1);
        return vec ? EWG_ACC(BF16, F32, 8) : EWG_ACC(BF16, F32, 1);
    }
    if (mg_bf16) return vec ? EWG_ACC(F32, BF16, 4) : EWG_ACC(F32, BF16, 1);
    return vec ? EWG_ACC(F32, F32, 4) : EWG_ACC(F32, F32, 1);
#undef EWG_ACC
}

}  // namespace

hipError_t launch_accumulate(bool ids_int64, bool grad_bf16, bool mg_bf16, bool vec,
                             const void *ids, int n, int num_embeddings, int64_t id_base,
                             bool skip_outside, int pos_bits, int id_bits,
                             const void *grad, int64_t grad_stride, void *main_grad,
                             int64_t mg_stride, int hidden, void *workspace, const WsLayout &l,
                             int num_cus, uint32_t epoch, int defer_odd_shares,
                             hipEvent_t kstart, hipEvent_t kstop, hipStream_t stream) {
    if (ids_int64)
        return dispatch_types<int64_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, id_base,
                                       skip_outside ? 1 : 0, pos_bits, id_bits, grad, grad_stride,
                                       main_grad, mg_stride, hidden, workspace, l, num_cus, epoch,
                                       defer_odd_shares, kstart, kstop, stream);
    return dispatch_types<int32_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, id_base,
                                   skip_outside ? 1 : 0, pos_bits, id_bits, grad, grad_stride,
                                   main_grad, mg_stride, hidden, workspace, l, num_cus, epoch,
                                   defer_odd_shares, kstart, kstop, stream);
}

}  // namespace ewg
