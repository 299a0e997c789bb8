// The whole accumulation in one kernel: sort, chunk sums, runs of at most 10
// rows finished in place, and long runs finished by column blocks. One
// 1024-thread workgroup per compute unit (at least two workgroups).
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad": the
// introduction's two bullets (equal ids ordered by ascending position; fp32
// chunk sums of ten consecutive rows or fewer; those sums folded left to
// right from +0 with a single conversion to grad's dtype at the end; then an
// fp32 add onto the main_grad row, converted back to main_grad's dtype),
// _sort_tokens_kernel,
// _partial_sums_kernel (a run of at most NROWS rows is finished there) and
// _long_run_sums_kernel (the partial sums of a longer run added in order).
//
// Phases of one launch:
//   1. Workgroup 0 (dispatched first, it never waits for anyone) radix-sorts
//      the packed keys in LDS (sort_lds.h) and writes, with device-coherent
//      stores, one record per chunk of a run longer than 10 rows (its row
//      positions and run) and one per such run (main_grad row, first chunk,
//      chunk count, width of its column blocks, first block). Once every
//      store has completed it sets the ready flag to the call's epoch (a
//      nonzero number per call); the number of blocks comes with the flag.
//   2. Meanwhile every other workgroup builds an LDS hash table of the ids
//      and finishes its equal-cost share of the runs of at most 10 rows (a run
//      of at most 10 rows is one chunk: it needs its rows in position order,
//      not a global sort).
//   3. Then every workgroup takes column blocks of long runs from a device-
//      wide ticket until none is left. A block is one long run over a range of
//      columns. Each workgroup first stages the positions of every long chunk
//      in LDS (once per call); for a block its waves sum every chunk of the
//      block (fp32, from +0, rows in position order) into LDS; then each
//      column adds its chunk sums in chunk order from +0, rounds once and is
//      added to main_grad. The chunk sums never leave the compute unit, and no
//      workgroup waits for another except for the flag. A run's blocks are as
//      wide as its chunk sums fit in LDS and its grad bytes fit about one
//      round of loads of the workgroup (one 10-row item in flight per wave),
//      so a deep run is spread over many workgroups and a shallow one covers
//      up to 2048 columns.
//   4. The last workgroup to finish clears the ticket, the exit counters and
//      the flag for the next call (they live in the workspace header).
// The flag is raised by workgroup 0, which waits for nothing before it, so the
// one wait of the kernel ends whatever number of workgroups runs at once. It
// is bounded all the same; a wait that gives up is counted in the workspace
// header and its work skipped.
//
// A column tile of the short runs is 64 lanes x VEC columns (8 for bf16 grad,
// 4 for fp32), laid out in lane-contiguous pieces (piece_cols in ewg_device.h).
#include <hip/hip_ext.h>

#include "chunk_sums.h"
#include "ewg_device.h"
#include "ewg_internal.h"
#include "sort_lds.h"

namespace ewg {
namespace {

constexpr int64_t kWaitLimit = 1 << 22;  // polls before a wait gives up (seconds)
constexpr int kHashSlots = 16384;        // > 2 x kMaxTokens: linear probing always ends
constexpr int kHashBits = 14;
constexpr int kOwnedMax = 256;           // short runs gathered per round by one follower
constexpr uint32_t kNoSlot = 0xffffu;    // slot of a position whose id is left out
constexpr int kMaxLongRuns = kMaxTokens / 11;
constexpr int kMaxLongChunks = 2 * kMaxTokens / 11;
constexpr int kMaxRunChunks = (kMaxTokens + kNRows - 1) / kNRows;   // chunks of the longest run
constexpr int kBlockStageFloats = 26624; // chunk sums of one column block (104 KiB of LDS)
constexpr int kMinBlockLog = 4;          // narrowest column block: 16 columns (64 bytes of fp32)
constexpr int kMaxBlockLog = 11;         // widest column block: 2048 columns
constexpr int kFoldCols = (1 << kMaxBlockLog) / kSortThreads;   // fold columns per thread
// grad bytes of a column block: one item of 10 rows x 64 lanes x 16 bytes for
// each of the 16 waves, so that a block is one round of loads
constexpr uint64_t kBlockBytes = (uint64_t)kSortWaves * kNRows * 64 * 16;
static_assert((kMaxRunChunks << kMinBlockLog) <= kBlockStageFloats,
              "the narrowest block of the longest run fits the stage");

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

struct BlockSmem {
    float stage[kBlockStageFloats];          // chunk sums of one block, [chunk][column]
    u32x4 runs[kMaxLongRuns + 1];            // run records
    alignas(4) uint16_t pos[kMaxLongChunks * kNRows];   // positions of every long chunk, kNRows each
    uint8_t rows[kMaxLongChunks];            // rows of every long chunk
    alignas(16) float trash[8];              // the stores of lanes without a piece
};

union AccSmem {
    SortSmem sort;
    FollowerSmem fol;
    BlockSmem blk;
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
                                                    int me, int followers, int32_t *fails) {
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
        // (the slot, key and count words of the thread's positions are all
        // read before the first is used)
        const int p0 = tid * kSortItems;
        static_assert(kSortItems == 8, "eight 16-bit slots per thread");
        const u32x4 sw = reinterpret_cast<const u32x4 *>(fs.slot_of_pos)[tid];
        const uint32_t sw4[4] = {sw.x, sw.y, sw.z, sw.w};
        uint32_t hs[kSortItems], kw[kSortItems], cw[kSortItems];
#pragma unroll
        for (int j = 0; j < kSortItems; ++j)
            hs[j] = p0 + j < n ? (sw4[j >> 1] >> (16 * (j & 1))) & 0xffffu : kNoSlot;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t a = hs[j] & (uint32_t)(kHashSlots - 1);   // in the table for kNoSlot too
            kw[j] = fs.key[a];
            cw[j] = fs.cnt[a];
        }
        uint32_t v[kSortItems];
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t c = cw[j] & 0xffffu;
            const bool first_pos = hs[j] != kNoSlot && (kw[j] >> id_shift) == (uint32_t)(p0 + j);
            v[j] = first_pos && c <= (uint32_t)kNRows ? (c * row_cost + end_cost) | (1u << kCostBits) : 0u;
            sum += v[j];
        }
        uint32_t total;
        const uint32_t run = block_exclusive_scan32(sum, fs.scan32, &total);
        // cost_all < 2^kCostBits and followers < 2^12: 32-bit products
        const uint32_t cost_all = total & kCostMask;
        const uint32_t lo = cost_all * (uint32_t)me / (uint32_t)followers;
        const uint32_t hi = cost_all * (uint32_t)(me + 1) / (uint32_t)followers;
        static_assert((uint64_t)kCostMask * (kMaxGrid + 1) < (1ull << 32), "32-bit share bounds");
        // runs are numbered in position order; this follower's (cost start in
        // [lo, hi)) are a contiguous range of numbers
        {
            uint32_t x = run;
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < kSortItems; ++j) {
                const uint32_t start = x & kCostMask;
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
                const uint32_t start = x & kCostMask;
                if (v[j] && start >= lo && start < hi) {
                    const int li = (int)((x >> kCostBits) - first) - r0;
                    if (li >= 0 && li < kOwnedMax) {
                        fs.run_id[li] = (kw[j] & id_mask) - 1u;
                        fs.run_len[li] = 0u;
                        fs.run_slot[li] = hs[j];
                        fs.cnt[hs[j]] |= (uint32_t)(li + 1) << 16;
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
        {
            uint32_t m[kSortItems], k[kSortItems];
#pragma unroll
            for (int j = 0; j < kSortItems; ++j)
                m[j] = hs[j] != kNoSlot ? fs.cnt[hs[j]] >> 16 : 0u;   // run of the round + 1, or 0
#pragma unroll
            for (int j = 0; j < kSortItems; ++j)
                if (m[j]) k[j] = atomicAdd(&fs.run_len[checked_index<uint32_t>(m[j] - 1u, kOwnedMax, fails)], 1u);
#pragma unroll
            for (int j = 0; j < kSortItems; ++j)
                if (m[j])
                    fs.run_pos[checked_index<uint32_t>(m[j] - 1u, kOwnedMax, fails)]
                              [checked_index<uint32_t>(k[j], kNRows, fails)] = (uint16_t)(p0 + j);
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


// log2 of the column-block width of a long run of `chunks` chunks: the widest
// power of two up to 2048 columns (no wider than hidden needs) whose chunk
// sums fit the LDS stage and whose grad bytes (at most 10 rows per chunk) stay
// within one round of loads of the workgroup, but no narrower than 128 bytes
// of a grad row (64 bf16 or 32 fp32 columns: memory moves whole 128-byte
// lines), or 64 bytes where the chunk sums of 128 would not fit the stage. A
// deep run's block may then take several rounds of loads (block_stage).
__device__ __forceinline__ int block_log_width(uint32_t chunks, int hidden, int grad_bytes) {
    // 128 bytes of a grad row when the chunk sums fit the stage, else 64
    const int lw128 = grad_bytes >= 4 ? kMinBlockLog + 1 : kMinBlockLog + 2;
    const int min_lw = ((uint64_t)chunks << lw128) <= (uint64_t)kBlockStageFloats ? lw128 : lw128 - 1;
    int lw = min_lw;
    while (lw < kMaxBlockLog && (1 << lw) < hidden) ++lw;
    const uint64_t row_bytes = (uint64_t)chunks * kNRows * (uint64_t)grad_bytes;
    while (lw > min_lw &&
           (((uint64_t)chunks << lw) > (uint64_t)kBlockStageFloats || (row_bytes << lw) > kBlockBytes))
        --lw;
    return lw;
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

// The runs of the sorted keys that the long phase needs, for the sorting
// workgroup (the inspection entry point marks every run with mark_runs in
// sort_lds.h). Blocked arrangement: thread t owns sorted slots [8t, 8t + 8).
// Out, in LDS: per long chunk c its first slot and rows (lc_info[c] = slot |
// (rows - 1) << 13) and its long run (lc_run[c]); per long run r {main_grad
// row, first long chunk, chunk count, 0} (lr[4r .. 4r + 3]). Every LDS read
// of a step is issued before the first use, and the two scans are wave-level
// DPP scans. Line 0 of the header gets the counts (invalid_ids = 0).
struct LongRuns {
    int n_long, n_long_chunks;
};

__device__ __forceinline__ LongRuns mark_long_runs(SortSmem &sm, int cur, int n, int pos_bits,
                                                   uint32_t *lc_info, uint32_t *lc_run,
                                                   uint32_t *lr, WsHeader *__restrict__ hdr) {
    const int tid = threadIdx.x;
    const uint32_t *sk = sm.keys[cur];
    const int s0 = tid * kSortItems;
    uint32_t k[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) k[j] = sk[s0 + j];
    uint32_t prev = s0 > 0 ? (sk[s0 - 1] >> pos_bits) : 0u;
    uint32_t start_bits = 0, nstart = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t id = k[j] >> pos_bits;
        const bool st = s0 + j < n && (s0 + j == 0 || id != prev);
        start_bits |= (uint32_t)st << j;
        nstart += st;
        prev = id;
    }
    uint32_t num_runs;
    const uint32_t run_base =
        block_exclusive_scan32(nstart, reinterpret_cast<uint32_t *>(sm.scan), &num_runs);
    // first slot of every run, plus n after the last: runs are [rs[r], rs[r+1])
    uint32_t *rs = sm.aux;
    uint32_t run_of[kSortItems];
    {
        uint32_t r = run_base;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            if ((start_bits >> j) & 1u) rs[r++] = (uint32_t)(s0 + j);
            run_of[j] = r > 0u ? r - 1u : 0u;   // in [0, num_runs): slot 0 starts a run
        }
    }
    if (tid == 0) rs[num_runs] = (uint32_t)n;
    __syncthreads();
    uint32_t f[kSortItems], e[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        f[j] = rs[run_of[j]];
        e[j] = rs[run_of[j] + 1u];
    }
    // per slot: bit 0 = first slot of a long chunk, bit 16 = first slot of a
    // long run, bit 32 = first slot of a chunk of any run
    uint64_t flag[kSortItems], nflag = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t sj = (uint32_t)(s0 + j), off = sj - f[j];
        const bool valid = s0 + j < n;
        const bool longer = valid && e[j] - f[j] > (uint32_t)kNRows;
        const bool chunk_start = valid && off % kNRows == 0u;
        flag[j] = (uint64_t)(chunk_start && longer) | ((uint64_t)(longer && off == 0u) << 16) |
                  ((uint64_t)chunk_start << 32);
        nflag += flag[j];
    }
    uint64_t totals;
    uint64_t idx = block_exclusive_scan(nflag, sm.scan, &totals);
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t sj = (uint32_t)(s0 + j);
        const uint32_t lc = (uint32_t)(idx & 0xffffu), r = (uint32_t)((idx >> 16) & 0xffffu);
        const bool run_start = (flag[j] >> 16) & 1u;
        if (flag[j] & 1u) {
            const uint32_t left = e[j] - sj;
            lc_info[lc] = sj | ((left < (uint32_t)kNRows ? left : (uint32_t)kNRows) - 1u) << 13;
            // a long chunk belongs to the long run that starts at its slot,
            // or else to the last one started before it
            lc_run[lc] = run_start ? r : r - 1u;
        }
        if (run_start) {
            lr[4 * r + 0] = k[j] >> pos_bits;
            lr[4 * r + 1] = lc;
            lr[4 * r + 2] = (e[j] - f[j] + kNRows - 1) / kNRows;
            lr[4 * r + 3] = 0u;
        }
        idx += flag[j];
    }
    LongRuns res;
    res.n_long_chunks = (int)(totals & 0xffffu);
    res.n_long = (int)((totals >> 16) & 0xffffu);
    if (tid == 0) {
        hdr->invalid_ids = 0;
        hdr->num_chunks = (int32_t)(totals >> 32);
        hdr->num_long_runs = res.n_long;
        hdr->num_long_chunks = res.n_long_chunks;
        hdr->num_runs = (int32_t)num_runs;
    }
    __syncthreads();   // the long-run tables are complete
    return res;
}

// Sort, mark runs, write the unit and run records (with the width of each
// run's column blocks), zero the block ticket, publish the counts and raise
// the flag. With an id out of
// range there is nothing to do: all counts are 0.
template <typename IdT>
__device__ __forceinline__ void leader_publish(SortSmem &ss, const IdT *__restrict__ ids, int n,
                                               int num_embeddings, int64_t id_base,
                                               bool skip_outside, int pos_bits, int id_bits,
                                               int hidden, int grad_bytes,
                                               WsHeader *__restrict__ hdr,
                                               __amdgpu_buffer_rsrc_t units_rs,
                                               __amdgpu_buffer_rsrc_t runs_rs, uint32_t epoch) {
    const int tid = threadIdx.x;
    uint32_t n_lc = 0, n_lr = 0, n_blocks = 0;
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
        const int cur = radix_sort_ids(ss, pos_bits, id_bits, n);
        // after the sort, aux holds: the run of every long chunk, the long-run
        // list (4 words each) and the chunk word of every long chunk
        uint32_t *lc_run = ss.aux;
        uint32_t *lr = ss.aux + 2048;
        uint32_t *lc_info = ss.aux + 8192;
        static_assert(kMaxLongChunks <= 2048 && 2048 + 4 * kMaxLongRuns <= 8192 &&
                          8192 + kMaxLongChunks <= (kSortWaves << kMaxDigitBits),
                      "long-run tables fit the sort's counter space");
        const LongRuns res = mark_long_runs(ss, cur, ss.n_keys, pos_bits, lc_info, lc_run, lr, hdr);
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
                const uint32_t a = 2 * i < rows ? ss.keys[cur][f + 2 * i] & pos_mask : 0u;
                const uint32_t b = 2 * i + 1 < rows ? ss.keys[cur][f + 2 * i + 1] & pos_mask : 0u;
                w[i] = a | (b << 16);
            }
            w[5] = (uint32_t)rows | (lc_run[c] << 16);
            w[6] = (uint32_t)c;
            w[7] = epoch;
            store_coherent16(units_rs, (uint32_t)c * kUnitRecordBytes, u32x4{w[0], w[1], w[2], w[3]});
            store_coherent16(units_rs, (uint32_t)c * kUnitRecordBytes + 16, u32x4{w[4], w[5], w[6], w[7]});
        }
        // run records: chunk count and block width, and the exclusive prefix of
        // the runs' column blocks (a block reads at most kBlockBytes of grad)
        uint32_t blocks = 0, code = 0;
        if (tid < (int)n_lr) {
            const uint32_t chunks = lr[4 * tid + 2];
            const int lw = block_log_width(chunks, hidden, grad_bytes);
            blocks = (uint32_t)(((int64_t)hidden + (1 << lw) - 1) >> lw);
            code = chunks | (uint32_t)lw << 16;
        }
        uint64_t total;
        const uint32_t first_block = (uint32_t)block_exclusive_scan(blocks, ss.scan, &total);
        if (tid < (int)n_lr)
            store_coherent16(runs_rs, (uint32_t)tid * kRunRecordBytes,
                             u32x4{lr[4 * tid], lr[4 * tid + 1], code, first_block});
        n_blocks = (uint32_t)total;
    }
    if (tid == 0) {
        store_coherent(&hdr->pub_long_chunks, n_lc);
        store_coherent(&hdr->pub_long_runs, n_lr);
        store_coherent(&hdr->pub_blocks, n_blocks);
        store_coherent(&hdr->block_ticket, 0u);
    }
    // every store of every wave has completed, then the flag goes up
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) store_coherent(&hdr->ready, epoch);
}

// ---- phase 3: column blocks of long runs ----------------------------------------

// and the published counts (column blocks, long chunks, long runs) are read by
// one 16-byte load: the counts had completed before the flag was stored, so
// the load that sees the flag returns them too.
__device__ __forceinline__ bool wave_wait_ready(WsHeader *__restrict__ hdr, uint32_t epoch,
                                                uint32_t *n_blocks, uint32_t *n_lc, uint32_t *n_lr) {
    static_assert(offsetof(WsHeader, ready) % 16 == 0 &&
                      offsetof(WsHeader, pub_blocks) == offsetof(WsHeader, ready) + 4 &&
                      offsetof(WsHeader, pub_long_chunks) == offsetof(WsHeader, ready) + 8 &&
                      offsetof(WsHeader, pub_long_runs) == offsetof(WsHeader, ready) + 12,
                  "flag and counts in one 16-byte word");
    const __amdgpu_buffer_rsrc_t h = buffer_range(hdr, (uint32_t)sizeof(WsHeader));
    int64_t spins = 0;
    for (;;) {
        const u32x4 v = load_coherent16(h, (uint32_t)offsetof(WsHeader, ready));
        if ((uint32_t)__builtin_amdgcn_readfirstlane(v.x) == epoch) {
            *n_blocks = __builtin_amdgcn_readfirstlane(v.y);
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

// One column block [col0, col0 + wc) of the long run whose `chunks` chunks
// start at long chunk `first` (main_grad row `row`), wc = min(2^lw, hidden -
// col0). Every thread of the workgroup holds the same description.
struct BlockDesc {
    uint32_t row, first, chunks;
    int lw, col0, wc;
    bool valid;
    int32_t *fails;   // the header's check_failures word (checked builds)
};

// The block of ticket number b: the last run whose first block is at or
// before b, and the column range b - (that first block) of it. `bad` is set
// when the record does not describe a block of this call.
__device__ __forceinline__ BlockDesc describe_block(const BlockSmem &bs, uint32_t b, uint32_t n_lr,
                                                    uint32_t n_lc, int num_embeddings, int hidden,
                                                    bool staged_ok, bool *bad, int32_t *fails) {
    int lo = 0, hi = (int)n_lr;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (bs.runs[mid].w <= b) lo = mid; else hi = mid;
    }
    const u32x4 rec = bs.runs[lo];
    BlockDesc d;
    d.fails = fails;
    d.row = rec.x;
    d.first = rec.y;
    d.chunks = rec.z & 0xffffu;
    d.lw = (int)((rec.z >> 16) & 0xffu);
    const bool shape_ok = rec.w <= b && d.lw >= kMinBlockLog && d.lw <= kMaxBlockLog &&
                          d.chunks > 1u && d.chunks <= (uint32_t)kMaxRunChunks &&
                          (d.chunks << d.lw) <= (uint32_t)kBlockStageFloats;
    const int64_t col0 = shape_ok ? (int64_t)(b - rec.w) << d.lw : (int64_t)hidden;
    d.valid = staged_ok && shape_ok && d.row < (uint32_t)num_embeddings && d.first < n_lc &&
              d.chunks <= n_lc - d.first && col0 < hidden;
    *bad = !d.valid;
    d.col0 = d.valid ? (int)col0 : 0;
    const int width = 1 << d.lw;
    d.wc = d.valid ? (hidden - d.col0 < width ? hidden - d.col0 : width) : 0;
    return d;
}

// The lanes of a block take (chunk, piece) pairs: a row of the block is
// 2^lw / VEC pieces of VEC columns and a wave covers 64 of them, so several
// chunks when the block is narrower than 64 pieces and one tile of 64 pieces
// of one chunk otherwise. Item `it` of the block is one such wave's worth.
template <int VEC>
struct ItemShape {
    int llog, tlog, per, items;
    __device__ __forceinline__ ItemShape(int lw, uint32_t chunks) {
        constexpr int kVecLog = VEC == 8 ? 3 : (VEC == 4 ? 2 : (VEC == 2 ? 1 : 0));
        static_assert((1 << kVecLog) == VEC, "VEC is 1, 2, 4 or 8");
        const int plog = lw - kVecLog;   // pieces per row, log2 (>= 2)
        llog = plog < 6 ? plog : 6;      // lanes per row, log2
        tlog = plog - llog;              // tiles of 64 pieces per row, log2
        per = 64 >> llog;                // chunks per wave item
        items = (((int)chunks + per - 1) / per) << tlog;
    }
};

// This lane's part of item `it`: its chunk k, its column lc in the block, and
// whether the piece is inside the block (active) and whole (VEC columns).
struct LanePiece {
    int k, lc, rows;
    bool active, whole;
};

template <int VEC>
__device__ __forceinline__ LanePiece lane_piece(const BlockSmem &bs, const BlockDesc &d,
                                                const ItemShape<VEC> &sh, int it, int lane) {
    LanePiece q;
    q.k = (it >> sh.tlog) * sh.per + (lane >> sh.llog);
    q.lc = (((it & ((1 << sh.tlog) - 1)) << 6) + (lane & ((1 << sh.llog) - 1))) * VEC;
    q.active = d.valid && it < sh.items && q.k < (int)d.chunks && q.lc < d.wc;
    q.whole = q.active && q.lc + VEC <= d.wc;
    const int rows = (int)bs.rows[checked_index<uint32_t>(q.active ? d.first + q.k : 0u,
                                                          kMaxLongChunks, d.fails)];   // every lane reads
    q.rows = q.active ? rows : 0;
    return q;
}

// The rows of this lane's piece (whole pieces only; see stage_piece). Every
// load is issued whatever the lane's piece: a row past the chunk's last
// re-reads its first row and a lane without a whole piece reads grad's first
// VEC elements, so that the compiler's count of loads in flight is exact and
// no load waits for an earlier one (a load under a lane condition leaves its
// register possibly pending, and the next write of that register then waits
// for every load in flight).
template <typename GT, int VEC>
__device__ __forceinline__ void load_piece_rows(const BlockSmem &bs, const BlockDesc &d,
                                                const LanePiece &q, const GT *__restrict__ grad,
                                                int64_t grad_stride, GT (&raw)[kNRows][VEC]) {
    static_assert(kNRows % 2 == 0 && (kNRows * sizeof(uint16_t)) % 4 == 0,
                  "a chunk's positions are whole 32-bit words");
    // the chunk's positions as 32-bit words, all LDS reads issued before the first use
    const uint32_t *pw = reinterpret_cast<const uint32_t *>(
        &bs.pos[checked_index<uint32_t>(q.whole ? d.first + q.k : 0u, kMaxLongChunks, d.fails) * kNRows]);
    uint32_t w[kNRows / 2];
#pragma unroll
    for (int i = 0; i < kNRows / 2; ++i) w[i] = pw[i];
    const GT *base = q.whole ? grad + d.col0 + q.lc : grad;
#pragma unroll
    for (int r = 0; r < kNRows; ++r) {
        const uint32_t pr = r < q.rows ? (w[r >> 1] >> (16 * (r & 1))) & 0xffffu : w[0] & 0xffffu;
        const int64_t p = q.whole ? (int64_t)pr : 0;
        load_vec<GT, VEC>(base + p * grad_stride, raw[r]);
    }
}

// The chunk sum of a piece from its loaded rows: fp32, from +0, rows in
// position order, into the LDS stage at [chunk][column]. Every register of
// `raw` is read and every lane stores (a lane without a whole piece into
// bs.trash), so that no load result stays pending past this point.
template <typename G, int VEC>
__device__ __forceinline__ void stage_piece(BlockSmem &bs, int lw, const LanePiece &q,
                                            const typename G::T (&raw)[kNRows][VEC],
                                            int32_t *fails) {
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < kNRows; ++r) {
        const bool take = r < q.rows;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float t = acc[e] + G::widen(raw[r][e]);
            acc[e] = take ? t : acc[e];
        }
    }
    float *dst = q.whole ? &bs.stage[checked_index((q.k << lw) + q.lc, kBlockStageFloats - VEC + 1, fails)]
                         : bs.trash;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[e] = acc[e];
}

// The ragged end of a row (fewer than VEC columns left), element by element.
template <typename G, int VEC>
__device__ __forceinline__ void stage_ragged(BlockSmem &bs, const BlockDesc &d, const LanePiece &q,
                                             const typename G::T *__restrict__ grad,
                                             int64_t grad_stride) {
    const uint16_t *pp = &bs.pos[checked_index<uint32_t>(d.first + q.k, kMaxLongChunks, d.fails) * kNRows];
    const typename G::T *gcol = grad + d.col0 + q.lc;
    for (int e = 0; e < VEC && q.lc + e < d.wc; ++e) {
        float a = 0.0f;
        for (int r = 0; r < q.rows; ++r) a = a + G::widen(gcol[(int64_t)pp[r] * grad_stride + e]);
        bs.stage[checked_index((q.k << d.lw) + q.lc + e, kBlockStageFloats, d.fails)] = a;
    }
}

// Loads of a block issued ahead of its use: the main_grad values its fold
// adds to (first), then the rows of this wave's first item. Both wait in
// registers while the workgroup folds the previous block.
template <typename G, typename M, int VEC>
__device__ __forceinline__ void block_prefetch(const BlockSmem &bs, const BlockDesc &d,
                                               const typename G::T *__restrict__ grad,
                                               int64_t grad_stride,
                                               const typename M::T *__restrict__ main_grad,
                                               int64_t mg_stride, LanePiece &q,
                                               typename G::T (&raw)[kNRows][VEC],
                                               typename M::T (&old)[kFoldCols]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const typename M::T *mrow = main_grad + (int64_t)d.row * mg_stride + d.col0;
#pragma unroll
    for (int i = 0; i < kFoldCols; ++i) {
        const int j = tid + i * kSortThreads;
        if (j < d.wc) old[i] = mrow[j];
    }
    const ItemShape<VEC> sh(d.lw, d.chunks);
    q = lane_piece<VEC>(bs, d, sh, wave, lane);
    load_piece_rows<typename G::T, VEC>(bs, d, q, grad, grad_stride, raw);
}

// The chunk sums of a block into the LDS stage: this wave's first item from
// the prefetched rows, then its further items (a block of more items than the
// workgroup has waves) with their loads issued here.
template <typename G, int VEC>
__device__ __forceinline__ void block_stage(BlockSmem &bs, const BlockDesc &d, const LanePiece &q,
                                            const typename G::T (&raw)[kNRows][VEC],
                                            const typename G::T *__restrict__ grad,
                                            int64_t grad_stride) {
    using GT = typename G::T;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    stage_piece<G, VEC>(bs, d.lw, q, raw, d.fails);
    if (q.active && !q.whole) stage_ragged<G, VEC>(bs, d, q, grad, grad_stride);
    const ItemShape<VEC> sh(d.lw, d.chunks);
    for (int it = wave + kSortWaves; it < sh.items; it += kSortWaves) {   // uniform over the wave
        const LanePiece e = lane_piece<VEC>(bs, d, sh, it, lane);
        GT more[kNRows][VEC];
        load_piece_rows<GT, VEC>(bs, d, e, grad, grad_stride, more);
        stage_piece<G, VEC>(bs, d.lw, e, more, d.fails);
        if (e.active && !e.whole) stage_ragged<G, VEC>(bs, d, e, grad, grad_stride);
    }
}

// After the stage is complete: each column adds its chunk sums in chunk order
// from +0, rounds once to grad's dtype and is added to main_grad (old values
// from block_prefetch).
template <typename G, typename M>
__device__ __forceinline__ void block_fold(const BlockSmem &bs, const BlockDesc &d,
                                           typename M::T *__restrict__ main_grad, int64_t mg_stride,
                                           const typename M::T (&old)[kFoldCols]) {
    const int tid = threadIdx.x;
    typename M::T *mrow = main_grad + (int64_t)d.row * mg_stride + d.col0;
#pragma unroll
    for (int i = 0; i < kFoldCols; ++i) {
        const int wave_j0 = (tid & ~63) + i * kSortThreads;
        if (wave_j0 < d.wc) {   // uniform over the wave
            const int j = tid + i * kSortThreads;
            const float *col = &bs.stage[j < d.wc ? j : wave_j0];
            float acc = 0.0f;
            // the adds stay in chunk order; the LDS reads of a group of 8 are
            // all issued before the first add
            int k = 0;
            for (; k + 8 <= (int)d.chunks; k += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = col[(k + u) << d.lw];
#pragma unroll
                for (int u = 0; u < 8; ++u) acc = acc + v[u];
            }
            for (; k < (int)d.chunks; ++k) acc = acc + col[k << d.lw];
            if (j < d.wc) mrow[j] = finish<G, M>(acc, old[i]);
        }
    }
}

// Wait for the flag (wave 0); stage the run records and the positions and
// rows of every long chunk in LDS (once: every block reads them from there);
// then take column blocks from the device-wide ticket until none is left
// (take = false: wait, take nothing). A record that does not describe this
// call's work is counted in the header's wait-timeout word and the blocks
// that would use it are skipped.
template <typename G, typename M, int VEC>
__device__ __forceinline__ void long_blocks(BlockSmem &bs, uint32_t *s_word,
                                            WsHeader *__restrict__ hdr,
                                            __amdgpu_buffer_rsrc_t units_rs,
                                            __amdgpu_buffer_rsrc_t runs_rs, uint32_t n_lc_max,
                                            uint32_t n_lr_max, int n, int num_embeddings,
                                            const typename G::T *__restrict__ grad,
                                            int64_t grad_stride,
                                            typename M::T *__restrict__ main_grad,
                                            int64_t mg_stride, int hidden, uint32_t epoch,
                                            bool take) {
    using GT = typename G::T;
    using MT = typename M::T;
    const int tid = threadIdx.x;
    if (tid < 64) {   // wave 0
        uint32_t nb = 0u, lc = 0u, lr = 0u;
        const bool ok = wave_wait_ready(hdr, epoch, &nb, &lc, &lr);
        if (tid == 0) {
            s_word[0] = ok ? nb : 0u;
            s_word[1] = lc;
            s_word[2] = lr;
            s_word[3] = 0u;   // staging errors, below
        }
    }
    __syncthreads();
    const uint32_t n_blocks = s_word[0];
    const uint32_t n_lc = min(s_word[1], n_lc_max), n_lr = min(s_word[2], n_lr_max);
    __syncthreads();   // every thread has read s_word before it is reused
    if (!take || n_blocks == 0u || n_lr == 0u) return;   // uniform
    // the first claim goes out before the records are loaded, so that the two
    // round trips overlap
    uint32_t first_claim = 0u;
    if (tid == 0) first_claim = fetch_add_coherent(&hdr->block_ticket, 1u);
    for (uint32_t r = (uint32_t)tid; r < n_lr; r += kSortThreads)
        bs.runs[r] = load_coherent16(runs_rs, r * (uint32_t)kRunRecordBytes);
    uint32_t bad = 0u;
    for (uint32_t c = (uint32_t)tid; c < n_lc; c += kSortThreads) {
        const u32x4 a = load_coherent16(units_rs, c * (uint32_t)kUnitRecordBytes);
        const u32x4 b = load_coherent16(units_rs, c * (uint32_t)kUnitRecordBytes + 16u);
        const uint32_t w[5] = {a.x, a.y, a.z, a.w, b.x};
        uint32_t rows = b.y & 0xffffu;
        if (b.w != epoch || (b.y >> 16) >= n_lr || b.z != c || rows < 1u || rows > (uint32_t)kNRows)
            bad = 1u;
        rows = rows < 1u ? 1u : (rows > (uint32_t)kNRows ? (uint32_t)kNRows : rows);
        bs.rows[c] = (uint8_t)rows;
#pragma unroll
        for (int i = 0; i < kNRows; ++i) {
            const uint32_t q = (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
            bs.pos[c * kNRows + i] = (uint16_t)(q < (uint32_t)n ? q : 0u);   // every row inside grad
        }
    }
    if (bad) atomicOr(&s_word[3], 1u);
    if (tid == 0) s_word[0] = first_claim;
    __syncthreads();
    const bool staged_ok = s_word[3] == 0u;   // s_word[3] is not written again
    uint32_t b = s_word[0];
    __syncthreads();   // every thread has read the claim before the next one lands
    if (b >= n_blocks) return;   // uniform
    // Software pipeline over the blocks this workgroup takes: the loads of
    // the next block are in flight while the current one is folded. Per
    // block: stage its chunk sums; barrier; issue the next block's loads
    // (its number was claimed one block earlier) and claim the one after;
    // fold this one; barrier. The main_grad loads of a block are issued
    // before its grad rows, so the wait for the rows (at its stage) also
    // covers them and the fold waits on no load in flight.
    const uint32_t one = (tid == 0) ? 1u : 0u;
    bool bad_desc = false;
    int32_t *fails = &hdr->check_failures;
    BlockDesc d = describe_block(bs, b, n_lr, n_lc, num_embeddings, hidden, staged_ok, &bad_desc,
                                 fails);
    uint32_t bad_blocks = bad_desc ? one : 0u;
    LanePiece q;
    GT raw[kNRows][VEC];
    MT old[kFoldCols];
    block_prefetch<G, M, VEC>(bs, d, grad, grad_stride, main_grad, mg_stride, q, raw, old);
    uint32_t next = 0u;
    if (tid == 0) next = fetch_add_coherent(&hdr->block_ticket, 1u);
    for (int par = 1;; par ^= 1) {
        block_stage<G, VEC>(bs, d, q, raw, grad, grad_stride);
        if (tid == 0) s_word[par] = next;   // claimed one block earlier
        __syncthreads();
        const uint32_t b1 = s_word[par];
        const bool more = b1 < n_blocks;   // uniform
        BlockDesc d1 = d;
        MT old1[kFoldCols];
        if (more) {
            d1 = describe_block(bs, b1, n_lr, n_lc, num_embeddings, hidden, staged_ok, &bad_desc,
                                fails);
            if (bad_desc) bad_blocks += one;
            block_prefetch<G, M, VEC>(bs, d1, grad, grad_stride, main_grad, mg_stride, q, raw, old1);
            if (tid == 0) next = fetch_add_coherent(&hdr->block_ticket, 1u);
        }
        if (d.valid) block_fold<G, M>(bs, d, main_grad, mg_stride, old);
        __syncthreads();   // the stage is free for the next block; s_word[par] was read
        if (!more) break;
        d = d1;
#pragma unroll
        for (int i = 0; i < kFoldCols; ++i) old[i] = old1[i];
    }
    if (bad_blocks)
        fetch_add_coherent(reinterpret_cast<uint32_t *>(&hdr->wait_timeouts), bad_blocks);
}

template <typename IdT, typename G, typename M, int VEC>
__global__ __launch_bounds__(kSortThreads) void accumulate_kernel(
    const IdT *__restrict__ ids, int n, int num_embeddings, int64_t id_base, int skip_outside,
    int pos_bits, int id_bits,
    const typename G::T *__restrict__ grad, int64_t grad_stride,
    typename M::T *__restrict__ main_grad, int64_t mg_stride, int hidden, int tiles,
    WsHeader *__restrict__ hdr, uint8_t *__restrict__ units, uint8_t *__restrict__ runs,
    uint32_t epoch, int odd_skip_long) {
    __shared__ AccSmem sm;
    __shared__ uint32_t s_word[4];   // LDS broadcasts
    const int tid = threadIdx.x;
    const uint32_t n_lc_max = (uint32_t)(2 * n / 11), n_lr_max = (uint32_t)(n / 11);
    const __amdgpu_buffer_rsrc_t units_rs = buffer_range(units, n_lc_max * (uint32_t)kUnitRecordBytes);
    const __amdgpu_buffer_rsrc_t runs_rs = buffer_range(runs, n_lr_max * (uint32_t)kRunRecordBytes);

    if (blockIdx.x == 0) {
        leader_publish<IdT>(sm.sort, ids, n, num_embeddings, id_base, skip_outside != 0, pos_bits,
                            id_bits, hidden, (int)sizeof(typename G::T), hdr, units_rs, runs_rs,
                            epoch);
    } else {
        // the waves leave this one by one, as their short-run units run out
        follower_short_runs<IdT, G, M, VEC>(sm.fol, ids, n, num_embeddings, id_base,
                                            skip_outside != 0, pos_bits, grad, grad_stride,
                                            main_grad, mg_stride, hidden, tiles,
                                            (int)blockIdx.x - 1, (int)gridDim.x - 1,
                                            &hdr->check_failures);
    }
    __syncthreads();   // the LDS of phases 1 and 2 is free from here on
    // phase 3 (a test setting keeps odd workgroups out of it)
    const bool take = !(odd_skip_long && (blockIdx.x & 1u));
    long_blocks<G, M, VEC>(sm.blk, s_word, hdr, units_rs, runs_rs, n_lc_max, n_lr_max, n,
                           num_embeddings, grad, grad_stride, main_grad, mg_stride, hidden, epoch,
                           take);

    // ---- phase 4: the last workgroup out resets the call's shared state ----
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
            store_coherent(&hdr->block_ticket, 0u);
            store_coherent(&hdr->ready, 0u);
        }
    }
}

template <typename IdT, typename G, typename M, int VEC>
hipError_t launch(const void *ids, int n, int num_embeddings, int64_t id_base, int skip_outside,
                  int pos_bits, int id_bits,
                  const void *grad, int64_t grad_stride, void *main_grad, int64_t mg_stride,
                  int hidden, void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                  int odd_skip_long, hipEvent_t kstart, hipEvent_t kstop, hipStream_t stream) {
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
    if (kstart && kstop)   // events taken by the dispatch itself: the kernel's own duration
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kSortThreads), 0, stream, kstart, kstop, 0,
                              ids_t, n, num_embeddings, id_base, skip_outside, pos_bits, id_bits,
                              grad_t, grad_stride, mg_t, mg_stride, hidden, tiles, hdr, units, runs,
                              epoch, odd_skip_long);
    else
        kernel<<<grid, kSortThreads, 0, stream>>>(ids_t, n, num_embeddings, id_base, skip_outside,
                                                  pos_bits, id_bits, grad_t, grad_stride, mg_t,
                                                  mg_stride, hidden, tiles, hdr, units, runs, epoch,
                                                  odd_skip_long);
    return hipGetLastError();
}

template <typename IdT>
hipError_t dispatch_types(bool grad_bf16, bool mg_bf16, bool vec, const void *ids, int n,
                          int num_embeddings, int64_t id_base, int skip_outside, int pos_bits,
                          int id_bits, const void *grad,
                          int64_t grad_stride, void *main_grad, int64_t mg_stride, int hidden,
                          void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                          int odd_skip_long, hipEvent_t kstart, hipEvent_t kstop,
                          hipStream_t stream) {
#define EWG_ACC(G, M, V)                                                                        \
    launch<IdT, G, M, V>(ids, n, num_embeddings, id_base, skip_outside, pos_bits, id_bits, grad,   \
                         grad_stride, main_grad, mg_stride, hidden, workspace, l, num_cus, epoch, \
                         odd_skip_long, kstart, kstop, stream)
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
                             int num_cus, uint32_t epoch, int odd_skip_long,
                             hipEvent_t kstart, hipEvent_t kstop, hipStream_t stream) {
    if (ids_int64)
        return dispatch_types<int64_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, id_base,
                                       skip_outside ? 1 : 0, pos_bits, id_bits, grad, grad_stride,
                                       main_grad, mg_stride, hidden, workspace, l, num_cus, epoch,
                                       odd_skip_long, kstart, kstop, stream);
    return dispatch_types<int32_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, id_base,
                                   skip_outside ? 1 : 0, pos_bits, id_bits, grad, grad_stride,
                                   main_grad, mg_stride, hidden, workspace, l, num_cus, epoch,
                                   odd_skip_long, kstart, kstop, stream);
}

}  // namespace ewg
