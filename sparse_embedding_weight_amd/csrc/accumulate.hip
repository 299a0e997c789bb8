// Fused kernel: sort, single-chunk runs, and the chunks of long runs. One
// 1024-thread workgroup per compute unit (at least two workgroups).
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad": the
// introduction's two bullets (sort the ids with their positions, sum each
// token's rows in position order into fp32 partial sums of up to 10 rows, add
// the partial sums in order from 0, round once to the gradient dtype, add in
// fp32 into main_grad and round to its dtype), _sort_tokens_kernel and
// _partial_sums_kernel ("a run of at most NROWS rows is finished here").
//
// The two kinds of runs need different things:
//   * a run of at most 10 rows is one chunk. Its rows only need to be found
//     and put in position order, which needs no global sort. Every workgroup
//     but 0 (the "followers") builds an LDS hash table of all ids (occurrence
//     count per id, hash slot per position), takes the runs of at most 10 rows
//     falling in its equal-cost share of the first-occurrence order (which
//     every follower computes identically from its own table), gathers their
//     positions, orders them, sums the rows and finishes the main_grad row,
//     all while workgroup 0 sorts;
//   * a run of more than 10 rows is cut into chunks counted from its first
//     row, which needs its rows in position order: workgroup 0 (dispatched
//     first, so it never waits for anyone) radix-sorts the packed keys in LDS
//     (sort_lds.h), lists the chunks of long runs with their byte cost,
//     publishes the sorted keys and that list in the workspace with
//     device-coherent stores, waits for them to complete and then sets the
//     ready flag to this call's epoch (a nonzero number the host draws per
//     call). The followers wait for the flag, copy the list into LDS with
//     device-coherent loads (checking every entry against its bounds), and then
//     every wave of every workgroup takes a contiguous range of (long chunk,
//     column tile) units of about equal byte cost and stores their fp32 sums in
//     the partial buffer. The ordered combine of those sums is the next kernel
//     (long_run_sums.hip), which also sets the flag back to 0.
//
// A column tile is 64 lanes x VEC columns (8 for bf16 grad, 4 for fp32), laid
// out in lane-contiguous pieces (piece_cols in ewg_device.h), and the rows of up
// to kTilesPerUnit tiles of a chunk are loaded before the first add.
#include "ewg_device.h"
#include "ewg_internal.h"
#include "sort_lds.h"

namespace ewg {
namespace {

constexpr int kTilesPerUnit = 4;         // most column tiles of one chunk per batch of loads
constexpr int64_t kWaitLimit = 1 << 22;  // polls of the ready flag before giving up (seconds)
constexpr int kHashSlots = 16384;        // > 2 x kMaxTokens: linear probing always ends
constexpr int kHashBits = 14;
constexpr int kOwnedMax = 256;           // short runs gathered per round by one follower
constexpr uint32_t kIdMask = (1u << 20) - 1;   // key word: id + 1 in 20 bits, round mark above

struct FollowerSmem {
    uint32_t key[kHashSlots];               // (id + 1) | (round-local run + 1) << 20; 0 = empty
    uint32_t cnt[kHashSlots];               // occurrences | first position << 16
    uint16_t slot_of_pos[kMaxTokens];
    uint16_t run_pos[kOwnedMax][kNRows];
    uint32_t run_len[kOwnedMax];
    uint32_t run_id[kOwnedMax];
    uint32_t run_slot[kOwnedMax];
    uint64_t scan[kSortWaves + 1];
    int bad;
    uint32_t first_rank;   // number of this follower's first run
    uint32_t n_mine;       // runs in this follower's share
};

struct TableSmem {                          // the published long-chunk list, copied
    uint32_t keys[kMaxTokens];
    uint32_t info[kMaxTokens];
    uint32_t cost[kMaxTokens + 1];
};

union AccSmem {
    SortSmem sort;
    FollowerSmem fol;
    TableSmem tab;
};

__device__ __forceinline__ uint32_t hash_home(uint32_t id) {
    return (id * 0x9E3779B1u) >> (32 - kHashBits);
}

// NT full column tiles of one chunk of exactly R rows on the vector path,
// tiles starting at column tile_col (wave-uniform), k * 64 * VEC apart: the
// R x NT row loads (and the main_grad loads of a single-chunk run) are
// straight-line code, so they are all in flight before the first add.
// dest < 0: finish into main_grad row `row`; else store the fp32 chunk sums
// in row `dest` of the partial buffer.
template <typename G, typename M, int VEC, int R, int NT>
__device__ __forceinline__ void chunk_tiles(const int32_t *pos, int row, int dest,
                                            const typename G::T *__restrict__ grad,
                                            int64_t grad_stride, typename M::T *__restrict__ main_grad,
                                            int64_t mg_stride, float *__restrict__ partial,
                                            int64_t partial_stride, int tile_col) {
    using GT = typename G::T;
    using MT = typename M::T;
    constexpr int P = piece_cols<G, M, VEC>(), S = VEC / P;
    const int lane = threadIdx.x & 63;
    int col[NT][S];
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
        for (int s = 0; s < S; ++s) col[k][s] = tile_col + k * 64 * VEC + s * 64 * P + lane * P;

    GT raw[R][NT][VEC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const GT *grow = grad + (int64_t)pos[r] * grad_stride;
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int s = 0; s < S; ++s) load_piece<GT, P>(grow + col[k][s], &raw[r][k][s * P]);
    }
    MT *mrow = main_grad + (int64_t)row * mg_stride;
    MT old[NT][VEC];
    if (dest < 0) {
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int s = 0; s < S; ++s) load_piece<MT, P>(mrow + col[k][s], &old[k][s * P]);
    }

    float acc[NT][VEC];
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[k][e] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[k][e] = acc[k][e] + G::widen(raw[r][k][e]);

    if (dest < 0) {
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            MT out[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) out[e] = finish<G, M>(0.0f + acc[k][e], old[k][e]);
#pragma unroll
            for (int s = 0; s < S; ++s) store_piece<MT, P>(mrow + col[k][s], &out[s * P]);
        }
    } else {
        float *prow = partial + (int64_t)dest * partial_stride;
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int s = 0; s < S; ++s) store_piece<float, P>(prow + col[k][s], &acc[k][s * P]);
    }
}

// The ragged last tile (starting at column tile_col) of one chunk, element by
// element, in the same lane layout.
template <typename G, typename M, int VEC>
__device__ __forceinline__ void chunk_ragged_tile(const int32_t *pos, int nrows, int row, int dest,
                                                  const typename G::T *__restrict__ grad,
                                                  int64_t grad_stride,
                                                  typename M::T *__restrict__ main_grad,
                                                  int64_t mg_stride, float *__restrict__ partial,
                                                  int64_t partial_stride, int hidden, int tile_col) {
    using MT = typename M::T;
    constexpr int P = piece_cols<G, M, VEC>(), S = VEC / P;
    const int lane = threadIdx.x & 63;
    for (int s = 0; s < S; ++s)
        for (int i = 0; i < P; ++i) {
            const int j = tile_col + s * 64 * P + lane * P + i;
            if (j >= hidden) continue;
            float acc = 0.0f;
            for (int r = 0; r < nrows; ++r) acc = acc + G::widen(grad[(int64_t)pos[r] * grad_stride + j]);
            if (dest < 0) {
                MT *m = main_grad + (int64_t)row * mg_stride + j;
                *m = finish<G, M>(0.0f + acc, *m);
            } else {
                partial[(int64_t)dest * partial_stride + j] = acc;
            }
        }
}

// Tiles per batch of loads for chunks of R rows: as many as fit about 256 bytes
// of loaded data, old main_grad and sums per lane (64 registers), at most
// kTilesPerUnit.
template <typename G, typename M, int VEC, int R>
constexpr int tiles_per_batch() {
    constexpr int per_tile = R * VEC * (int)sizeof(typename G::T) +
                             VEC * (int)sizeof(typename M::T) + VEC * 4;
    constexpr int b = 256 / per_tile;
    return b < 1 ? 1 : (b > kTilesPerUnit ? kTilesPerUnit : b);
}

// Tiles [t0, t_end) of one chunk of R rows: full tiles in batches of loads,
// then the ragged last tile if it is among them.
template <typename G, typename M, int VEC, int R>
__device__ __forceinline__ void chunk_tile_range(const int32_t *pos, int row, int dest,
                                                 const typename G::T *__restrict__ grad,
                                                 int64_t grad_stride,
                                                 typename M::T *__restrict__ main_grad,
                                                 int64_t mg_stride, float *__restrict__ partial,
                                                 int64_t partial_stride, int hidden, int t0,
                                                 int t_end, int full_tiles) {
    constexpr int B = tiles_per_batch<G, M, VEC, R>();
    const int t_full = t_end < full_tiles ? t_end : full_tiles;
    int t = t0;
    for (; t + B <= t_full; t += B)
        chunk_tiles<G, M, VEC, R, B>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, t * 64 * VEC);
    for (; t < t_full; ++t)
        chunk_tiles<G, M, VEC, R, 1>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, t * 64 * VEC);
    if (t < t_end)
        chunk_ragged_tile<G, M, VEC>(pos, R, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, hidden, t * 64 * VEC);
}

// Dispatch on the row count of a chunk (1..10).
template <typename G, typename M, int VEC>
__device__ __forceinline__ void chunk_tiles_any(const int32_t *pos, int nrows, int row, int dest,
                                                const typename G::T *__restrict__ grad,
                                                int64_t grad_stride,
                                                typename M::T *__restrict__ main_grad,
                                                int64_t mg_stride, float *__restrict__ partial,
                                                int64_t partial_stride, int hidden, int t0,
                                                int t_end, int full_tiles) {
#define EWG_CHUNK(R)                                                                           \
    case R:                                                                                    \
        chunk_tile_range<G, M, VEC, R>(pos, row, dest, grad, grad_stride, main_grad, mg_stride, \
                                       partial, partial_stride, hidden, t0, t_end, full_tiles); \
        break;
    switch (nrows) {
        EWG_CHUNK(1) EWG_CHUNK(2) EWG_CHUNK(3) EWG_CHUNK(4) EWG_CHUNK(5)
        EWG_CHUNK(6) EWG_CHUNK(7) EWG_CHUNK(8) EWG_CHUNK(9) EWG_CHUNK(10)
        default: break;
    }
#undef EWG_CHUNK
}

// Follower part 1: the runs of at most 10 rows in this follower's share.
// Every follower inserts all ids into its LDS hash table (occurrences and the
// first position per id, the slot of every position). Walking the positions
// in order, the first occurrence of every id with at most 10 occurrences
// carries the byte cost of its run; follower `me` takes the runs whose cost
// prefix starts in [me, me + 1) * total / followers. That order and those
// costs depend only on the ids, so all followers agree without talking. The
// positions of the taken runs are gathered in rounds of up to kOwnedMax runs,
// put in order, and the runs finished in main_grad.
template <typename IdT, typename G, typename M, int VEC>
__device__ __forceinline__ void follower_short_runs(FollowerSmem &fs, const IdT *__restrict__ ids,
                                                    int n, int num_embeddings,
                                                    const typename G::T *__restrict__ grad,
                                                    int64_t grad_stride,
                                                    typename M::T *__restrict__ main_grad,
                                                    int64_t mg_stride, int hidden, int tiles,
                                                    int me, int followers) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int kSlotsPerThread = kHashSlots / kSortThreads;

    // load the ids (all 8 loads in flight) while the table is cleared
    int64_t id[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int p = i * kSortThreads + tid;
        id[i] = (int64_t)ids[p < n ? p : n - 1];
    }
#pragma unroll
    for (int k = 0; k < kSlotsPerThread; ++k) {
        fs.key[k * kSortThreads + tid] = 0u;
        fs.cnt[k * kSortThreads + tid] = 0u;
    }
    if (tid == 0) fs.bad = 0;
    __syncthreads();

    // insert: occurrences per id, slot per position
    int bad = 0;
    uint32_t slot[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int p = i * kSortThreads + tid;
        slot[i] = 0;
        if (p >= n) continue;
        if (id[i] < 0 || id[i] >= num_embeddings) {
            ++bad;
            continue;
        }
        const uint32_t k1 = (uint32_t)id[i] + 1u;
        uint32_t h = hash_home((uint32_t)id[i]);
        for (;;) {
            const uint32_t cur = fs.key[h];
            if (cur == k1) break;
            if (cur == 0u) {
                const uint32_t old = atomicCAS(&fs.key[h], 0u, k1);
                if (old == 0u || old == k1) break;
            }
            h = (h + 1u) & (kHashSlots - 1);
        }
        atomicAdd(&fs.cnt[h], 1u);
        fs.slot_of_pos[p] = (uint16_t)h;
        slot[i] = h;
    }
    if (bad) atomicAdd(&fs.bad, bad);
    __syncthreads();
    if (fs.bad) return;   // uniform: the sorting workgroup reports it, nothing is touched

    // first position per id: the high half starts at all ones, then the
    // smallest position wins (the low half, the count, is the same for all)
#pragma unroll
    for (int k = 0; k < kSlotsPerThread; ++k) {
        const int h = k * kSortThreads + tid;
        if (fs.key[h]) fs.cnt[h] |= 0xffff0000u;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int p = i * kSortThreads + tid;
        if (p < n) atomicMin(&fs.cnt[slot[i]], ((uint32_t)p << 16) | (fs.cnt[slot[i]] & 0xffffu));
    }
    __syncthreads();

    // per-tile byte cost of a run of c rows, in 16-byte lane loads
    const uint32_t row_cost = (uint32_t)(VEC * sizeof(typename G::T) + 15) / 16;
    const uint32_t end_cost = 2u * (uint32_t)(VEC * sizeof(typename M::T) + 15) / 16;
    const int full_tiles = hidden / (64 * VEC);
    const int groups = (tiles + kTilesPerUnit - 1) / kTilesPerUnit;

    for (int r0 = 0;; r0 += kOwnedMax) {
        if (tid == 0) {
            fs.first_rank = 0xffffffffu;
            fs.n_mine = 0u;
        }
        // positions in blocked order: thread t owns [8t, 8t + 8); low 32 bits
        // of the scanned value = cost, high 32 bits = number of runs
        const int p0 = tid * kSortItems;
        uint64_t v[kSortItems];
        uint64_t sum = 0;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const int p = p0 + j;
            v[j] = 0;
            if (p < n) {
                const uint32_t w = fs.cnt[fs.slot_of_pos[p]];
                const uint32_t c = w & 0xffffu;
                if ((w >> 16) == (uint32_t)p && c <= (uint32_t)kNRows)
                    v[j] = (uint64_t)(c * row_cost + end_cost) | (1ull << 32);
            }
            sum += v[j];
        }
        uint64_t total;
        const uint64_t run = block_exclusive_scan(sum, fs.scan, &total);
        const uint64_t cost_all = total & 0xffffffffull;
        const uint64_t lo = cost_all * (uint64_t)me / (uint64_t)followers;
        const uint64_t hi = cost_all * (uint64_t)(me + 1) / (uint64_t)followers;
        // runs are numbered in position order; this follower's (cost start in
        // [lo, hi)) are a contiguous range of numbers
        {
            uint64_t x = run;
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < kSortItems; ++j) {
                const uint64_t start = x & 0xffffffffull;
                if (v[j] && start >= lo && start < hi) {
                    atomicMin(&fs.first_rank, (uint32_t)(x >> 32));
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
            uint64_t x = run;
#pragma unroll
            for (int j = 0; j < kSortItems; ++j) {
                const uint64_t start = x & 0xffffffffull;
                if (v[j] && start >= lo && start < hi) {
                    const int li = (int)((uint32_t)(x >> 32) - first) - r0;
                    if (li >= 0 && li < kOwnedMax) {
                        const uint32_t h = fs.slot_of_pos[p0 + j];
                        fs.run_id[li] = (fs.key[h] & kIdMask) - 1u;
                        fs.run_len[li] = 0u;
                        fs.run_slot[li] = h;
                        fs.key[h] |= (uint32_t)(li + 1) << 20;
                    }
                }
                x += v[j];
            }
        }
        __syncthreads();
        const int n_round = total_mine - r0 < kOwnedMax ? total_mine - r0 : kOwnedMax;
        if (n_round <= 0) break;

        // gather the positions of the round's runs, then put each run in order
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            const int p = i * kSortThreads + tid;
            if (p >= n) continue;
            const uint32_t m = fs.key[fs.slot_of_pos[p]] >> 20;
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

        // (run, group of kTilesPerUnit tiles) units over the waves
        const int units = n_round * groups;
        for (int u = wave; u < units; u += kSortWaves) {
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
        __syncthreads();
        if (tid < n_round) fs.key[fs.run_slot[tid]] &= kIdMask;
        __syncthreads();
        if (total_mine - r0 <= kOwnedMax) break;
    }
}

// First unit whose start lies at or after x, in units of per-tile cost: chunk
// c starts at cost[c] * tiles and its tiles cost cost[c+1] - cost[c] each.
__device__ __forceinline__ void first_unit(const uint32_t *cost, int n_chunks, int tiles,
                                           uint64_t x, int &c, int &t) {
    const uint64_t q = x / (uint64_t)tiles;
    int lo = 0, hi = n_chunks;   // largest c with cost[c] <= q, in [0, n_chunks)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((uint64_t)__builtin_amdgcn_readfirstlane(cost[mid]) <= q) lo = mid; else hi = mid;
    }
    c = lo;
    const uint64_t start = (uint64_t)__builtin_amdgcn_readfirstlane(cost[c]) * (uint64_t)tiles;
    const uint64_t per_tile = (uint64_t)(__builtin_amdgcn_readfirstlane(cost[c + 1]) -
                                         __builtin_amdgcn_readfirstlane(cost[c]));
    const uint64_t tt = (x - start + per_tile - 1) / per_tile;   // first tile starting at or after x
    if (tt >= (uint64_t)tiles) {
        ++c;
        t = 0;
    } else {
        t = (int)tt;
    }
}

template <typename IdT, typename G, typename M, int VEC>
__global__ __launch_bounds__(kSortThreads) void accumulate_kernel(
    const IdT *__restrict__ ids, int n, int num_embeddings, int pos_bits, int id_bits,
    const typename G::T *__restrict__ grad, int64_t grad_stride,
    typename M::T *__restrict__ main_grad, int64_t mg_stride, float *__restrict__ partial,
    int64_t partial_stride, int hidden, int tiles, WsHeader *__restrict__ hdr,
    uint32_t *__restrict__ tab_keys, uint32_t *__restrict__ tab_info,
    uint32_t *__restrict__ tab_cost, LongRunDesc *__restrict__ long_runs, uint32_t epoch) {
    __shared__ AccSmem sm;
    __shared__ int s_flag;
    const int tid = threadIdx.x, wave = tid >> 6;

    const uint32_t *keys, *info, *cost;
    int n_lc;              // chunks of long runs
    uint32_t cost_total;   // their summed per-tile cost
    if (blockIdx.x == 0) {
        // ---- the sorting workgroup ----
        SortSmem &ss = sm.sort;
        const SortOutputs out = {{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr},
                                 long_runs, hdr};
        const int bad = load_keys<IdT>(ss, ids, n, num_embeddings, pos_bits);
        if (bad) {
            report_invalid(out, bad);
            n_lc = 0;
            cost_total = 0;
            keys = info = cost = nullptr;
        } else {
            const int cur = radix_sort_ids(ss, pos_bits, id_bits);
            const SortResult res = mark_runs(ss, cur, n, pos_bits, out);
            // the long chunks in order: a long chunk's index is stored in its word
            uint32_t *lc_info = ss.aux;
            uint32_t *lc_cost = ss.aux + kMaxTokens;
            for (int c = tid; c < res.n_chunks; c += kSortThreads) {
                const uint32_t x = res.chunk_info[c];
                if (x & kInfoLong) lc_info[info_long_chunk(x)] = x;
            }
            __syncthreads();
            n_lc = res.n_long_chunks;
            // per-tile cost in 16-byte lane loads: the grad rows and the partial store
            const uint32_t row_cost = (uint32_t)(VEC * sizeof(typename G::T) + 15) / 16;
            const uint32_t end_cost = (uint32_t)(VEC * 4 + 15) / 16;
            cost_total = chunk_cost_prefix(ss, lc_info, n_lc, lc_cost, row_cost, end_cost);
            keys = res.keys;
            info = lc_info;
            cost = lc_cost;
            // device-coherent stores: they reach the coherence point, no L2 write-back
            for (int i = tid; i < n; i += kSortThreads)
                __hip_atomic_store(&tab_keys[i], keys[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int i = tid; i < n_lc; i += kSortThreads)
                __hip_atomic_store(&tab_info[i], info[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int i = tid; i <= n_lc; i += kSortThreads)
                __hip_atomic_store(&tab_cost[i], cost[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) {
            __hip_atomic_store(&hdr->num_long_chunks, n_lc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->cost_total, cost_total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // every store of every wave has completed, then the flag goes up
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&hdr->ready, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // ---- the followers: short runs, then wait for the long-chunk list ----
        follower_short_runs<IdT, G, M, VEC>(sm.fol, ids, n, num_embeddings, grad, grad_stride,
                                            main_grad, mg_stride, hidden, tiles,
                                            (int)blockIdx.x - 1, (int)gridDim.x - 1);
        if (tid == 0) {
            int ok = 1;
            int64_t spins = 0;
            while (__hip_atomic_load(&hdr->ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kWaitLimit) {
                    atomicAdd(&hdr->wait_timeouts, 1);
                    ok = 0;
                    break;
                }
            }
            s_flag = ok;
        }
        __syncthreads();
        if (!s_flag) return;   // uniform; never expected
        n_lc = __hip_atomic_load(&hdr->num_long_chunks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        cost_total = __hip_atomic_load(&hdr->cost_total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the list must be in bounds whatever was read: clamp the count
        const int max_lc = 2 * n / 11;
        n_lc = n_lc < 0 ? 0 : (n_lc > max_lc ? max_lc : n_lc);
        if (n_lc > 0) {
            // one round trip: every load of the copy is issued before the first store
            TableSmem &tb = sm.tab;
            uint32_t kv[kSortItems], iv[2], cv[2];
#pragma unroll
            for (int i = 0; i < kSortItems; ++i) {
                const int j = i * kSortThreads + tid;
                kv[i] = __hip_atomic_load(&tab_keys[j < n ? j : n - 1], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int j = i * kSortThreads + tid;
                iv[i] = __hip_atomic_load(&tab_info[j < n_lc ? j : n_lc - 1], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                cv[i] = __hip_atomic_load(&tab_cost[j <= n_lc ? j : n_lc], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            }
            const uint32_t pos_mask = (1u << pos_bits) - 1u;
#pragma unroll
            for (int i = 0; i < kSortItems; ++i) {
                const int j = i * kSortThreads + tid;
                // keep every position below n
                if (j < n) tb.keys[j] = (kv[i] & pos_mask) < (uint32_t)n ? kv[i] : (kv[i] & ~pos_mask);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int j = i * kSortThreads + tid;
                if (j < n_lc) {
                    // first slot and rows inside [0, n), chunk index inside the list
                    uint32_t x = iv[i];
                    const int f = info_first(x), r = info_rows(x);
                    if (f + r > n || info_long_chunk(x) >= max_lc) x = (uint32_t)j << 17;   // 1 row at slot 0
                    tb.info[j] = x;
                }
                if (j <= n_lc) tb.cost[j] = cv[i];
            }
            __syncthreads();
            // costs must increase for the range search: one wave checks
            if (wave == 0) {
                bool ok = true;
                for (int j = tid; j < n_lc; j += 64) ok = ok && tb.cost[j] < tb.cost[j + 1];
                if (!__all(ok)) {
                    for (int j = tid; j <= n_lc; j += 64) tb.cost[j] = (uint32_t)j;
                    if (tid == 0) cost_total = (uint32_t)n_lc;
                }
            }
            __syncthreads();
            cost_total = tb.cost[n_lc];
        }
        keys = sm.tab.keys;
        info = sm.tab.info;
        cost = sm.tab.cost;
    }
    if (n_lc == 0) return;

    // ---- long chunks: this wave's units start in [x0, x1) of the cost line ----
    const uint32_t pos_mask = (1u << pos_bits) - 1u;
    const uint64_t nw = (uint64_t)gridDim.x * kSortWaves;
    const uint64_t gw = (uint64_t)blockIdx.x * kSortWaves + (uint64_t)__builtin_amdgcn_readfirstlane(wave);
    const uint64_t total = (uint64_t)cost_total * (uint64_t)tiles;
    int c, t, ce, te;
    first_unit(cost, n_lc, tiles, total * gw / nw, c, t);
    if (gw + 1 == nw) {
        ce = n_lc;
        te = 0;
    } else {
        first_unit(cost, n_lc, tiles, total * (gw + 1) / nw, ce, te);
    }
    const int full_tiles = hidden / (64 * VEC);
    for (; c < ce || (c == ce && t < te); ++c, t = 0) {
        const uint32_t x = __builtin_amdgcn_readfirstlane(info[c]);
        const int f = info_first(x), nrows = info_rows(x);
        const int dest = info_long_chunk(x);
        int32_t pos[kNRows];
#pragma unroll
        for (int r = 0; r < kNRows; ++r)
            pos[r] = r < nrows ? (int32_t)(__builtin_amdgcn_readfirstlane(keys[f + r]) & pos_mask) : 0;
        const int t_stop = c == ce ? te : tiles;
        chunk_tiles_any<G, M, VEC>(pos, nrows, 0, dest, grad, grad_stride, main_grad, mg_stride,
                                   partial, partial_stride, hidden, t, t_stop, full_tiles);
    }
}

template <typename IdT, typename G, typename M, int VEC>
hipError_t launch(const void *ids, int n, int num_embeddings, int pos_bits, int id_bits,
                  const void *grad, int64_t grad_stride, void *main_grad, int64_t mg_stride,
                  int hidden, void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                  hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    const int tiles = (hidden + 64 * VEC - 1) / (64 * VEC);
    // at least one follower; workgroup 0 never waits, so any residency works
    const int grid = num_cus > 2 ? num_cus : 2;
    accumulate_kernel<IdT, G, M, VEC><<<grid, kSortThreads, 0, stream>>>(
        static_cast<const IdT *>(ids), n, num_embeddings, pos_bits, id_bits,
        static_cast<const typename G::T *>(grad), grad_stride,
        static_cast<typename M::T *>(main_grad), mg_stride,
        reinterpret_cast<float *>(ws + l.partial), l.partial_stride, hidden, tiles,
        reinterpret_cast<WsHeader *>(ws), reinterpret_cast<uint32_t *>(ws + l.keys),
        reinterpret_cast<uint32_t *>(ws + l.info), reinterpret_cast<uint32_t *>(ws + l.cost),
        reinterpret_cast<LongRunDesc *>(ws + l.long_runs), epoch);
    return hipGetLastError();
}

template <typename IdT>
hipError_t dispatch_types(bool grad_bf16, bool mg_bf16, bool vec, const void *ids, int n,
                          int num_embeddings, int pos_bits, int id_bits, const void *grad,
                          int64_t grad_stride, void *main_grad, int64_t mg_stride, int hidden,
                          void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                          hipStream_t stream) {
#define EWG_ACC(G, M, V)                                                                        \
    launch<IdT, G, M, V>(ids, n, num_embeddings, pos_bits, id_bits, grad, grad_stride, main_grad, \
                         mg_stride, hidden, workspace, l, num_cus, epoch, stream)
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
                             const void *ids, int n, int num_embeddings, int pos_bits, int id_bits,
                             const void *grad, int64_t grad_stride, void *main_grad,
                             int64_t mg_stride, int hidden, void *workspace, const WsLayout &l,
                             int num_cus, uint32_t epoch, hipStream_t stream) {
    if (ids_int64)
        return dispatch_types<int64_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, pos_bits,
                                       id_bits, grad, grad_stride, main_grad, mg_stride, hidden,
                                       workspace, l, num_cus, epoch, stream);
    return dispatch_types<int32_t>(grad_bf16, mg_bf16, vec, ids, n, num_embeddings, pos_bits,
                                   id_bits, grad, grad_stride, main_grad, mg_stride, hidden,
                                   workspace, l, num_cus, epoch, stream);
}

}  // namespace ewg
