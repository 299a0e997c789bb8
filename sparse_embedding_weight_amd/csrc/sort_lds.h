// The sort step as device code for one 1024-thread workgroup: packed
// (id << pos_bits | position) keys sorted in LDS, runs of equal ids marked,
// and the chunk table built in LDS. Used by the fused accumulate kernel (only
// its workgroup 0 sorts; it publishes the long chunks and runs through the
// workspace), by the many-token path's tile sort, and by the sort-only kernel
// that writes the tables out.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad":
// _sort_tokens_kernel (sort the (token, position) pairs, give every sorted
// slot the first and last slot of its run, list the runs longer than NROWS),
// _position_bits, and the introduction, first bullet (the ids are sorted with
// their positions and each id's rows are summed in the order of those
// positions).
//
// The keys enter in position order and every radix pass is stable, so
// sorting on the id bits alone yields (id, position) order; the position bits
// need no pass. Ids have at most 19 bits (31 - 12): at most two passes of at
// most 10 bits. Inside a pass each wavefront ranks its keys with one ballot
// per digit bit (the lanes holding the same digit), a masked popcount (the
// rank among them) and a per-wave LDS counter per digit that carries counts
// across the wave's 8 groups of 64 keys; a digit-major scan of the 16 x 2^bits
// counters gives the scatter offsets.
#pragma once

#include "ewg_internal.h"

namespace ewg {

constexpr int kWaveSlots = kSortItems * 64;   // 512 consecutive slots per wave

// chunk_info word: first sorted slot (13 bits) | rows - 1 (4 bits) << 13 |
// long-chunk index (11 bits) << 17 | run-is-long (1 bit) << 28
constexpr uint32_t kInfoLong = 1u << 28;
__device__ __forceinline__ int info_first(uint32_t x) { return (int)(x & 0x1fffu); }
__device__ __forceinline__ int info_rows(uint32_t x) { return (int)((x >> 13) & 0xfu) + 1; }
__device__ __forceinline__ int info_long_chunk(uint32_t x) { return (int)((x >> 17) & 0x7ffu); }
static_assert(2 * kMaxTokens / 11 <= 0x7ff, "long-chunk index fits 11 bits");

struct SortSmem {
    uint32_t keys[2][kMaxTokens];               // ping-pong key buffers
    uint32_t aux[kSortWaves << kMaxDigitBits];  // radix counters, then run starts
    uint64_t scan[kSortWaves + 1];
    int bad;
    int n_keys;                                 // keys of ids inside the table (sorted first)
    int n_chunks, n_long, n_long_chunks, n_runs;
    int long_seen;                              // a quick check found an id on > 10 keys
};

// Sort results for one call.
struct SortResult {
    const uint32_t *keys;        // sorted keys, LDS
    const uint32_t *chunk_info;  // n_chunks words, LDS
    int n_chunks, n_long, n_long_chunks, n_runs;
};

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sums over the 64 lanes of a wave with DPP moves (GFX9):
// row_shr:1, 2, 4 and 8 sum inside each row of 16 lanes (a lane with no
// source reads 0), then row_bcast:15 adds the last lane of rows 0 and 2 to
// rows 1 and 3, and row_bcast:31 adds lane 31 to rows 2 and 3 (a row outside
// the row mask keeps the 0 it started from). Every lane of the wave must be
// active.
constexpr int kDppRowShr = 0x110;       // + shift (1..15)
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_take(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_take64(uint64_t v) {
    const uint32_t lo = dpp_take<CTRL, ROW_MASK>((uint32_t)v);
    const uint32_t hi = dpp_take<CTRL, ROW_MASK>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_inclusive_scan32(uint32_t v) {
    v += dpp_take<kDppRowShr + 1, 0xf>(v);
    v += dpp_take<kDppRowShr + 2, 0xf>(v);
    v += dpp_take<kDppRowShr + 4, 0xf>(v);
    v += dpp_take<kDppRowShr + 8, 0xf>(v);
    v += dpp_take<kDppRowBcast15, 0xa>(v);
    v += dpp_take<kDppRowBcast31, 0xc>(v);
    return v;
}

__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t v, int /*lane*/) {
    v += dpp_take64<kDppRowShr + 1, 0xf>(v);
    v += dpp_take64<kDppRowShr + 2, 0xf>(v);
    v += dpp_take64<kDppRowShr + 4, 0xf>(v);
    v += dpp_take64<kDppRowShr + 8, 0xf>(v);
    v += dpp_take64<kDppRowBcast15, 0xa>(v);
    v += dpp_take64<kDppRowBcast31, 0xc>(v);
    return v;
}

// Exclusive prefix sum over the 1024 threads in thread order; *total gets the
// sum of all. Every thread of the workgroup must call it.
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t *s_tmp,
                                                         uint64_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t inc = wave_inclusive_scan(v, lane);
    if (lane == 63) s_tmp[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        uint64_t w = lane < kSortWaves ? s_tmp[lane] : 0;
        uint64_t wi = wave_inclusive_scan(w, lane);
        if (lane < kSortWaves) s_tmp[lane] = wi - w;
        if (lane == kSortWaves - 1) s_tmp[kSortWaves] = wi;
    }
    __syncthreads();
    uint64_t excl = s_tmp[wave] + inc - v;
    *total = s_tmp[kSortWaves];
    __syncthreads();
    return excl;
}

// The same over 32-bit values (the scan uses s_tmp[0 .. kSortWaves]).
__device__ __forceinline__ uint32_t block_exclusive_scan32(uint32_t v, uint32_t *s_tmp,
                                                           uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_inclusive_scan32(v);
    if (lane == 63) s_tmp[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const uint32_t w = lane < kSortWaves ? s_tmp[lane] : 0u;
        const uint32_t wi = wave_inclusive_scan32(w);
        if (lane < kSortWaves) s_tmp[lane] = wi - w;
        if (lane == kSortWaves - 1) s_tmp[kSortWaves] = wi;
    }
    __syncthreads();
    const uint32_t excl = s_tmp[wave] + inc - v;
    *total = s_tmp[kSortWaves];
    __syncthreads();
    return excl;
}

// Load the ids and build the keys in position order: wave w holds slots
// [w*512, w*512 + 512) as 8 groups of 64; slots past n hold 0xffffffff, which
// every pass ranks last. The key of position s holds id - id_base, for ids in
// [id_base, id_base + num_embeddings). With skip_outside, any other id is
// left out: its slot holds 0xffffffff too (the id bits of a kept key are never
// all ones, so kept keys rank first) and sm.n_keys counts the kept ones.
// Otherwise an id outside is invalid: the number of those is returned (the
// same value in every thread), and n_keys is n.
template <typename IdT>
__device__ __forceinline__ int load_keys(SortSmem &sm, const IdT *__restrict__ ids, int n, int num_embeddings,
                         int pos_bits, int64_t id_base, bool skip_outside) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        sm.bad = 0;
        sm.n_keys = 0;
    }
    int64_t id[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {   // unconditional loads: all 8 in flight
        const int s = wave * kWaveSlots + i * 64 + lane;
        id[i] = (int64_t)ids[s < n ? s : n - 1];
    }
    __syncthreads();
    int bad = 0, kept = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int s = wave * kWaveSlots + i * 64 + lane;
        uint32_t key = 0xffffffffu;
        if (s < n) {
            const int64_t v = id[i] - id_base;
            if (v < 0 || v >= num_embeddings) {
                if (!skip_outside) {
                    ++bad;
                    key = 0;
                }
            } else {
                key = ((uint32_t)v << pos_bits) | (uint32_t)s;
                ++kept;
            }
        }
        sm.keys[0][s] = key;
    }
    if (bad) atomicAdd(&sm.bad, bad);
    if (kept) atomicAdd(&sm.n_keys, kept);
    __syncthreads();
    return sm.bad;
}

// Stable LSD radix passes over the id bits. Returns the buffer that holds
// the sorted keys.
__device__ __forceinline__ int radix_sort_ids(SortSmem &sm, int pos_bits, int id_bits, int n) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int cur = 0;
    const int npass = (id_bits + kMaxDigitBits - 1) / kMaxDigitBits;
    int done = 0;
    for (int p = 0; p < npass; ++p) {
        const int bits = (id_bits - done + (npass - p) - 1) / (npass - p);
        const int shift = pos_bits + done;
        done += bits;
        const uint32_t mask = (1u << bits) - 1u;
        const int radix = 1 << bits;
        uint32_t *cnt = sm.aux + (wave << kMaxDigitBits);

        for (int d = lane; d < radix; d += 64) cnt[d] = 0;

        uint32_t key[kSortItems], dig[kSortItems], rank[kSortItems];
        uint64_t peers[kSortItems];
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            key[i] = sm.keys[cur][wave * kWaveSlots + i * 64 + lane];
            dig[i] = (key[i] >> shift) & mask;
            peers[i] = ~0ull;
        }
        // Slots [n, kMaxTokens) hold padding keys (all ones) in every pass: they
        // come after every position and each pass is stable. A wave of them
        // only ranks them in order, with the largest digit.
        if (wave * kWaveSlots >= n) {   // uniform over the wave
#pragma unroll
            for (int i = 0; i < kSortItems; ++i) rank[i] = (uint32_t)(i * 64 + lane);
            if (lane == 0) cnt[mask] = (uint32_t)kWaveSlots;   // after the clearing above
        } else {
        // lanes of the same 64-key group with the same digit (8 groups in
        // flight): per bit, m is all ones where the lane's bit is set and
        // every lane keeps the peers whose ballot bit equals its own,
        // peers & ~(m ^ ballot) on each 32-bit half (one v_bitop3 on gfx950)
        for (int b = 0; b < bits; ++b) {
#pragma unroll
            for (int i = 0; i < kSortItems; ++i) {
                const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)dig[i], b, 1);
                const uint64_t bal = __ballot(m != 0u);
                const uint32_t lo = (uint32_t)peers[i] & ~(m ^ (uint32_t)bal);
                const uint32_t hi = (uint32_t)(peers[i] >> 32) & ~(m ^ (uint32_t)(bal >> 32));
                peers[i] = ((uint64_t)hi << 32) | lo;
            }
        }
        // The lowest lane of each digit adds the digit's keys of the group to
        // the wave's counter and gets back the count of earlier groups (the
        // LDS executes one wave's instructions in order, so the 8 adds need no
        // wait between them); its peers take that base from it.
        uint32_t base[kSortItems];
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            base[i] = 0u;
            if (popc_below(peers[i]) == 0u)
                base[i] = atomicAdd(&cnt[dig[i]], (uint32_t)__popcll(peers[i]));
            __builtin_amdgcn_wave_barrier();   // group order (free: the wave runs in lockstep)
        }
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            const int leader = (int)__builtin_ctzll(peers[i]);   // peers holds this lane
            rank[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(leader << 2, (int)base[i]) +
                      popc_below(peers[i]);
        }
        }
        __syncthreads();

        // digit-major exclusive offsets: keys with a smaller digit, plus keys
        // of the same digit in earlier waves
        uint32_t c[kSortWaves];
        uint32_t digit_total = 0;
        if (tid < radix) {
#pragma unroll
            for (int w = 0; w < kSortWaves; ++w) c[w] = sm.aux[(w << kMaxDigitBits) + tid];
#pragma unroll
            for (int w = 0; w < kSortWaves; ++w) {
                const uint32_t t = c[w];
                c[w] = digit_total;
                digit_total += t;
            }
        }
        uint64_t all;
        const uint32_t digit_base = (uint32_t)block_exclusive_scan(digit_total, sm.scan, &all);
        if (tid < radix) {
#pragma unroll
            for (int w = 0; w < kSortWaves; ++w) sm.aux[(w << kMaxDigitBits) + tid] = c[w] + digit_base;
        }
        __syncthreads();

#pragma unroll
        for (int i = 0; i < kSortItems; ++i) sm.keys[cur ^ 1][cnt[dig[i]] + rank[i]] = key[i];
        __syncthreads();
        cur ^= 1;
    }
    return cur;
}

// Optional outputs of the sort step.
struct SortOutputs {
    SortTables tables;            // per-slot tables, global (all null if not wanted)
    WsHeader *hdr;                // counts, global (or null)
    uint32_t *lc_run;             // LDS: run number of every long chunk (or null)
    uint32_t *lr;                 // LDS: per long run {main_grad row, first long chunk,
                                  //      chunk count, 0} (or null)
};

// Runs, chunks and long runs from the sorted keys. Blocked arrangement:
// thread t owns sorted slots [8t, 8t + 8). chunk_info goes to the other key
// buffer. Global outputs are written when their pointers are non-null.
__device__ __forceinline__ SortResult mark_runs(SortSmem &sm, int cur, int n, int pos_bits,
                                const SortOutputs &out) {
    const int tid = threadIdx.x;
    const uint32_t *sk = sm.keys[cur];
    uint32_t *info = sm.keys[cur ^ 1];
    const uint32_t pos_mask = (1u << pos_bits) - 1u;
    const int s0 = tid * kSortItems;
    uint32_t k[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) k[j] = sk[s0 + j];

    uint32_t prev_id = s0 > 0 ? (sk[s0 - 1] >> pos_bits) : 0u;
    uint32_t start_bits = 0, nstart = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int s = s0 + j;
        const uint32_t id = k[j] >> pos_bits;
        const bool st = s < n && (s == 0 || id != prev_id);
        start_bits |= (uint32_t)st << j;
        prev_id = id;
        nstart += st;
    }
    uint64_t num_runs;
    const uint32_t run_base = (uint32_t)block_exclusive_scan(nstart, sm.scan, &num_runs);

    // first slot of every run, plus n after the last: runs are [rs[r], rs[r+1])
    uint32_t *rs = sm.aux;
    int run_of[kSortItems];
    {
        uint32_t r = run_base;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            if ((start_bits >> j) & 1u) rs[r++] = (uint32_t)(s0 + j);
            run_of[j] = (int)r - 1;
        }
    }
    if (tid == 0) rs[num_runs] = (uint32_t)n;
    __syncthreads();

    // per slot: bit 0 = first slot of a chunk, bit 16 = first slot of a long
    // run, bit 32 = first slot of a chunk of a long run
    uint32_t first[kSortItems], end[kSortItems];
    uint64_t flag[kSortItems];
    uint64_t nflag = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int s = s0 + j;
        flag[j] = 0;
        first[j] = end[j] = 0;
        if (s < n) {
            first[j] = rs[run_of[j]];
            end[j] = rs[run_of[j] + 1];
            const uint32_t off = (uint32_t)s - first[j];
            const bool longer = end[j] - first[j] > (uint32_t)kNRows;
            const bool chunk_start = off % kNRows == 0;
            flag[j] = (uint64_t)chunk_start | ((uint64_t)(off == 0 && longer) << 16) |
                      ((uint64_t)(chunk_start && longer) << 32);
        }
        nflag += flag[j];
    }
    uint64_t totals;
    uint64_t idx = block_exclusive_scan(nflag, sm.scan, &totals);

#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int s = s0 + j;
        if (s < n) {
            const int c_idx = (int)(idx & 0xffff);
            const int lr_idx = (int)((idx >> 16) & 0xffff);
            const int lc_idx = (int)(idx >> 32);
            const bool longer = end[j] - first[j] > (uint32_t)kNRows;
            if (flag[j] & 1) {
                const int left = (int)end[j] - s;
                const int rows = left < kNRows ? left : kNRows;
                info[c_idx] = (uint32_t)s | ((uint32_t)(rows - 1) << 13) |
                              (longer ? ((uint32_t)lc_idx << 17) | kInfoLong : 0u);
                if (out.tables.chunk_first) out.tables.chunk_first[1 + c_idx] = s;
            }
            if (((flag[j] >> 16) & 1) && out.lr) {
                out.lr[4 * lr_idx + 0] = k[j] >> pos_bits;
                out.lr[4 * lr_idx + 1] = (uint32_t)lc_idx;
                out.lr[4 * lr_idx + 2] = (end[j] - first[j] + kNRows - 1) / kNRows;
                out.lr[4 * lr_idx + 3] = 0u;
            }
            // a long chunk belongs to the long run that starts at its slot, or
            // else to the last one started before it
            if ((flag[j] >> 32) & 1 && out.lc_run)
                out.lc_run[lc_idx] = (uint32_t)(((flag[j] >> 16) & 1) ? lr_idx : lr_idx - 1);
            if (((flag[j] >> 16) & 1) && out.tables.long_runs) out.tables.long_runs[1 + lr_idx] = s;
            if (out.tables.sorted_ids) {
                out.tables.sorted_ids[s] = (int32_t)(k[j] >> pos_bits);
                out.tables.positions[s] = (int32_t)(k[j] & pos_mask);
                out.tables.run_first[s] = (int32_t)first[j];
                out.tables.run_last[s] = (int32_t)end[j] - 1;
            }
        }
        idx += flag[j];
    }

    SortResult res;
    res.keys = sk;
    res.chunk_info = info;
    res.n_chunks = (int)(totals & 0xffff);
    res.n_long = (int)((totals >> 16) & 0xffff);
    res.n_long_chunks = (int)(totals >> 32);
    res.n_runs = (int)num_runs;
    if (tid == 0) {
        if (out.hdr) {
            out.hdr->invalid_ids = 0;
            out.hdr->num_chunks = res.n_chunks;
            out.hdr->num_long_runs = res.n_long;
            out.hdr->num_long_chunks = res.n_long_chunks;
            out.hdr->num_runs = res.n_runs;
        }
        if (out.tables.long_runs) out.tables.long_runs[0] = res.n_long;
        if (out.tables.chunk_first) out.tables.chunk_first[0] = res.n_chunks;
    }
    __syncthreads();   // chunk_info complete
    return res;
}

// Nothing to accumulate (some id out of range): zero counts, error count.
__device__ __forceinline__ void report_invalid(const SortOutputs &out, int bad) {
    if (threadIdx.x == 0) {
        if (out.hdr) {
            out.hdr->invalid_ids = bad;
            out.hdr->num_chunks = 0;
            out.hdr->num_long_runs = 0;
            out.hdr->num_long_chunks = 0;
            out.hdr->num_runs = 0;
        }
        if (out.tables.long_runs) out.tables.long_runs[0] = 0;
        if (out.tables.chunk_first) out.tables.chunk_first[0] = 0;
    }
}

}  // namespace ewg
