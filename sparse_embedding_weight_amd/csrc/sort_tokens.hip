// Sort step: packed (id << pos_bits | position) keys sorted in LDS by one
// workgroup, runs of equal ids marked, and the work lists for the two
// accumulation kernels written to the workspace.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad":
// _sort_tokens_kernel (sort the (token, position) pairs, give every sorted
// slot the first and last slot of its run, list the runs longer than NROWS),
// _position_bits, and the introduction ("sorts the token ids together with
// their positions", rows summed "in position order").
//
// The keys enter in position order and the radix sort is stable, so sorting
// on the id bits alone yields (id, position) order; the position bits need no
// pass. Ids have at most 19 bits (31 - 12), hence at most two passes of at
// most 10 bits.
//
// Ranking inside a pass is done per wavefront with ballots: for every key the
// lanes holding the same digit are found with one ballot per digit bit, its
// rank among them is a masked popcount, and a per-wave LDS counter per digit
// carries the count across the wave's 8 key groups. A digit-major scan of the
// 16 x 2^bits counters turns them into scatter offsets.
#include "ewg_device.h"
#include "ewg_internal.h"

namespace ewg {
namespace {

constexpr int kWaveSlots = kSortItems * 64;   // 512 consecutive slots per wave

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
    uint32_t lo = __shfl_up((uint32_t)v, d, 64);
    uint32_t hi = __shfl_up((uint32_t)(v >> 32), d, 64);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint64_t o = shfl_up_u64(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive prefix sum over the 1024 threads in thread order; *total gets the
// sum of all. Every thread must call it. s_tmp holds kSortWaves + 1 values.
__device__ uint64_t block_exclusive_scan(uint64_t v, uint64_t *s_tmp, uint64_t *total) {
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

template <typename IdT>
__global__ __launch_bounds__(kSortThreads) void sort_tokens_kernel(
    const IdT *__restrict__ ids, int n, int num_embeddings, int pos_bits, int id_bits,
    WsHeader *__restrict__ hdr, ChunkDesc *__restrict__ chunks,
    LongRunDesc *__restrict__ long_runs, SortTables tables) {
    __shared__ uint32_t s_keys[2][kMaxTokens];
    __shared__ uint32_t s_counts[kSortWaves << kMaxDigitBits];
    __shared__ uint64_t s_scan[kSortWaves + 1];
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_bad = 0;
    __syncthreads();

    // Keys in position order; wave w holds slots [w*512, w*512 + 512) as 8
    // groups of 64. Slots past n hold 0xffffffff, which every pass ranks last.
    int bad = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int s = wave * kWaveSlots + i * 64 + lane;
        uint32_t key = 0xffffffffu;
        if (s < n) {
            const int64_t id = (int64_t)ids[s];
            if (id < 0 || id >= num_embeddings) {
                ++bad;
                key = 0;
            } else {
                key = ((uint32_t)id << pos_bits) | (uint32_t)s;
            }
        }
        s_keys[0][s] = key;
    }
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    if (s_bad) {   // uniform: nothing is accumulated
        if (tid == 0) {
            hdr->invalid_ids = s_bad;
            hdr->num_chunks = 0;
            hdr->num_long_runs = 0;
            hdr->num_long_chunks = 0;
            hdr->num_runs = 0;
            if (tables.long_runs) tables.long_runs[0] = 0;
            if (tables.chunk_first) tables.chunk_first[0] = 0;
        }
        return;
    }

    // ---- stable LSD radix passes over the id bits --------------------------
    int cur = 0;
    const int npass = (id_bits + kMaxDigitBits - 1) / kMaxDigitBits;
    int done = 0;
    for (int p = 0; p < npass; ++p) {
        const int bits = (id_bits - done + (npass - p) - 1) / (npass - p);
        const int shift = pos_bits + done;
        done += bits;
        const uint32_t mask = (1u << bits) - 1u;
        const int radix = 1 << bits;
        uint32_t *cnt = s_counts + (wave << kMaxDigitBits);

        for (int d = lane; d < radix; d += 64) cnt[d] = 0;
        __builtin_amdgcn_wave_barrier();

        uint32_t key[kSortItems], rank[kSortItems];
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            key[i] = s_keys[cur][wave * kWaveSlots + i * 64 + lane];
            const uint32_t d = (key[i] >> shift) & mask;
            uint64_t peers = ~0ull;
            for (int b = 0; b < bits; ++b) {
                const bool set = (d >> b) & 1u;
                const uint64_t bal = __ballot(set);
                peers &= set ? bal : ~bal;
            }
            const uint32_t below = popc_below(peers);
            const uint32_t base = cnt[d];
            rank[i] = base + below;
            __builtin_amdgcn_wave_barrier();
            if (below == 0) cnt[d] = base + (uint32_t)__popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
        __syncthreads();

        // digit-major exclusive offsets: for digit d and wave w, the number of
        // keys with a smaller digit plus those of digit d in waves before w
        uint32_t digit_total = 0;
        if (tid < radix) {
            uint32_t run = 0;
            for (int w = 0; w < kSortWaves; ++w) {
                const uint32_t c = s_counts[(w << kMaxDigitBits) + tid];
                s_counts[(w << kMaxDigitBits) + tid] = run;
                run += c;
            }
            digit_total = run;
        }
        uint64_t all;
        const uint32_t digit_base = (uint32_t)block_exclusive_scan(digit_total, s_scan, &all);
        if (tid < radix) {
            for (int w = 0; w < kSortWaves; ++w) s_counts[(w << kMaxDigitBits) + tid] += digit_base;
        }
        __syncthreads();

#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            const uint32_t d = (key[i] >> shift) & mask;
            s_keys[cur ^ 1][cnt[d] + rank[i]] = key[i];
        }
        __syncthreads();
        cur ^= 1;
    }

    // ---- runs, chunks, long runs ------------------------------------------
    // Blocked arrangement: thread t owns sorted slots [8t, 8t + 8).
    const uint32_t *sk = s_keys[cur];
    const uint32_t pos_mask = (1u << pos_bits) - 1u;
    const int s0 = tid * kSortItems;
    uint32_t k[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) k[j] = sk[s0 + j];

    uint32_t prev_id = s0 > 0 ? (sk[s0 - 1] >> pos_bits) : 0u;
    bool is_start[kSortItems];
    uint32_t nstart = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int s = s0 + j;
        const uint32_t id = k[j] >> pos_bits;
        is_start[j] = s < n && (s == 0 || id != prev_id);
        prev_id = id;
        nstart += is_start[j];
    }
    uint64_t num_runs;
    const uint32_t run_base = (uint32_t)block_exclusive_scan(nstart, s_scan, &num_runs);

    // first slot of every run, plus n after the last: runs are [rs[r], rs[r+1])
    uint32_t *rs = s_counts;
    int run_of[kSortItems];
    {
        uint32_t r = run_base;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            if (is_start[j]) rs[r++] = (uint32_t)(s0 + j);
            run_of[j] = (int)r - 1;
        }
    }
    if (tid == 0) rs[num_runs] = (uint32_t)n;
    __syncthreads();

    // per slot: bit 0 = first slot of a chunk, bit 16 = first slot of a long
    // run, bit 32 = first slot of a chunk of a long run
    uint64_t flag[kSortItems];
    uint32_t first[kSortItems], last_excl[kSortItems];
    uint64_t nflag = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int s = s0 + j;
        flag[j] = 0;
        if (s < n) {
            first[j] = rs[run_of[j]];
            last_excl[j] = rs[run_of[j] + 1];
            const uint32_t off = (uint32_t)s - first[j];
            const bool longer = last_excl[j] - first[j] > (uint32_t)kNRows;
            const bool chunk_start = off % kNRows == 0;
            flag[j] = (uint64_t)chunk_start | ((uint64_t)(off == 0 && longer) << 16) |
                      ((uint64_t)(chunk_start && longer) << 32);
        }
        nflag += flag[j];
    }
    uint64_t totals;
    uint64_t idx = block_exclusive_scan(nflag, s_scan, &totals);
    const int n_chunks = (int)(totals & 0xffff);
    const int n_long = (int)((totals >> 16) & 0xffff);
    const int n_long_chunks = (int)(totals >> 32);

#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const int s = s0 + j;
        if (s >= n) break;
        const uint32_t id = k[j] >> pos_bits;
        const int c_idx = (int)(idx & 0xffff);
        const int lr_idx = (int)((idx >> 16) & 0xffff);
        const int lc_idx = (int)(idx >> 32);
        const bool longer = last_excl[j] - first[j] > (uint32_t)kNRows;
        if (flag[j] & 1) {
            ChunkDesc dsc;
            dsc.row = (int32_t)id;
            dsc.dest = longer ? lc_idx : -1;
            const int left = (int)last_excl[j] - s;
            dsc.nrows = left < kNRows ? left : kNRows;
            dsc.unused = 0;
#pragma unroll
            for (int r = 0; r < 12; ++r)
                dsc.pos[r] = r < dsc.nrows ? (int32_t)(sk[s + r] & pos_mask) : 0;
            chunks[c_idx] = dsc;
            if (tables.chunk_first) tables.chunk_first[1 + c_idx] = s;
        }
        if ((flag[j] >> 16) & 1) {
            LongRunDesc lr;
            lr.row = (int32_t)id;
            lr.first_partial = lc_idx;
            lr.nchunks = (int32_t)((last_excl[j] - first[j] + kNRows - 1) / kNRows);
            lr.unused = 0;
            long_runs[lr_idx] = lr;
            if (tables.long_runs) tables.long_runs[1 + lr_idx] = s;
        }
        if (tables.sorted_ids) {
            tables.sorted_ids[s] = (int32_t)id;
            tables.positions[s] = (int32_t)(k[j] & pos_mask);
            tables.run_first[s] = (int32_t)first[j];
            tables.run_last[s] = (int32_t)last_excl[j] - 1;
        }
        idx += flag[j];
    }

    if (tid == 0) {
        hdr->invalid_ids = 0;
        hdr->num_chunks = n_chunks;
        hdr->num_long_runs = n_long;
        hdr->num_long_chunks = n_long_chunks;
        hdr->num_runs = (int32_t)num_runs;
        if (tables.long_runs) tables.long_runs[0] = n_long;
        if (tables.chunk_first) tables.chunk_first[0] = n_chunks;
    }
}

}  // namespace

hipError_t launch_sort_tokens(const void *ids, bool ids_int64, int n, int num_embeddings,
                              int pos_bits, int id_bits, void *workspace, const WsLayout &l,
                              const SortTables &tables, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws);
    ChunkDesc *chunks = reinterpret_cast<ChunkDesc *>(ws + l.chunks);
    LongRunDesc *long_runs = reinterpret_cast<LongRunDesc *>(ws + l.long_runs);
    if (ids_int64)
        sort_tokens_kernel<int64_t><<<1, kSortThreads, 0, stream>>>(
            static_cast<const int64_t *>(ids), n, num_embeddings, pos_bits, id_bits, hdr,
            chunks, long_runs, tables);
    else
        sort_tokens_kernel<int32_t><<<1, kSortThreads, 0, stream>>>(
            static_cast<const int32_t *>(ids), n, num_embeddings, pos_bits, id_bits, hdr,
            chunks, long_runs, tables);
    return hipGetLastError();
}

}  // namespace ewg
