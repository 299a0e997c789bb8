// Fused sort + partial-sum kernel, one 1024-thread workgroup per compute unit.
//
// Workgroup 0 (dispatched first) sorts the packed (id, position) keys in LDS
// (sort_lds.h), marks runs and chunks, publishes the sorted keys, the chunk
// table and the per-chunk cost prefix to the workspace and sets the ready
// flag to this call's epoch (a nonzero number the host draws per call). Meanwhile every other workgroup pulls its share of the grad rows and
// of the touched main_grad rows towards the Infinity Cache, then waits for
// the flag and copies the tables into its own LDS. Then every wave takes a
// contiguous range of (chunk, column tile) units of about equal byte cost:
// every chunk (up to 10 grad rows of one id, in position order) is summed in
// fp32 from +0; a run that is a single chunk is finished here (one rounding to
// grad's dtype, fp32 add into main_grad, rounding to main_grad's dtype); the
// chunk sums of longer runs go to the partial buffer for the ordered combine
// (long_run_sums.hip), which also sets the flag back to 0.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad":
// _partial_sums_kernel ("a run of at most NROWS rows is finished here") and
// the introduction's two bullets.
//
// A column tile is 64 lanes x VEC columns; with 16-byte rows a lane moves 16
// bytes of grad per row (8 bf16 or 4 fp32), so a wave reads 1 KiB of each grad
// row per load instruction, and the rows of up to kTilesPerUnit tiles of a
// chunk are loaded before the first add.
#include "ewg_device.h"
#include "ewg_internal.h"
#include "sort_lds.h"

namespace ewg {
namespace {

constexpr int kTilesPerUnit = 4;         // most column tiles of one chunk per batch of loads
constexpr int kPrefetchBatch = 16;       // 1-byte loads (one per 64-byte line) per lane per batch
constexpr int64_t kWaitLimit = 1 << 22;  // polls of the ready flag before giving up (seconds)

// NT full column tiles of one chunk of exactly R rows on the 16-byte path: the
// R x NT row loads (and the main_grad loads of a single-chunk run) are
// straight-line code, so they are all in flight before the first add. Tile k
// covers columns col + k * 64 * VEC.
template <typename G, typename M, int VEC, int R, int NT>
__device__ __forceinline__ void chunk_tiles(const int32_t *pos, int row, int dest,
                                            const typename G::T *__restrict__ grad,
                                            int64_t grad_stride, typename M::T *__restrict__ main_grad,
                                            int64_t mg_stride, float *__restrict__ partial,
                                            int64_t partial_stride, int col) {
    using GT = typename G::T;
    using MT = typename M::T;
    GT raw[R][NT][VEC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < NT; ++k)
            load_vec<GT, VEC>(grad + (int64_t)pos[r] * grad_stride + col + k * 64 * VEC, raw[r][k]);
    MT *mrow = main_grad + (int64_t)row * mg_stride + col;
    MT old[NT][VEC];
    if (dest < 0) {
#pragma unroll
        for (int k = 0; k < NT; ++k) load_vec<MT, VEC>(mrow + k * 64 * VEC, old[k]);
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
            store_vec<MT, VEC>(mrow + k * 64 * VEC, out);
        }
    } else {
        float *prow = partial + (int64_t)dest * partial_stride + col;
#pragma unroll
        for (int k = 0; k < NT; ++k) store_vec<float, VEC>(prow + k * 64 * VEC, acc[k]);
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

// The full tiles [t0, t0 + nt) of one chunk of R rows, in batches of loads.
template <typename G, typename M, int VEC, int R>
__device__ __forceinline__ void chunk_full_tiles(const int32_t *pos, int row, int dest,
                                                 const typename G::T *__restrict__ grad,
                                                 int64_t grad_stride,
                                                 typename M::T *__restrict__ main_grad,
                                                 int64_t mg_stride, float *__restrict__ partial,
                                                 int64_t partial_stride, int col0, int nt) {
    constexpr int B = tiles_per_batch<G, M, VEC, R>();
    int k = 0;
    for (; k + B <= nt; k += B)
        chunk_tiles<G, M, VEC, R, B>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, col0 + k * 64 * VEC);
    for (; k < nt; ++k)
        chunk_tiles<G, M, VEC, R, 1>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, col0 + k * 64 * VEC);
}

// Pull the grad rows at positions [lo, hi) and the main_grad rows of their
// ids towards the caches: wave w takes rows lo + w, lo + w + 16, ...; each lane
// loads one byte of every 64th 64-byte line, 16 lines per batch, and waits for
// the batch before the next. Stops as soon as the ready flag holds this call's
// epoch. Ids outside
// [0, num_embeddings) are skipped.
template <typename IdT, typename G, typename M>
__device__ __forceinline__ void follower_prefetch(const IdT *__restrict__ ids, int num_embeddings,
                                                  const typename G::T *grad, int64_t grad_stride,
                                                  const typename M::T *mg, int64_t mg_stride,
                                                  int hidden, int lo, int hi,
                                                  const uint32_t *ready, uint32_t epoch) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t g_bytes = (int64_t)hidden * (int64_t)sizeof(typename G::T);
    const int64_t m_bytes = (int64_t)hidden * (int64_t)sizeof(typename M::T);
    const int g_lines = (int)((g_bytes + 63) / 64);
    const int lines = g_lines + (int)((m_bytes + 63) / 64);
    for (int r = lo + wave; r < hi; r += kSortWaves) {
        const uint8_t *gp = reinterpret_cast<const uint8_t *>(grad + (int64_t)r * grad_stride);
        const int64_t id = (int64_t)ids[r];
        const bool id_ok = id >= 0 && id < num_embeddings;
        const uint8_t *mp = reinterpret_cast<const uint8_t *>(mg + (id_ok ? id : 0) * mg_stride);
        for (int l0 = 0; l0 < lines; l0 += 64 * kPrefetchBatch) {
            uint32_t v[kPrefetchBatch];
#pragma unroll
            for (int k = 0; k < kPrefetchBatch; ++k) {
                const int line = l0 + k * 64 + lane;
                const uint8_t *p;
                if (line < g_lines) {
                    p = gp + (int64_t)line * 64;
                } else {
                    const int64_t off = (int64_t)(line - g_lines) * 64;
                    p = mp + (off < m_bytes ? off : m_bytes - 1);
                }
                v[k] = *(line < lines ? p : gp);
            }
#pragma unroll
            for (int k = 0; k < kPrefetchBatch; ++k) asm volatile("" ::"v"(v[k]));
            if (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) return;
        }
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
    using MT = typename M::T;
    __shared__ SortSmem sm;
    __shared__ int s_flag;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const uint32_t *keys, *info, *cost;
    int n_chunks;
    uint32_t cost_total;
    if (blockIdx.x == 0) {
        // ---- the sorting workgroup ----
        const SortOutputs out = {{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr},
                                 long_runs, hdr};
        const int bad = load_keys<IdT>(sm, ids, n, num_embeddings, pos_bits);
        if (bad) {
            report_invalid(out, bad);
            n_chunks = 0;
            cost_total = 0;
            keys = info = cost = nullptr;
        } else {
            const int cur = radix_sort_ids(sm, pos_bits, id_bits);
            const SortResult res = mark_runs(sm, cur, n, pos_bits, out);
            // per-tile cost in 16-byte lane loads: grad rows, main_grad read +
            // write of a single-chunk run, or the store of a partial sum
            const uint32_t row_cost = (uint32_t)(VEC * sizeof(typename G::T) + 15) / 16;
            const uint32_t short_cost = 2u * (uint32_t)(VEC * sizeof(MT) + 15) / 16;
            const uint32_t long_cost = (uint32_t)(VEC * 4 + 15) / 16;
            cost_total = chunk_cost_prefix(sm, res, sm.aux, row_cost, short_cost, long_cost);
            keys = res.keys;
            info = res.chunk_info;
            cost = sm.aux;
            n_chunks = res.n_chunks;
            for (int i = tid; i < n; i += kSortThreads) tab_keys[i] = keys[i];
            for (int i = tid; i < n_chunks; i += kSortThreads) tab_info[i] = info[i];
            for (int i = tid; i <= n_chunks; i += kSortThreads) tab_cost[i] = cost[i];
        }
        if (tid == 0) hdr->cost_total = cost_total;
        // publish: every thread's stores are made visible, then the flag goes up
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&hdr->ready, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // ---- every other workgroup: prefetch, wait, copy the tables ----
        const int followers = (int)gridDim.x - 1;
        const int b = (int)blockIdx.x - 1;
        const int lo = (int)((int64_t)n * b / followers);
        const int hi = (int)((int64_t)n * (b + 1) / followers);
        follower_prefetch<IdT, G, M>(ids, num_embeddings, grad, grad_stride, main_grad, mg_stride,
                                     hidden, lo, hi, &hdr->ready, epoch);
        if (tid == 0) {
            int ok = 1;
            int64_t spins = 0;
            while (__hip_atomic_load(&hdr->ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
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
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        n_chunks = __hip_atomic_load(&hdr->num_chunks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        cost_total = __hip_atomic_load(&hdr->cost_total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = tid; i < n; i += kSortThreads) sm.keys[0][i] = tab_keys[i];
        for (int i = tid; i < n_chunks; i += kSortThreads) sm.keys[1][i] = tab_info[i];
        for (int i = tid; i <= n_chunks; i += kSortThreads) sm.aux[i] = tab_cost[i];
        __syncthreads();
        keys = sm.keys[0];
        info = sm.keys[1];
        cost = sm.aux;
    }
    if (n_chunks == 0) return;

    // ---- this wave's units: starts in [x0, x1) of the cost line ----
    const uint32_t pos_mask = (1u << pos_bits) - 1u;
    const uint64_t nw = (uint64_t)gridDim.x * kSortWaves;
    const uint64_t gw = (uint64_t)blockIdx.x * kSortWaves + (uint64_t)__builtin_amdgcn_readfirstlane(wave);
    const uint64_t total = (uint64_t)cost_total * (uint64_t)tiles;
    int c, t, ce, te;
    first_unit(cost, n_chunks, tiles, total * gw / nw, c, t);
    if (gw + 1 == nw) {
        ce = n_chunks;
        te = 0;
    } else {
        first_unit(cost, n_chunks, tiles, total * (gw + 1) / nw, ce, te);
    }
    const int full_tiles = hidden / (64 * VEC);
    for (; c < ce || (c == ce && t < te); ++c, t = 0) {
        const uint32_t x = __builtin_amdgcn_readfirstlane(info[c]);
        const int f = info_first(x), nrows = info_rows(x);
        const int dest = (x & kInfoLong) ? info_long_chunk(x) : -1;
        const int row = (int)(__builtin_amdgcn_readfirstlane(keys[f]) >> pos_bits);
        int32_t pos[kNRows];
#pragma unroll
        for (int r = 0; r < kNRows; ++r)
            pos[r] = r < nrows ? (int32_t)(__builtin_amdgcn_readfirstlane(keys[f + r]) & pos_mask) : 0;
        const int t_stop = c == ce ? te : tiles;
        const int t_full = t_stop < full_tiles ? t_stop : full_tiles;   // [t, t_full) are full tiles
        if (t_full > t) {
            const int col0 = t * (64 * VEC) + lane * VEC;
#define EWG_CHUNK(R)                                                                          \
    case R:                                                                                   \
        chunk_full_tiles<G, M, VEC, R>(pos, row, dest, grad, grad_stride, main_grad, mg_stride, \
                                       partial, partial_stride, col0, t_full - t);            \
        break;
            switch (nrows) {
                EWG_CHUNK(1) EWG_CHUNK(2) EWG_CHUNK(3) EWG_CHUNK(4) EWG_CHUNK(5)
                EWG_CHUNK(6) EWG_CHUNK(7) EWG_CHUNK(8) EWG_CHUNK(9) EWG_CHUNK(10)
                default: break;
            }
#undef EWG_CHUNK
        }
        if (t_stop > t_full && t_stop > t) {
            // the ragged last tile: element by element
            const int tr = t_full > t ? t_full : t;
            for (int j = tr * (64 * VEC) + lane * VEC, e = 0; e < VEC; ++e, ++j) {
                if (j >= hidden) break;
                float acc = 0.0f;
                for (int r = 0; r < nrows; ++r)
                    acc = acc + G::widen(grad[(int64_t)pos[r] * grad_stride + j]);
                if (dest < 0) {
                    MT *m = main_grad + (int64_t)row * mg_stride + j;
                    *m = finish<G, M>(0.0f + acc, *m);
                } else {
                    partial[(int64_t)dest * partial_stride + j] = acc;
                }
            }
        }
    }
}

template <typename IdT, typename G, typename M, int VEC>
hipError_t launch(const void *ids, int n, int num_embeddings, int pos_bits, int id_bits,
                  const void *grad, int64_t grad_stride, void *main_grad, int64_t mg_stride,
                  int hidden, void *workspace, const WsLayout &l, int num_cus, uint32_t epoch,
                  hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    const int tiles = (hidden + 64 * VEC - 1) / (64 * VEC);
    accumulate_kernel<IdT, G, M, VEC><<<num_cus, kSortThreads, 0, stream>>>(
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
