// Chunk sums and the ordered combine as device code shared by the kernels:
// the sum of one chunk's rows (at most 10, in position order, from +0 in
// fp32) over a range of column tiles, either finished into main_grad (a run
// of one chunk) or stored as a partial row (a chunk of a longer run), and the
// fold of a long run's partial rows in chunk order.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad": the
// introduction (fp32 chunk sums of ten consecutive rows or fewer, folded left
// to right from +0 with one conversion to grad's dtype, then an fp32 update
// of main_grad), _partial_sums_kernel and _long_run_sums_kernel.
#pragma once

#include "ewg_device.h"
#include "ewg_internal.h"

namespace ewg {

constexpr int kTilesPerUnit = 4;         // most column tiles of one chunk per unit / batch of loads
constexpr int kStageFloats = 32768;      // default combine staging: 128 KiB of chunk sums
constexpr int kMaxCombineCols = 8192;    // columns of one combine block (8 per thread)

// Columns of one combine task for a run of `chunks` chunk sums: the widest
// multiple of 64 columns that lets the whole run fit the staging buffer of
// STAGE floats, at least kMinCombineCols, at most kMaxCombineCols and at most
// hidden rounded up to 64. Deep runs get narrow tasks (many in parallel, one
// load round trip each, or two at the minimum width), shallow runs one task
// for all columns. (A minimum of 64 columns, 256-byte pieces of each partial
// row, took the many-token call on 32768 tokens ~1 µs longer.)
constexpr int kMinCombineCols = 128;
template <int STAGE = kStageFloats>
__device__ __forceinline__ int combine_width(int chunks, int hidden) {
    int w = STAGE / (chunks > 1 ? chunks : 1);
    w = w / 64 * 64;
    w = w < kMinCombineCols ? kMinCombineCols : (w > kMaxCombineCols ? kMaxCombineCols : w);
    const int h = (hidden + 63) / 64 * 64;
    return w < h ? w : h;
}

// NT full column tiles of one chunk of exactly R rows on the vector path,
// tiles starting at column tile_col (wave-uniform), k * 64 * VEC apart: the
// R x NT row loads (and the main_grad loads of a single-chunk run) are
// straight-line code, so they are all in flight before the first add.
// dest < 0: finish into main_grad row `row`; else store the fp32 chunk sums
// in row `dest` of the partial buffer.
template <typename G, typename M, int VEC, int R, int NT, int CP>
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
        // CP: device-coherent stores when another workgroup of this launch
        // reads them, plain ones when only a later kernel does
        const __amdgpu_buffer_rsrc_t prow =
            buffer_range(partial + (int64_t)dest * partial_stride, (uint32_t)(partial_stride * 4));
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int s = 0; s < S; ++s)
                store_coherent_floats<P, CP>(prow, (uint32_t)col[k][s] * 4u, &acc[k][s * P]);
    }
}

// The ragged last tile (starting at column tile_col) of one chunk, element by
// element, in the same lane layout.
template <typename G, typename M, int VEC, int CP>
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
                float *d = partial + (int64_t)dest * partial_stride + j;
                if constexpr (CP != 0) store_coherent(reinterpret_cast<uint32_t *>(d), __float_as_uint(acc));
                else *d = acc;
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
template <typename G, typename M, int VEC, int R, int CP>
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
        chunk_tiles<G, M, VEC, R, B, CP>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, t * 64 * VEC);
    for (; t < t_full; ++t)
        chunk_tiles<G, M, VEC, R, 1, CP>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, t * 64 * VEC);
    if (t < t_end)
        chunk_ragged_tile<G, M, VEC, CP>(pos, R, row, dest, grad, grad_stride, main_grad, mg_stride,
                                     partial, partial_stride, hidden, t * 64 * VEC);
}

// Dispatch on the row count of a chunk (1..10).
template <typename G, typename M, int VEC, int CP = kDeviceScope>
__device__ __forceinline__ void chunk_tiles_any(const int32_t *pos, int nrows, int row, int dest,
                                                const typename G::T *__restrict__ grad,
                                                int64_t grad_stride,
                                                typename M::T *__restrict__ main_grad,
                                                int64_t mg_stride, float *__restrict__ partial,
                                                int64_t partial_stride, int hidden, int t0,
                                                int t_end, int full_tiles) {
#define EWG_CHUNK(R)                                                                           \
    case R:                                                                                    \
        chunk_tile_range<G, M, VEC, R, CP>(pos, row, dest, grad, grad_stride, main_grad, mg_stride, \
                                       partial, partial_stride, hidden, t0, t_end, full_tiles); \
        break;
    switch (nrows) {
        EWG_CHUNK(1) EWG_CHUNK(2) EWG_CHUNK(3) EWG_CHUNK(4) EWG_CHUNK(5)
        EWG_CHUNK(6) EWG_CHUNK(7) EWG_CHUNK(8) EWG_CHUNK(9) EWG_CHUNK(10)
        default: break;
    }
#undef EWG_CHUNK
}


// One block of columns [col0, col0 + wdt) of a long run whose `chunks`
// partial rows start at row `first` of the partial buffer, by all 1024
// threads: the partial rows are staged in LDS (`stage`, STAGE floats),
// as many at a time as fit, and every column's running total adds them in
// chunk order starting from +0; the total is then rounded once and added to
// main_grad row `row`. wdt is combine_width<STAGE>(chunks, hidden).
template <typename G, typename M, int STAGE = kStageFloats, int CP = kDeviceScope, int FOLD = 8>
__device__ __forceinline__ void combine_block(float *stage, uint32_t row, uint32_t first,
                                              uint32_t chunks, int64_t col0, int wdt,
                                              const float *__restrict__ partial,
                                              int64_t partial_stride,
                                              typename M::T *__restrict__ main_grad,
                                              int64_t mg_stride, int hidden) {
    using MT = typename M::T;
    const int tid = threadIdx.x;
    const int wc = (int)(hidden - col0 < wdt ? hidden - col0 : wdt);
    MT *mrow = main_grad + (int64_t)row * mg_stride + col0;
    constexpr int kCols = kMaxCombineCols / kSortThreads;   // columns per thread
    MT old[kCols];
    float total[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const int j = tid + i * kSortThreads;
        total[i] = 0.0f;
        if (j < wc) old[i] = mrow[j];
    }
    const int quads = (wc + 3) / 4;           // 16-byte pieces of one chunk row
    // chunks per stage: the buffer, and a byte range below 2 GiB
    int per_stage = STAGE / wdt;
    const int64_t by_range = ((int64_t)1 << 29) / partial_stride;
    if (per_stage > by_range) per_stage = (int)by_range;
    for (int k0 = 0; k0 < (int)chunks; k0 += per_stage) {
        const int ks = (int)chunks - k0 < per_stage ? (int)chunks - k0 : per_stage;
        const float *base = partial + (int64_t)(first + k0) * partial_stride + col0;
        const uint32_t range = (uint32_t)(((int64_t)(ks - 1) * partial_stride + 4 * quads) * 4);
        const __amdgpu_buffer_rsrc_t rs = buffer_range(base, range);
        const int pieces = ks * quads;
        constexpr int kLoads = STAGE / 4 / kSortThreads;
        u32x4 v[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {   // all loads in flight; past the range they read 0
            const int p = tid + i * kSortThreads;
            const int kk = p / quads, q = p - kk * quads;
            const uint32_t off = p < pieces ? (uint32_t)(((int64_t)kk * partial_stride + 4 * q) * 4)
                                            : 0xfffffff0u;
            v[i] = load_coherent16<CP>(rs, off);
        }
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int p = tid + i * kSortThreads;
            if (p < pieces) {
                const int kk = p / quads, q = p - kk * quads;
                float *d = &stage[kk * wdt + 4 * q];
                d[0] = __uint_as_float(v[i].x);
                d[1] = __uint_as_float(v[i].y);
                d[2] = __uint_as_float(v[i].z);
                d[3] = __uint_as_float(v[i].w);
            }
        }
        __syncthreads();
        // in chunk order, one running total per column; waves without
        // a column of this slot skip it
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
            const int wave_j0 = (tid & ~63) + i * kSortThreads;
            if (wave_j0 < wc) {
                const int j = tid + i * kSortThreads;
                const float *col = &stage[j < wc ? j : wave_j0];
                float acc = total[i];
                // the adds stay in chunk order; the LDS reads of a group
                // of FOLD are all issued before the first add
                int kk = 0;
                for (; kk + FOLD <= ks; kk += FOLD) {
                    float v[FOLD];
#pragma unroll
                    for (int q = 0; q < FOLD; ++q) v[q] = col[(kk + q) * wdt];
#pragma unroll
                    for (int q = 0; q < FOLD; ++q) acc = acc + v[q];
                }
                for (; kk < ks; ++kk) acc = acc + col[kk * wdt];
                total[i] = acc;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const int j = tid + i * kSortThreads;
        if (j < wc) mrow[j] = finish<G, M>(total[i], old[i]);
    }
}

}  // namespace ewg
