// Partial-sum pass: every chunk (up to 10 grad rows of one id, in position
// order) is summed in fp32 from +0, column by column. A run that is a single
// chunk is finished here (one rounding to grad's dtype, fp32 add into
// main_grad, rounding to main_grad's dtype); the chunk sums of longer runs go
// to the partial buffer for the ordered combine.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad":
// _partial_sums_kernel ("a run of at most NROWS rows is finished here") and
// the introduction's two bullets.
//
// Work unit = (chunk, column tile); one wavefront per unit, grid-stride over
// units, so one launch of a fixed grid covers any chunk count (read on the
// device). A tile is 64 lanes x VEC columns; with 16-byte rows a lane moves
// 16 bytes of grad per row (8 bf16 or 4 fp32), so a wave reads 1 KiB of each
// grad row per load instruction. All rows of a chunk are loaded before the
// first add, giving up to 10 independent 16-byte loads per lane in flight.
#include "ewg_device.h"
#include "ewg_internal.h"

namespace ewg {
namespace {

constexpr int kThreads = 256;

// One (chunk, tile) on the 16-byte path, for a chunk of exactly R rows: the
// R row loads (and the main_grad load of a single-chunk run) are straight-line
// code, so they are all in flight before the first add.
template <typename G, typename M, int VEC, int R>
__device__ __forceinline__ void chunk_tile(const int32_t (&pos)[kNRows], int row, int dest,
                                           const typename G::T *__restrict__ grad,
                                           int64_t grad_stride, typename M::T *__restrict__ main_grad,
                                           int64_t mg_stride, float *__restrict__ partial,
                                           int64_t partial_stride, int col) {
    using GT = typename G::T;
    using MT = typename M::T;
    GT raw[R][VEC];
#pragma unroll
    for (int r = 0; r < R; ++r)
        load_vec<GT, VEC>(grad + (int64_t)pos[r] * grad_stride + col, raw[r]);
    MT *mrow = main_grad + (int64_t)row * mg_stride + col;
    MT old[VEC];
    if (dest < 0) load_vec<MT, VEC>(mrow, old);

    float acc[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] = acc[k] + G::widen(raw[r][k]);

    if (dest < 0) {
        MT out[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) out[k] = finish<G, M>(0.0f + acc[k], old[k]);
        store_vec<MT, VEC>(mrow, out);
    } else {
        store_vec<float, VEC>(partial + (int64_t)dest * partial_stride + col, acc);
    }
}

template <typename G, typename M, int VEC>
__global__ __launch_bounds__(kThreads) void partial_sums_kernel(
    const WsHeader *__restrict__ hdr, const ChunkDesc *__restrict__ chunks,
    const typename G::T *__restrict__ grad, int64_t grad_stride,
    typename M::T *__restrict__ main_grad, int64_t mg_stride, float *__restrict__ partial,
    int64_t partial_stride, int hidden, int tiles) {
    using MT = typename M::T;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * kThreads + threadIdx.x) >> 6));
    const int nwaves = (int)((gridDim.x * kThreads) >> 6);
    const uint32_t units = (uint32_t)hdr->num_chunks * (uint32_t)tiles;

    for (uint32_t u = (uint32_t)wave; u < units; u += (uint32_t)nwaves) {
        const uint32_t c = u / (uint32_t)tiles;
        const int t = (int)(u - c * (uint32_t)tiles);
        const ChunkDesc d = chunks[c];   // wave-uniform: scalar loads
        int32_t pos[kNRows];
#pragma unroll
        for (int r = 0; r < kNRows; ++r) pos[r] = d.pos[r];
        const int row = d.row, dest = d.dest, nrows = d.nrows;
        const int col = t * (64 * VEC) + lane * VEC;
        if (col >= hidden) continue;

        if (col + VEC <= hidden) {
#define EWG_CHUNK(R)                                                                       \
    case R:                                                                                \
        chunk_tile<G, M, VEC, R>(pos, row, dest, grad, grad_stride, main_grad, mg_stride,  \
                                 partial, partial_stride, col);                            \
        break;
            switch (nrows) {
                EWG_CHUNK(1) EWG_CHUNK(2) EWG_CHUNK(3) EWG_CHUNK(4) EWG_CHUNK(5)
                EWG_CHUNK(6) EWG_CHUNK(7) EWG_CHUNK(8) EWG_CHUNK(9) EWG_CHUNK(10)
                default: break;
            }
#undef EWG_CHUNK
        } else {
            // ragged last tile: element by element
            for (int j = col; j < hidden; ++j) {
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

template <typename G, typename M, int VEC>
hipError_t launch(const void *grad, int64_t grad_stride, void *main_grad, int64_t mg_stride,
                  int hidden, void *workspace, const WsLayout &l, int max_chunks, int num_cus,
                  hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    const int tiles = (hidden + 64 * VEC - 1) / (64 * VEC);
    const int64_t max_units = (int64_t)max_chunks * tiles;
    int64_t blocks = (max_units + (kThreads / 64) - 1) / (kThreads / 64);
    const int64_t cap = (int64_t)num_cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    partial_sums_kernel<G, M, VEC><<<(unsigned)blocks, kThreads, 0, stream>>>(
        reinterpret_cast<const WsHeader *>(ws), reinterpret_cast<const ChunkDesc *>(ws + l.chunks),
        static_cast<const typename G::T *>(grad), grad_stride,
        static_cast<typename M::T *>(main_grad), mg_stride,
        reinterpret_cast<float *>(ws + l.partial), l.partial_stride, hidden, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_sums(bool grad_bf16, bool mg_bf16, bool vec, const void *grad,
                               int64_t grad_stride, void *main_grad, int64_t mg_stride,
                               int hidden, void *workspace, const WsLayout &l, int max_chunks,
                               int num_cus, hipStream_t stream) {
#define EWG_PS(G, M, V) \
    launch<G, M, V>(grad, grad_stride, main_grad, mg_stride, hidden, workspace, l, max_chunks, num_cus, stream)
    if (grad_bf16) {
        if (mg_bf16) return vec ? EWG_PS(BF16, BF16, 8) : EWG_PS(BF16, BF16, 1);
        return vec ? EWG_PS(BF16, F32, 8) : EWG_PS(BF16, F32, 1);
    }
    if (mg_bf16) return vec ? EWG_PS(F32, BF16, 4) : EWG_PS(F32, BF16, 1);
    return vec ? EWG_PS(F32, F32, 4) : EWG_PS(F32, F32, 1);
#undef EWG_PS
}

}  // namespace ewg
