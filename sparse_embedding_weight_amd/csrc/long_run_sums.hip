// Ordered combine of the runs longer than 10 rows: the chunk sums of a run
// are added in chunk order to a running fp32 total that starts at +0, which
// is then rounded once to grad's dtype, added to the main_grad row in fp32
// and rounded to main_grad's dtype. Only the rows of these runs are read and
// written.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad":
// _long_run_sums_kernel ("add the partial sums of a run longer than NROWS rows
// in order, round, add to main_grad") and the introduction ("adds the
// partial sums in order starting from 0").
//
// Work unit = (long run, column tile of 64 lanes x VEC fp32 columns); one
// wavefront per unit, grid-stride. The adds of one column are a dependent
// chain in chunk order, so the loads of 8 chunk sums are issued before they
// are added. Block 0 also clears the fused kernel's ready flag: this kernel
// ends every call.
#include "ewg_device.h"
#include "ewg_internal.h"

namespace ewg {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;

template <typename G, typename M, int VEC>
__global__ __launch_bounds__(kThreads) void long_run_sums_kernel(
    WsHeader *__restrict__ hdr, const LongRunDesc *__restrict__ runs,
    const float *__restrict__ partial, int64_t partial_stride,
    typename M::T *__restrict__ main_grad, int64_t mg_stride, int hidden, int tiles) {
    using MT = typename M::T;
    // the call is over for the fused kernel: clear its ready flag for the next call
    if (blockIdx.x == 0 && threadIdx.x == 0) hdr->ready = 0u;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * kThreads + threadIdx.x) >> 6));
    const int nwaves = (int)((gridDim.x * kThreads) >> 6);
    const uint32_t units = (uint32_t)hdr->num_long_runs * (uint32_t)tiles;

    for (uint32_t u = (uint32_t)wave; u < units; u += (uint32_t)nwaves) {
        const uint32_t r = u / (uint32_t)tiles;
        const int t = (int)(u - r * (uint32_t)tiles);
        const LongRunDesc &d = runs[r];
        const int row = d.row, nchunks = d.nchunks;
        const int col = t * (64 * VEC) + lane * VEC;
        if (col >= hidden) continue;
        const float *p = partial + (int64_t)d.first_partial * partial_stride;

        if (col + VEC <= hidden) {
            MT *mrow = main_grad + (int64_t)row * mg_stride + col;
            MT old[VEC];
            load_vec<MT, VEC>(mrow, old);
            float total[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) total[k] = 0.0f;
            for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
                float buf[kBatch][VEC];
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
                    if (c0 + b < nchunks)
                        load_vec<float, VEC>(p + (int64_t)(c0 + b) * partial_stride + col, buf[b]);
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
                    if (c0 + b < nchunks) {
#pragma unroll
                        for (int k = 0; k < VEC; ++k) total[k] = total[k] + buf[b][k];
                    }
            }
            MT out[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) out[k] = finish<G, M>(total[k], old[k]);
            store_vec<MT, VEC>(mrow, out);
        } else {
            for (int j = col; j < hidden; ++j) {
                float total = 0.0f;
                for (int c = 0; c < nchunks; ++c) total = total + p[(int64_t)c * partial_stride + j];
                MT *m = main_grad + (int64_t)row * mg_stride + j;
                *m = finish<G, M>(total, *m);
            }
        }
    }
}

template <typename G, typename M, int VEC>
hipError_t launch(void *main_grad, int64_t mg_stride, int hidden, void *workspace,
                  const WsLayout &l, int max_long_runs, int num_cus, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    const int tiles = (hidden + 64 * VEC - 1) / (64 * VEC);
    const int64_t max_units = (int64_t)max_long_runs * tiles;
    int64_t blocks = (max_units + (kThreads / 64) - 1) / (kThreads / 64);
    const int64_t cap = (int64_t)num_cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    long_run_sums_kernel<G, M, VEC><<<(unsigned)blocks, kThreads, 0, stream>>>(
        reinterpret_cast<WsHeader *>(ws),
        reinterpret_cast<const LongRunDesc *>(ws + l.long_runs),
        reinterpret_cast<const float *>(ws + l.partial), l.partial_stride,
        static_cast<typename M::T *>(main_grad), mg_stride, hidden, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_long_run_sums(bool grad_bf16, bool mg_bf16, bool vec, void *main_grad,
                                int64_t mg_stride, int hidden, void *workspace,
                                const WsLayout &l, int max_long_runs, int num_cus,
                                hipStream_t stream) {
#define EWG_LR(G, M, V) launch<G, M, V>(main_grad, mg_stride, hidden, workspace, l, max_long_runs, num_cus, stream)
    if (grad_bf16) {
        if (mg_bf16) return vec ? EWG_LR(BF16, BF16, 4) : EWG_LR(BF16, BF16, 1);
        return vec ? EWG_LR(BF16, F32, 4) : EWG_LR(BF16, F32, 1);
    }
    if (mg_bf16) return vec ? EWG_LR(F32, BF16, 4) : EWG_LR(F32, BF16, 1);
    return vec ? EWG_LR(F32, F32, 4) : EWG_LR(F32, F32, 1);
#undef EWG_LR
}

}  // namespace ewg
