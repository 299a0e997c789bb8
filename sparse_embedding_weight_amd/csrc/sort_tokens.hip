// Sort step on its own, with its tables written out (the inspection entry
// point accumulate_embedding_wgrad_sort_tokens). The sort itself is the
// device code in sort_lds.h that the fused accumulate kernel runs.
//
// Megatron-Core API docs, "core.fusions.fused_embedding_wgrad",
// _sort_tokens_kernel.
#include "ewg_internal.h"
#include "sort_lds.h"

namespace ewg {
namespace {

template <typename IdT>
__global__ __launch_bounds__(kSortThreads) void sort_tokens_kernel(
    const IdT *__restrict__ ids, int n, int num_embeddings, int pos_bits, int id_bits,
    WsHeader *__restrict__ hdr, SortTables tables) {
    __shared__ SortSmem sm;
    const SortOutputs out = {tables, hdr, nullptr, nullptr};
    const int bad = load_keys<IdT>(sm, ids, n, num_embeddings, pos_bits, 0, false);
    if (bad) {
        report_invalid(out, bad);
        return;
    }
    const int cur = radix_sort_ids(sm, pos_bits, id_bits, n);
    mark_runs(sm, cur, n, pos_bits, out);
}

}  // namespace

hipError_t launch_sort_tokens(const void *ids, bool ids_int64, int n, int num_embeddings,
                              int pos_bits, int id_bits, void *workspace, const WsLayout &l,
                              const SortTables &tables, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws);
    (void)l;
    if (ids_int64)
        sort_tokens_kernel<int64_t><<<1, kSortThreads, 0, stream>>>(
            static_cast<const int64_t *>(ids), n, num_embeddings, pos_bits, id_bits, hdr, tables);
    else
        sort_tokens_kernel<int32_t><<<1, kSortThreads, 0, stream>>>(
            static_cast<const int32_t *>(ids), n, num_embeddings, pos_bits, id_bits, hdr, tables);
    return hipGetLastError();
}

}  // namespace ewg
