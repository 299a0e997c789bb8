// Host side of the C ABI declared in include/embedding_wgrad.h: argument
// checks, workspace layout, vector-path selection and the launch.
// Nothing here touches device memory or synchronises; every launch goes on
// the caller's stream.
#include "embedding_wgrad.h"
#include "embedding_wgrad_test.h"

#include <atomic>
#include <mutex>

#include "ewg_internal.h"

namespace {

using namespace ewg;

// Implementation limit on hidden: keeps (chunks x column tiles) in 32 bits.
constexpr int64_t kMaxHidden = int64_t(1) << 24;

int bit_length(uint64_t x) {
    int b = 0;
    while (x) {
        ++b;
        x >>= 1;
    }
    return b;
}

bool is_index_dtype(int d) { return d == EWG_INT32 || d == EWG_INT64; }
bool is_float_dtype(int d) { return d == EWG_BF16 || d == EWG_FP32; }
bool is_known_dtype(int d) { return d >= EWG_INT32 && d <= EWG_FP32; }
size_t float_size(int d) { return d == EWG_BF16 ? 2 : 4; }

bool aligned(const void *p, int64_t row_stride_bytes, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a == 0) && (row_stride_bytes % (int64_t)a == 0);
}

// Compute units of the current device, cached per device ordinal.
int num_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

int check_common(int64_t num_tokens, int64_t hidden, int64_t num_embeddings, int ids_dtype,
                 int grad_dtype, int main_grad_dtype) {
    if (!is_known_dtype(ids_dtype) || !is_known_dtype(grad_dtype) || !is_known_dtype(main_grad_dtype))
        return EWG_INVALID_ARGUMENT;
    if (!can_accumulate_embedding_wgrad(num_tokens, hidden, num_embeddings, ids_dtype, grad_dtype,
                                        main_grad_dtype))
        return EWG_UNSUPPORTED;
    return EWG_OK;
}

int check_workspace(const void *workspace, size_t workspace_bytes, int64_t num_tokens,
                    int64_t hidden) {
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return EWG_INVALID_ARGUMENT;
    if (workspace_bytes < ws_layout(num_tokens, hidden).total) return EWG_WORKSPACE_TOO_SMALL;
    return EWG_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? EWG_OK : EWG_HIP_ERROR; }

// A nonzero number per call: the value the kernel's sorting workgroup
// publishes in the workspace's ready flag, which its last workgroup clears.
uint32_t next_epoch() {
    static std::atomic<uint32_t> counter{0};
    uint32_t e;
    do {
        e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
    } while (e == 0);
    return e;
}

// One call. Unsharded: rows [0, num_embeddings), other ids invalid. Vocabulary
// shard (shard = true): rows are ids [id_base, id_base + num_embeddings), other
// ids left out, and the key's id field gets one more bit (so that a kept key
// never has all id bits set; left-out keys have).
int accumulate(const void *ids, const void *grad, void *main_grad, int64_t num_tokens,
               int64_t hidden, int64_t num_embeddings, int64_t id_base, bool shard,
               int64_t grad_row_stride, int64_t main_grad_row_stride, int ids_dtype,
               int grad_dtype, int main_grad_dtype, void *workspace, size_t workspace_bytes,
               hipStream_t stream, hipEvent_t *events, int grid = 0, int odd_skip_long = 0) {
    int st = shard ? (!is_known_dtype(ids_dtype) || !is_known_dtype(grad_dtype) ||
                              !is_known_dtype(main_grad_dtype)
                          ? EWG_INVALID_ARGUMENT
                          : (can_accumulate_embedding_wgrad_vocab_shard(num_tokens, hidden, id_base,
                                                                        num_embeddings, ids_dtype,
                                                                        grad_dtype, main_grad_dtype)
                                 ? EWG_OK
                                 : EWG_UNSUPPORTED))
                   : check_common(num_tokens, hidden, num_embeddings, ids_dtype, grad_dtype,
                                  main_grad_dtype);
    if (st != EWG_OK) return st;
    if (!ids || !grad || !main_grad) return EWG_INVALID_ARGUMENT;
    if (grad_row_stride < hidden || main_grad_row_stride < hidden) return EWG_INVALID_ARGUMENT;
    st = check_workspace(workspace, workspace_bytes, num_tokens, hidden);
    if (st != EWG_OK) return st;

    const bool g_bf16 = grad_dtype == EWG_BF16, m_bf16 = main_grad_dtype == EWG_BF16;
    const size_t gs = float_size(grad_dtype), ms = float_size(main_grad_dtype);
    // vector path: a lane moves 16 bytes of grad and the same columns of main_grad
    const int vec_g = (int)(16 / gs);
    const bool vec = aligned(grad, grad_row_stride * (int64_t)gs, 16) &&
                     aligned(main_grad, main_grad_row_stride * (int64_t)ms,
                             vec_g * ms < 16 ? vec_g * ms : 16);

    const WsLayout l = ws_layout(num_tokens, hidden);
    const int n = (int)num_tokens;
    const int pos_bits = ewg_position_bits(num_tokens);
    const int id_bits = bit_length((uint64_t)(shard ? num_embeddings : num_embeddings - 1));

    (void)hipGetLastError();   // start from a clean per-thread error state
    if (events && hipEventRecord(events[0], stream) != hipSuccess) return EWG_HIP_ERROR;
    st = to_status(launch_accumulate(ids_dtype == EWG_INT64, g_bf16, m_bf16, vec, ids, n,
                                     (int)num_embeddings, id_base, shard, pos_bits, id_bits, grad,
                                     grad_row_stride,
                                     main_grad, main_grad_row_stride, (int)hidden, workspace, l,
                                     grid > 0 ? grid : num_cus(), next_epoch(), odd_skip_long,
                                     events ? events[2] : nullptr, events ? events[3] : nullptr,
                                     stream));
    if (st != EWG_OK) return st;
    if (events && hipEventRecord(events[1], stream) != hipSuccess) return EWG_HIP_ERROR;
    return EWG_OK;
}

// One call of the many-token path.
int accumulate_many(const void *ids, const void *grad, void *main_grad, int64_t num_tokens,
                    int64_t hidden, int64_t num_embeddings, int64_t grad_row_stride,
                    int64_t main_grad_row_stride, int ids_dtype, int grad_dtype,
                    int main_grad_dtype, void *workspace, size_t workspace_bytes,
                    hipStream_t stream, hipEvent_t *events) {
    if (!is_known_dtype(ids_dtype) || !is_known_dtype(grad_dtype) || !is_known_dtype(main_grad_dtype))
        return EWG_INVALID_ARGUMENT;
    if (!can_accumulate_embedding_wgrad_many_tokens(num_tokens, hidden, num_embeddings, ids_dtype,
                                                    grad_dtype, main_grad_dtype))
        return EWG_UNSUPPORTED;
    if (!ids || !grad || !main_grad) return EWG_INVALID_ARGUMENT;
    if (grad_row_stride < hidden || main_grad_row_stride < hidden) return EWG_INVALID_ARGUMENT;
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return EWG_INVALID_ARGUMENT;
    const ManyLayout l = many_layout(num_tokens, hidden);
    if (workspace_bytes < l.total) return EWG_WORKSPACE_TOO_SMALL;

    const size_t gs = float_size(grad_dtype), ms = float_size(main_grad_dtype);
    const int vec_g = (int)(16 / gs);
    const bool vec = aligned(grad, grad_row_stride * (int64_t)gs, 16) &&
                     aligned(main_grad, main_grad_row_stride * (int64_t)ms,
                             vec_g * ms < 16 ? vec_g * ms : 16);
    (void)hipGetLastError();
    if (events && hipEventRecord(events[0], stream) != hipSuccess) return EWG_HIP_ERROR;
    int st = to_status(launch_many_tokens(
        ids_dtype == EWG_INT64, grad_dtype == EWG_BF16, main_grad_dtype == EWG_BF16, vec, ids,
        (int)num_tokens, (int)num_embeddings, bit_length((uint64_t)(num_embeddings - 1)), grad,
        grad_row_stride, main_grad, main_grad_row_stride, (int)hidden, workspace, l, num_cus(),
        stream));
    if (st != EWG_OK) return st;
    if (events && hipEventRecord(events[1], stream) != hipSuccess) return EWG_HIP_ERROR;
    return EWG_OK;
}

// ---- the entry point that allocates nothing ----------------------------------

// Workspace of accumulate_embedding_wgrad_no_alloc: one array on every device
// the library runs on, held until the process ends. On the host this name is
// only a stand-in for the symbol; host code uses the device address that
// hipGetSymbolAddress returns for the current device, never the name.
static __device__ __align__(256) uint8_t scratch[EWG_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device: looked up once per
// device, with that device current, and kept. nullptr if the lookup fails.
void *scratch_address() {
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        addr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

constexpr int kHeaderWords = (int)(sizeof(WsHeader) / sizeof(uint32_t));
static_assert(kHeaderWords <= 1024, "one workgroup clears the header");

// Zeroes the workspace header: the flag, tickets and counters a call starts
// from. A kernel rather than a memset node, so the call may be captured.
__global__ void clear_header_kernel(uint32_t *__restrict__ words) { words[threadIdx.x] = 0u; }

}  // namespace

extern "C" {

int ewg_position_bits(int64_t num_tokens) {
    return num_tokens <= 1 ? 0 : bit_length((uint64_t)(num_tokens - 1));
}

int can_accumulate_embedding_wgrad(int64_t num_tokens, int64_t hidden, int64_t num_embeddings,
                                   int ids_dtype, int grad_dtype, int main_grad_dtype) {
    if (num_tokens < EWG_MIN_TOKENS || num_tokens > EWG_MAX_TOKENS) return 0;
    if (hidden < 1 || hidden > kMaxHidden || num_embeddings < 1) return 0;
    if (!is_index_dtype(ids_dtype) || !is_float_dtype(grad_dtype) || !is_float_dtype(main_grad_dtype))
        return 0;
    const int pb = ewg_position_bits(num_tokens);
    // ((num_embeddings - 1) << pb) | (num_tokens - 1) < 2^31
    if (num_embeddings - 1 >= (int64_t(1) << (31 - pb))) return 0;
    return 1;
}

size_t accumulate_embedding_wgrad_workspace_bytes(int64_t num_tokens, int64_t hidden) {
    if (num_tokens < 1 || num_tokens > EWG_MAX_TOKENS || hidden < 1 || hidden > kMaxHidden) return 0;
    return ws_layout(num_tokens, hidden).total;
}

int accumulate_embedding_wgrad(const void *ids, const void *grad, void *main_grad,
                               int64_t num_tokens, int64_t hidden, int64_t num_embeddings,
                               int64_t grad_row_stride, int64_t main_grad_row_stride,
                               int ids_dtype, int grad_dtype, int main_grad_dtype,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return accumulate(ids, grad, main_grad, num_tokens, hidden, num_embeddings, 0, false,
                      grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                      main_grad_dtype, workspace, workspace_bytes, stream, nullptr);
}

int accumulate_embedding_wgrad_timed(const void *ids, const void *grad, void *main_grad,
                                     int64_t num_tokens, int64_t hidden, int64_t num_embeddings,
                                     int64_t grad_row_stride, int64_t main_grad_row_stride,
                                     int ids_dtype, int grad_dtype, int main_grad_dtype,
                                     void *workspace, size_t workspace_bytes,
                                     hipStream_t stream, hipEvent_t *events) {
    if (!events) return EWG_INVALID_ARGUMENT;
    return accumulate(ids, grad, main_grad, num_tokens, hidden, num_embeddings, 0, false,
                      grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                      main_grad_dtype, workspace, workspace_bytes, stream, events);
}

int accumulate_embedding_wgrad_no_alloc(const void *ids, const void *grad, void *main_grad,
                                        int64_t num_tokens, int64_t hidden,
                                        int64_t num_embeddings, int64_t grad_row_stride,
                                        int64_t main_grad_row_stride, int ids_dtype,
                                        int grad_dtype, int main_grad_dtype, hipStream_t stream) {
    int st = check_common(num_tokens, hidden, num_embeddings, ids_dtype, grad_dtype,
                          main_grad_dtype);
    if (st != EWG_OK) return st;
    if (!ids || !grad || !main_grad) return EWG_INVALID_ARGUMENT;
    if (grad_row_stride < hidden || main_grad_row_stride < hidden) return EWG_INVALID_ARGUMENT;
    if (ws_layout(num_tokens, hidden).total > (size_t)EWG_NO_ALLOC_SCRATCH_BYTES)
        return EWG_SCRATCH_TOO_SMALL;
    void *ws = scratch_address();
    if (!ws) return EWG_HIP_ERROR;
    (void)hipGetLastError();
    clear_header_kernel<<<1, kHeaderWords, 0, stream>>>(static_cast<uint32_t *>(ws));
    if (hipGetLastError() != hipSuccess) return EWG_HIP_ERROR;
    return accumulate(ids, grad, main_grad, num_tokens, hidden, num_embeddings, 0, false,
                      grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                      main_grad_dtype, ws, (size_t)EWG_NO_ALLOC_SCRATCH_BYTES, stream, nullptr);
}

int can_accumulate_embedding_wgrad_vocab_shard(int64_t num_tokens, int64_t hidden,
                                               int64_t vocab_start, int64_t shard_rows,
                                               int ids_dtype, int grad_dtype, int main_grad_dtype) {
    if (num_tokens < EWG_MIN_TOKENS || num_tokens > EWG_MAX_TOKENS) return 0;
    if (hidden < 1 || hidden > kMaxHidden || vocab_start < 0 || shard_rows < 1) return 0;
    if (!is_index_dtype(ids_dtype) || !is_float_dtype(grad_dtype) || !is_float_dtype(main_grad_dtype))
        return 0;
    // (shard_rows << pb) | (num_tokens - 1) < 2^31: one id bit more than the unsharded check
    const int pb = ewg_position_bits(num_tokens);
    if (shard_rows >= (int64_t(1) << (31 - pb))) return 0;
    return 1;
}

int accumulate_embedding_wgrad_vocab_shard(const void *ids, const void *grad, void *main_grad,
                                           int64_t num_tokens, int64_t hidden,
                                           int64_t vocab_start, int64_t shard_rows,
                                           int64_t grad_row_stride, int64_t main_grad_row_stride,
                                           int ids_dtype, int grad_dtype, int main_grad_dtype,
                                           void *workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
    return accumulate(ids, grad, main_grad, num_tokens, hidden, shard_rows, vocab_start, true,
                      grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                      main_grad_dtype, workspace, workspace_bytes, stream, nullptr);
}

int accumulate_embedding_wgrad_sort_tokens(const void *ids, int64_t num_tokens,
                                           int64_t num_embeddings, int ids_dtype,
                                           int32_t *sorted_ids, int32_t *positions,
                                           int32_t *run_first, int32_t *run_last,
                                           int32_t *long_runs, int32_t *chunk_first,
                                           void *workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
    if (!is_known_dtype(ids_dtype)) return EWG_INVALID_ARGUMENT;
    if (!can_accumulate_embedding_wgrad(num_tokens, 1, num_embeddings, ids_dtype, EWG_FP32, EWG_FP32))
        return EWG_UNSUPPORTED;
    if (!ids || !sorted_ids || !positions || !run_first || !run_last || !long_runs || !chunk_first)
        return EWG_INVALID_ARGUMENT;
    // the sort step uses only the table part of the workspace, which does not depend on hidden
    int st = check_workspace(workspace, workspace_bytes, num_tokens, 1);
    if (st != EWG_OK) return st;
    const WsLayout l = ws_layout(num_tokens, 1);
    const SortTables tables = {sorted_ids, positions, run_first, run_last, long_runs, chunk_first};
    (void)hipGetLastError();
    return to_status(launch_sort_tokens(ids, ids_dtype == EWG_INT64, (int)num_tokens,
                                        (int)num_embeddings, ewg_position_bits(num_tokens),
                                        bit_length((uint64_t)(num_embeddings - 1)), workspace, l,
                                        tables, stream));
}

int can_accumulate_embedding_wgrad_many_tokens(int64_t num_tokens, int64_t hidden,
                                               int64_t num_embeddings, int ids_dtype,
                                               int grad_dtype, int main_grad_dtype) {
    if (num_tokens < EWG_MIN_TOKENS || num_tokens > EWG_MANY_MAX_TOKENS) return 0;
    if (hidden < 1 || hidden > kMaxHidden) return 0;
    if (num_embeddings < 1 || num_embeddings > EWG_MANY_MAX_EMBEDDINGS) return 0;
    if (!is_index_dtype(ids_dtype) || !is_float_dtype(grad_dtype) || !is_float_dtype(main_grad_dtype))
        return 0;
    return 1;
}

size_t accumulate_embedding_wgrad_many_tokens_workspace_bytes(int64_t num_tokens, int64_t hidden) {
    if (num_tokens < 1 || num_tokens > EWG_MANY_MAX_TOKENS || hidden < 1 || hidden > kMaxHidden)
        return 0;
    return many_layout(num_tokens, hidden).total;
}

int accumulate_embedding_wgrad_many_tokens(const void *ids, const void *grad, void *main_grad,
                                           int64_t num_tokens, int64_t hidden,
                                           int64_t num_embeddings, int64_t grad_row_stride,
                                           int64_t main_grad_row_stride, int ids_dtype,
                                           int grad_dtype, int main_grad_dtype, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
    return accumulate_many(ids, grad, main_grad, num_tokens, hidden, num_embeddings,
                           grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                           main_grad_dtype, workspace, workspace_bytes, stream, nullptr);
}

int accumulate_embedding_wgrad_many_tokens_timed(const void *ids, const void *grad,
                                                 void *main_grad, int64_t num_tokens,
                                                 int64_t hidden, int64_t num_embeddings,
                                                 int64_t grad_row_stride,
                                                 int64_t main_grad_row_stride, int ids_dtype,
                                                 int grad_dtype, int main_grad_dtype,
                                                 void *workspace, size_t workspace_bytes,
                                                 hipStream_t stream, hipEvent_t *events) {
    if (!events) return EWG_INVALID_ARGUMENT;
    return accumulate_many(ids, grad, main_grad, num_tokens, hidden, num_embeddings,
                           grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                           main_grad_dtype, workspace, workspace_bytes, stream, events);
}

int ewg_test_accumulate_embedding_wgrad(const void *ids, const void *grad, void *main_grad,
                                        int64_t num_tokens, int64_t hidden,
                                        int64_t num_embeddings, int64_t grad_row_stride,
                                        int64_t main_grad_row_stride, int ids_dtype,
                                        int grad_dtype, int main_grad_dtype, void *workspace,
                                        size_t workspace_bytes, int grid, int odd_skip_long,
                                        hipStream_t stream) {
    if (grid < 2 || grid > kMaxGrid || (odd_skip_long != 0 && odd_skip_long != 1))
        return EWG_INVALID_ARGUMENT;
    return accumulate(ids, grad, main_grad, num_tokens, hidden, num_embeddings, 0, false,
                      grad_row_stride, main_grad_row_stride, ids_dtype, grad_dtype,
                      main_grad_dtype, workspace, workspace_bytes, stream, nullptr, grid,
                      odd_skip_long);
}

const char *ewg_status_string(int status) {
    switch (status) {
        case EWG_OK: return "success";
        case EWG_UNSUPPORTED: return "unsupported: outside the envelope of can_accumulate_embedding_wgrad";
        case EWG_INVALID_ARGUMENT: return "invalid argument (null pointer, stride below hidden, unknown dtype code or misaligned workspace)";
        case EWG_WORKSPACE_TOO_SMALL: return "workspace smaller than accumulate_embedding_wgrad_workspace_bytes()";
        case EWG_HIP_ERROR: return "HIP error while enqueueing a kernel";
        case EWG_SCRATCH_TOO_SMALL: return "sizes need more workspace than the library's static scratch (EWG_NO_ALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
