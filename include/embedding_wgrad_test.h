/*
 * embedding_wgrad_test.h -- test-only entry point of libembedding_wgrad.so.
 *
 * Not part of the product interface: the tests use it to drive launch shapes
 * that a normal call never takes (a normal call launches one workgroup per
 * compute unit, and every workgroup takes long-run work). The library reads
 * no environment variable; these settings reach it
 * only through this function's arguments.
 */
#ifndef EMBEDDING_WGRAD_TEST_H
#define EMBEDDING_WGRAD_TEST_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * accumulate_embedding_wgrad (same arguments, checks, arithmetic and result),
 * launched with `grid` workgroups (2 <= grid <= 4095) instead of one per
 * compute unit. With odd_skip_long = 1 every odd-numbered workgroup takes no
 * column block of a long run, as a workgroup that starts late would find
 * none left: the even ones take them all from the shared ticket. The result
 * is bit-identical either way. Returns EWG_INVALID_ARGUMENT for a grid or
 * flag outside these ranges, else what accumulate_embedding_wgrad returns.
 */
int ewg_test_accumulate_embedding_wgrad(const void *ids, const void *grad, void *main_grad,
                                        int64_t num_tokens, int64_t hidden,
                                        int64_t num_embeddings, int64_t grad_row_stride,
                                        int64_t main_grad_row_stride, int ids_dtype,
                                        int grad_dtype, int main_grad_dtype, void *workspace,
                                        size_t workspace_bytes, int grid, int odd_skip_long,
                                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EMBEDDING_WGRAD_TEST_H */
