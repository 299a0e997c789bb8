/*
 * CPU oracle for the embedding weight-gradient accumulation
 *     main_grad += embedding_dense_backward(grad, ids)
 * restricted to the rows of the ids that occur.
 *
 * TEST INFRASTRUCTURE. This file is the plain, slow definition that the GPU
 * path is checked against. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load it. It shares no code, header, table or
 * helper with the HIP library, and the library never calls it.
 *
 * Source of the arithmetic: Megatron-Core API docs,
 * "core.fusions.fused_embedding_wgrad", introduction (the two bullets and the
 * sentence after them) and the docstrings of _sort_tokens_kernel,
 * _partial_sums_kernel and _long_run_sums_kernel. In this file's words:
 *
 *   1. The pairs (token id, position) are sorted; equal ids keep their
 *      positions in ascending order (introduction, first bullet).
 *   2. A run is the set of sorted slots holding one id. It is cut into chunks
 *      of NROWS = 10 rows, counted from the start of the run, so a run of at
 *      most 10 rows is one chunk.
 *   3. Every chunk is summed in fp32, in position order, from +0.
 *   4. The chunk sums of a run are added in chunk order, in fp32, from +0.
 *   5. That total is rounded once to the gradient dtype.
 *   6. It is added to main_grad's row in fp32 and the result rounded to
 *      main_grad's dtype.
 *   7. Rows whose id does not occur are neither read nor written.
 *
 * Readings of points the page leaves open (each also pinned by a test):
 *   - "position" is the row-major flat index into ids, and grad row p is row p
 *     of grad viewed as [num_tokens, hidden];
 *   - chunk sums start from +0, like the combine;
 *   - rounding to bf16 is IEEE round-to-nearest-even; a NaN stays a NaN
 *     (its payload is not part of the definition);
 *   - for a bf16 main_grad the fp32 add and the bf16 rounding are two steps.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (no FTZ/DAZ: gradual
 * underflow is kept, as IEEE and PyTorch's default require).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_NROWS 10 /* NROWS_PER_THREAD on the page */

/* ---- dtype helpers ------------------------------------------------------ */

static float f32_from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bf16 is the upper half of a binary32; widening is exact. */
static float bf16_widen(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/*
 * Round a binary32 to bfloat16, round-to-nearest, ties to even: keep the top
 * 16 bits, then look at the 16 dropped bits. Above half -> round up; exactly
 * half -> round up only if the kept part is odd. A carry out of the
 * mantissa moves into the exponent, which is what turns the largest values
 * into infinity. NaN inputs return a quiet NaN with the same sign.
 */
uint16_t oracle_round_bf16(uint32_t x) {
    uint32_t kept = x >> 16;
    uint32_t dropped = x & 0xFFFFu;
    if ((x & 0x7F800000u) == 0x7F800000u && (x & 0x007FFFFFu) != 0)
        return (uint16_t)(kept | 0x0040u);
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1;
    return (uint16_t)kept;
}

void oracle_round_bf16_array(const uint32_t *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_bf16(x[i]);
}

/* ---- step 1: the sort of (id, position) pairs ---------------------------- */

typedef struct {
    int64_t id;
    int64_t pos;
} token_t;

static int token_cmp(const void *a, const void *b) {
    const token_t *x = (const token_t *)a, *y = (const token_t *)b;
    if (x->id != y->id) return x->id < y->id ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* Pairs sorted by id, ties in ascending position. Caller frees. */
static token_t *sorted_tokens(const void *ids, int ids_is_int64, int64_t n) {
    token_t *t = (token_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(token_t));
    if (!t) return NULL;
    for (int64_t p = 0; p < n; ++p) {
        t[p].id = ids_is_int64 ? ((const int64_t *)ids)[p] : (int64_t)((const int32_t *)ids)[p];
        t[p].pos = p;
    }
    /* positions are unique, so ordering by (id, pos) is the stable order by id */
    qsort(t, (size_t)n, sizeof(token_t), token_cmp);
    return t;
}

/*
 * The tables that the page's sort step produces, in this file's own format:
 *   sorted_ids[s], positions[s]        for sorted slot s
 *   run_first[s], run_last[s]          first and last slot (inclusive) of the
 *                                      run that holds slot s
 *   long_runs[0] = number of runs longer than NROWS, long_runs[1..] = their
 *                                      first slots, ascending
 *   chunk_first[0] = number of chunks, chunk_first[1..] = the first slot of
 *                                      every chunk, ascending
 * long_runs and chunk_first hold at least n + 1 entries.
 * Returns 0, or -1 if memory ran out.
 */
int oracle_sort_tokens(const void *ids, int ids_is_int64, int64_t n, int64_t *sorted_ids,
                       int64_t *positions, int64_t *run_first, int64_t *run_last,
                       int64_t *long_runs, int64_t *chunk_first) {
    token_t *t = sorted_tokens(ids, ids_is_int64, n);
    if (!t) return -1;
    int64_t n_long = 0, n_chunks = 0;
    int64_t s = 0;
    while (s < n) {
        int64_t e = s;
        while (e < n && t[e].id == t[s].id) ++e;
        for (int64_t q = s; q < e; ++q) {
            sorted_ids[q] = t[q].id;
            positions[q] = t[q].pos;
            run_first[q] = s;
            run_last[q] = e - 1;
        }
        if (e - s > ORACLE_NROWS) long_runs[1 + n_long++] = s;
        for (int64_t c = s; c < e; c += ORACLE_NROWS) chunk_first[1 + n_chunks++] = c;
        s = e;
    }
    long_runs[0] = n_long;
    chunk_first[0] = n_chunks;
    free(t);
    return 0;
}

/* ---- steps 2-7: the accumulation ----------------------------------------- */

/*
 * ids: n entries, int32 or int64, each in [0, rows of main_grad).
 * grad: n rows of `hidden` values, row p at grad + p * grad_row_stride
 *       (elements), bf16 (as raw uint16) or fp32.
 * main_grad: rows of `hidden` values at main_grad + id * main_grad_row_stride,
 *       bf16 (raw uint16) or fp32; updated in place on the rows that occur.
 * Returns 0, or -1 if memory ran out (main_grad is then untouched).
 */
int oracle_accumulate_embedding_wgrad(const void *ids, int ids_is_int64, int64_t n,
                                      const void *grad, int grad_is_bf16, int64_t grad_row_stride,
                                      void *main_grad, int main_grad_is_bf16,
                                      int64_t main_grad_row_stride, int64_t hidden) {
    token_t *t = sorted_tokens(ids, ids_is_int64, n);
    float *chunk_sum = (float *)malloc((size_t)(hidden > 0 ? hidden : 1) * sizeof(float));
    float *total = (float *)malloc((size_t)(hidden > 0 ? hidden : 1) * sizeof(float));
    if (!t || !chunk_sum || !total) {
        free(t);
        free(chunk_sum);
        free(total);
        return -1;
    }

    int64_t s = 0;
    while (s < n) {
        /* the run of one id: sorted slots [s, e) */
        int64_t e = s;
        while (e < n && t[e].id == t[s].id) ++e;

        for (int64_t j = 0; j < hidden; ++j) total[j] = 0.0f;

        /* chunks of NROWS rows counted from the start of the run */
        for (int64_t c = s; c < e; c += ORACLE_NROWS) {
            int64_t c_end = c + ORACLE_NROWS < e ? c + ORACLE_NROWS : e;
            for (int64_t j = 0; j < hidden; ++j) chunk_sum[j] = 0.0f;
            for (int64_t q = c; q < c_end; ++q) { /* position order */
                int64_t p = t[q].pos;
                for (int64_t j = 0; j < hidden; ++j) {
                    float g;
                    if (grad_is_bf16)
                        g = bf16_widen(((const uint16_t *)grad)[p * grad_row_stride + j]);
                    else
                        g = ((const float *)grad)[p * grad_row_stride + j];
                    chunk_sum[j] = chunk_sum[j] + g;
                }
            }
            /* combine in chunk order, from 0 */
            for (int64_t j = 0; j < hidden; ++j) total[j] = total[j] + chunk_sum[j];
        }

        /* round once to the gradient dtype, add in fp32, round to main_grad's */
        int64_t row = t[s].id;
        for (int64_t j = 0; j < hidden; ++j) {
            float g = grad_is_bf16 ? bf16_widen(oracle_round_bf16(bits_from_f32(total[j])))
                                   : total[j];
            int64_t k = row * main_grad_row_stride + j;
            if (main_grad_is_bf16) {
                uint16_t *m = (uint16_t *)main_grad;
                float sum = bf16_widen(m[k]) + g;
                m[k] = oracle_round_bf16(bits_from_f32(sum));
            } else {
                float *m = (float *)main_grad;
                m[k] = m[k] + g;
            }
        }
        s = e;
    }

    free(t);
    free(chunk_sum);
    free(total);
    return 0;
}
