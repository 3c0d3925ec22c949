/*
 * topk_oracle.c - plain CPU oracle for the windowed per-row top-k selection
 * with RAGGED and PAGED emit.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU library never
 * includes, links or calls anything here, and this file includes nothing of
 * the GPU library.
 *
 * What is computed, and where the pages say so:
 *
 *  - Window. Row b selects among the scores in columns
 *    [row_start_b, row_start_b + seq_len_b) of its score row; a missing
 *    row_starts array means row_start = 0 for every row.
 *    (sglang PR #35175 digest, "RAGGED prefill top-k moved to the v2 JIT
 *    kernel", section "Key source excerpts", topk_ragged_kernel: the
 *    kernel's header comment and its metadata prefetch.)
 *  - Trivial rows. If seq_len <= k the row's outputs are positions
 *    0 .. seq_len-1 and the scores are never read.
 *    (same excerpt, the "trivial path" branch.)
 *  - Count. Exactly min(k, seq_len) valid outputs per row; the remaining
 *    k - min(k, seq_len) slots hold -1.
 *    (same excerpt, trivial branch pads with -1; sglang PR #26788 digest,
 *    "faster top-k + page-table transform (runtime k <= 2048)", section
 *    "Key source excerpts", _assert_topk_close asserts the count.)
 *  - Order. The k largest scores. The pages leave equal scores unordered
 *    (the same test forgives equal-score swaps); this library fixes the
 *    rule: higher score first, and among equal scores (IEEE ==, so -0.0 and
 *    +0.0 are equal) the lower window position first.
 *  - RAGGED emit: position + out_offset_b.
 *    (PR #35175 digest, topk_ragged_kernel: the window is shifted by the
 *    alignment remainder and the bias is reduced by the same amount, so the
 *    output is the window position plus out_offsets[b]; TopKProblem::emit
 *    adds the bias.)
 *  - PAGED emit: page_table[b][pos / page_size] * page_size
 *    + pos % page_size, with page_size a power of two.
 *    (PR #35175 digest, TopKProblem::transform_output / page_to_indices
 *    with page_bits = log2(page_size).)
 *  - Packed PAGED emit: row b looks up table row table_rows[b] (b when
 *    absent) at table position table_starts[b] + pos (pos when absent):
 *    several query rows of one request share that request's table, and the
 *    score window's start in the batch-wide score layout (row_start) is
 *    separate from the window's start in the request's own table.
 *    (sglang/FlashInfer packed PAGED digest, "fix(dsa): use FlashInfer fused
 *    top-k for packed PAGED rows": page_table_row_starts = row_starts minus
 *    the request's cu_seqlens_k start, gathered by row_to_batch.)
 *  - Raw positions beside the PAGED output: the selected window positions
 *    themselves (PR #26788 digest, the transform's optional out_raw_indices;
 *    raw-index mode in the PR #35175 digest, "Motivation").
 *  - Comparison form: the valid outputs are compared as a sorted list,
 *    because the kernels' output order inside a row is free (the pages'
 *    test compares sets).
 *
 * Negative seq_len is read as 0 (an all -1 row). NaN scores are outside the
 * contract: the comparator below is not a total order on them.
 *
 * The selection is a full sort of (score, position) pairs per row with
 * qsort, rows spread over POSIX threads. No blocking, no partial selection,
 * no shortcuts beyond the trivial-row rule that the pages state.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float w;
    int32_t j;
} scored_pos;

/* Descending score; equal scores (IEEE ==) by ascending position. */
static int cmp_score_desc_pos_asc(const void* pa, const void* pb) {
    const scored_pos* a = (const scored_pos*)pa;
    const scored_pos* b = (const scored_pos*)pb;
    if (a->w > b->w) return -1;
    if (a->w < b->w) return 1;
    if (a->j < b->j) return -1;
    if (a->j > b->j) return 1;
    return 0;
}

static int cmp_i32_asc(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa;
    int32_t b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

typedef struct {
    const float* scores;
    int64_t stride;
    const int32_t* seq_lens;
    const int32_t* row_starts;
    int32_t num_rows;
    int32_t k;
    int32_t* sel;
    int32_t next_row; /* shared work counter */
    pthread_mutex_t lock;
    int failed;
} select_job;

/* One row: sel_row[0 .. n) = selected window positions in ascending order,
 * sel_row[n .. k) = -1. Returns 0, or -1 if scratch memory ran out. */
static int select_one_row(const select_job* job, int32_t b, scored_pos** scratch,
                          int64_t* scratch_cap) {
    int32_t L = job->seq_lens[b];
    if (L < 0) L = 0;
    int32_t k = job->k;
    int32_t* out = job->sel + (int64_t)b * k;
    int32_t n = L < k ? L : k;

    if (L <= k) {
        for (int32_t t = 0; t < k; ++t) out[t] = t < L ? t : -1;
        return 0;
    }
    if (*scratch_cap < L) {
        free(*scratch);
        *scratch = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)L);
        if (*scratch == NULL) {
            *scratch_cap = 0;
            return -1;
        }
        *scratch_cap = L;
    }
    int64_t s = job->row_starts ? job->row_starts[b] : 0;
    const float* row = job->scores + (int64_t)b * job->stride + s;
    scored_pos* e = *scratch;
    for (int32_t j = 0; j < L; ++j) {
        e[j].w = row[j];
        e[j].j = j;
    }
    qsort(e, (size_t)L, sizeof(scored_pos), cmp_score_desc_pos_asc);
    for (int32_t t = 0; t < n; ++t) out[t] = e[t].j;
    qsort(out, (size_t)n, sizeof(int32_t), cmp_i32_asc);
    for (int32_t t = n; t < k; ++t) out[t] = -1;
    return 0;
}

static void* select_worker(void* arg) {
    select_job* job = (select_job*)arg;
    scored_pos* scratch = NULL;
    int64_t cap = 0;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int32_t b = job->next_row++;
        pthread_mutex_unlock(&job->lock);
        if (b >= job->num_rows) break;
        if (select_one_row(job, b, &scratch, &cap) != 0) {
            pthread_mutex_lock(&job->lock);
            job->failed = 1;
            pthread_mutex_unlock(&job->lock);
            break;
        }
    }
    free(scratch);
    return NULL;
}

/*
 * Selected window positions per row.
 *   scores     fp32 [num_rows, stride], row-major, host memory
 *   seq_lens   int32 [num_rows]
 *   row_starts int32 [num_rows] or NULL (all zero)
 *   sel        int32 [num_rows, k] (written): ascending positions, then -1
 *   nthreads   worker threads (>= 1)
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
int oracle_select(const float* scores, int64_t stride, const int32_t* seq_lens,
                  const int32_t* row_starts, int32_t num_rows, int32_t k, int32_t* sel,
                  int32_t nthreads) {
    if (num_rows < 0 || k < 1 || nthreads < 1) return 1;
    if (num_rows == 0) return 0;
    if (scores == NULL || seq_lens == NULL || sel == NULL || stride < 1) return 1;
    select_job job;
    job.scores = scores;
    job.stride = stride;
    job.seq_lens = seq_lens;
    job.row_starts = row_starts;
    job.num_rows = num_rows;
    job.k = k;
    job.sel = sel;
    job.next_row = 0;
    job.failed = 0;
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads > num_rows) nthreads = num_rows;
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (tids == NULL) return 2;
    int32_t started = 0;
    for (int32_t t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, select_worker, &job) != 0) break;
        started = t;
    }
    select_worker(&job);
    for (int32_t t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    free(tids);
    pthread_mutex_destroy(&job.lock);
    return job.failed ? 2 : 0;
}

/*
 * RAGGED emit: out[b][t] = sel[b][t] + out_offsets[b] for valid slots,
 * -1 for padding. The ascending order of sel is kept (adding a constant).
 */
void oracle_emit_ragged(const int32_t* sel, int32_t num_rows, int32_t k,
                        const int32_t* out_offsets, int32_t* out) {
    for (int64_t b = 0; b < num_rows; ++b) {
        for (int32_t t = 0; t < k; ++t) {
            int32_t j = sel[b * k + t];
            out[b * k + t] = j < 0 ? -1 : j + out_offsets[b];
        }
    }
}

/*
 * PAGED emit: out = page_table[b][j >> log2(p)] * p + (j & (p - 1)) for
 * valid slots, -1 for padding; the valid slots are then sorted ascending.
 * page_size must be a power of two (checked: returns 1 otherwise).
 */
int oracle_emit_paged(const int32_t* sel, int32_t num_rows, int32_t k,
                      const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                      int32_t* out) {
    if (page_size < 1 || (page_size & (page_size - 1)) != 0) return 1;
    int32_t bits = 0;
    while ((1 << bits) < page_size) ++bits;
    for (int64_t b = 0; b < num_rows; ++b) {
        int32_t n = 0;
        for (int32_t t = 0; t < k; ++t) {
            int32_t j = sel[b * k + t];
            if (j < 0) {
                out[b * k + t] = -1;
            } else {
                int32_t page = page_table[b * pt_stride + (j >> bits)];
                out[b * k + t] = page * page_size + (j & (page_size - 1));
                ++n;
            }
        }
        qsort(out + b * k, (size_t)n, sizeof(int32_t), cmp_i32_asc);
    }
    return 0;
}

/*
 * Packed PAGED emit: q = table_starts[b] + j (j when table_starts is NULL),
 * out = page_table[tr][q >> log2(p)] * p + (q & (p - 1)) with
 * tr = table_rows[b] (b when table_rows is NULL), -1 for padding; the valid
 * slots are then sorted ascending. Returns 1 for a page_size that is not a
 * power of two, 2 for a negative table position.
 */
int oracle_emit_paged_packed(const int32_t* sel, int32_t num_rows, int32_t k,
                             const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                             const int32_t* table_rows, const int32_t* table_starts,
                             int32_t* out) {
    if (page_size < 1 || (page_size & (page_size - 1)) != 0) return 1;
    for (int64_t b = 0; b < num_rows; ++b) {
        int64_t tr = table_rows ? table_rows[b] : b;
        int64_t ts = table_starts ? table_starts[b] : 0;
        int32_t n = 0;
        for (int32_t t = 0; t < k; ++t) {
            int32_t j = sel[b * k + t];
            if (j < 0) {
                out[b * k + t] = -1;
                continue;
            }
            int64_t q = ts + j;
            if (q < 0) return 2;
            int64_t page = page_table[tr * pt_stride + q / page_size];
            out[b * k + t] = (int32_t)(page * page_size + q % page_size);
            ++n;
        }
        qsort(out + b * k, (size_t)n, sizeof(int32_t), cmp_i32_asc);
    }
    return 0;
}
