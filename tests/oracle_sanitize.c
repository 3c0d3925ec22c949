/*
 * oracle_sanitize.c - drives the CPU oracle (oracle/topk_oracle.c) under
 * gcc's AddressSanitizer + UndefinedBehaviorSanitizer, or ThreadSanitizer.
 *
 * Test infrastructure: built and run by tests/test_sanitized.py on
 * the host only; it links the oracle's C file directly and nothing of the
 * GPU library.
 *
 * Every case is checked against a rank definition that shares no code with
 * the oracle's sort: window position j is selected exactly when fewer than
 * k window positions beat it, where i beats j if its score is larger, or
 * equal (IEEE ==) with a lower position. The selected list is ascending and
 * padded with -1 to k slots; RAGGED adds out_offset, PAGED maps through the
 * page table and sorts the valid slots.
 *
 * Cases: random rows with ties, -0.0/+0.0, +-inf and FLT_MAX; empty,
 * negative and trivial (seq_len <= k) rows; k = 1 and k larger than the
 * stride; row starts that shift the window; page sizes 1, 2, 64; packed
 * table rows and table starts; worker counts 1 to 8 (more than rows, too).
 * Exit status 0 when every case matches; a sanitizer report aborts.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_select(const float* scores, int64_t stride, const int32_t* seq_lens,
                  const int32_t* row_starts, int32_t num_rows, int32_t k, int32_t* sel,
                  int32_t nthreads);
void oracle_emit_ragged(const int32_t* sel, int32_t num_rows, int32_t k,
                        const int32_t* out_offsets, int32_t* out);
int oracle_emit_paged(const int32_t* sel, int32_t num_rows, int32_t k,
                      const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                      int32_t* out);
int oracle_emit_paged_packed(const int32_t* sel, int32_t num_rows, int32_t k,
                             const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                             const int32_t* table_rows, const int32_t* table_starts,
                             int32_t* out);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static uint32_t next_u32(void) {
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

static int32_t below(int32_t n) { return n <= 0 ? 0 : (int32_t)(next_u32() % (uint32_t)n); }

static float draw_score(int style) {
    uint32_t r = next_u32() % 100;
    if (style == 1) return (float)(r % 4);  /* heavy ties */
    if (r == 0) return -0.0f;
    if (r == 1) return 0.0f;
    if (r == 2) return INFINITY;
    if (r == 3) return -INFINITY;
    if (r == 4) return FLT_MAX;
    if (r == 5) return -FLT_MAX;
    return (float)((int32_t)next_u32() % 20001) / 64.0f;
}

static int fails = 0;

static void expect_eq(const int32_t* got, const int32_t* want, int64_t n, const char* what,
                      int case_id) {
    for (int64_t i = 0; i < n; ++i) {
        if (got[i] != want[i]) {
            if (fails < 10)
                fprintf(stderr, "case %d %s: slot %lld got %d want %d\n", case_id, what,
                        (long long)i, got[i], want[i]);
            ++fails;
            return;
        }
    }
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Selected positions of one row by the rank definition. */
static void rank_select(const float* row, int32_t len, int32_t k, int32_t* out) {
    int32_t n = 0;
    for (int32_t j = 0; j < len; ++j) {
        int32_t beaten = 0;
        for (int32_t i = 0; i < len && beaten < k; ++i)
            if (row[i] > row[j] || (row[i] == row[j] && i < j)) ++beaten;
        if (beaten < k) out[n++] = j;
    }
    for (int32_t t = n; t < k; ++t) out[t] = -1;
}

static void run_case(int case_id, int32_t R, int64_t stride, int32_t k, int32_t nthreads,
                     int style, int with_starts) {
    float* scores = (float*)malloc(sizeof(float) * (size_t)(R * stride + 1));
    int32_t* lens = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R + 1));
    int32_t* starts = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R + 1));
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R * k + 1));
    int32_t* want = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R * k + 1));
    int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R * k + 1));
    int32_t* exp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R * k + 1));
    int32_t* offs = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R + 1));
    for (int64_t i = 0; i < R * stride; ++i) scores[i] = draw_score(style);
    for (int32_t b = 0; b < R; ++b) {
        int32_t kind = below(8);
        int32_t len;
        if (kind == 0) len = 0;
        else if (kind == 1) len = -1 - below(5);
        else if (kind == 2) len = below(k + 1);          /* trivial */
        else if (kind == 3) len = (int32_t)stride;        /* whole row */
        else len = below((int32_t)stride + 1);
        if (len > stride) len = (int32_t)stride;
        int32_t start = 0;
        if (with_starts && len < stride) start = below((int32_t)stride - (len > 0 ? len : 0) + 1);
        lens[b] = len;
        starts[b] = start;
        offs[b] = below(1 << 20);
    }
    int rc = oracle_select(scores, stride, lens, with_starts ? starts : NULL, R, k, sel,
                           nthreads);
    if (rc != 0) {
        fprintf(stderr, "case %d: oracle_select returned %d\n", case_id, rc);
        ++fails;
    }
    for (int32_t b = 0; b < R; ++b) {
        int32_t len = lens[b] > 0 ? lens[b] : 0;
        const float* row = scores + (int64_t)b * stride + (with_starts ? starts[b] : 0);
        rank_select(row, len, k, want + (int64_t)b * k);
    }
    expect_eq(sel, want, (int64_t)R * k, "select", case_id);

    oracle_emit_ragged(sel, R, k, offs, out);
    for (int64_t i = 0; i < (int64_t)R * k; ++i)
        exp[i] = want[i] < 0 ? -1 : want[i] + offs[i / k];
    expect_eq(out, exp, (int64_t)R * k, "ragged", case_id);

    static const int32_t page_sizes[3] = {1, 2, 64};
    for (int p = 0; p < 3; ++p) {
        int32_t ps = page_sizes[p];
        int64_t width = (stride + ps - 1) / ps;
        int32_t* table = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R * width + 1));
        for (int64_t i = 0; i < R * width; ++i) table[i] = below((1 << 22) / ps);
        if (oracle_emit_paged(sel, R, k, table, width, ps, out) != 0) {
            fprintf(stderr, "case %d: oracle_emit_paged rejected page size %d\n", case_id, ps);
            ++fails;
        }
        for (int32_t b = 0; b < R; ++b) {
            int32_t n = 0;
            for (int32_t t = 0; t < k; ++t) {
                int32_t j = want[(int64_t)b * k + t];
                if (j < 0) {
                    exp[(int64_t)b * k + t] = -1;
                } else {
                    exp[(int64_t)b * k + t] = table[(int64_t)b * width + j / ps] * ps + j % ps;
                    ++n;
                }
            }
            qsort(exp + (int64_t)b * k, (size_t)n, sizeof(int32_t), cmp_i32);
        }
        expect_eq(out, exp, (int64_t)R * k, "paged", case_id);

        /* Packed: rows share T = R/2 + 1 table rows, table starts shift the window. */
        int32_t T = R / 2 + 1;
        int64_t pwidth = (2 * stride + ps - 1) / ps;
        int32_t* ptab = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * pwidth + 1));
        int32_t* trow = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R + 1));
        int32_t* tstart = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R + 1));
        for (int64_t i = 0; i < T * pwidth; ++i) ptab[i] = below((1 << 22) / ps);
        for (int32_t b = 0; b < R; ++b) {
            trow[b] = below(T);
            tstart[b] = below((int32_t)stride + 1);
        }
        if (oracle_emit_paged_packed(sel, R, k, ptab, pwidth, ps, trow, tstart, out) != 0) {
            fprintf(stderr, "case %d: oracle_emit_paged_packed failed\n", case_id);
            ++fails;
        }
        for (int32_t b = 0; b < R; ++b) {
            int32_t n = 0;
            for (int32_t t = 0; t < k; ++t) {
                int32_t j = want[(int64_t)b * k + t];
                if (j < 0) {
                    exp[(int64_t)b * k + t] = -1;
                } else {
                    int64_t q = (int64_t)tstart[b] + j;
                    exp[(int64_t)b * k + t] =
                        ptab[(int64_t)trow[b] * pwidth + q / ps] * ps + (int32_t)(q % ps);
                    ++n;
                }
            }
            qsort(exp + (int64_t)b * k, (size_t)n, sizeof(int32_t), cmp_i32);
        }
        expect_eq(out, exp, (int64_t)R * k, "paged_packed", case_id);
        free(ptab);
        free(trow);
        free(tstart);
        free(table);
    }
    free(scores);
    free(lens);
    free(starts);
    free(sel);
    free(want);
    free(out);
    free(exp);
    free(offs);
}

int main(void) {
    int case_id = 0;
    static const int32_t ks[5] = {1, 2, 7, 64, 300};
    static const int64_t strides[4] = {1, 5, 97, 256};
    for (int ki = 0; ki < 5; ++ki)
        for (int si = 0; si < 4; ++si)
            for (int style = 0; style < 2; ++style)
                for (int ws = 0; ws < 2; ++ws) {
                    int32_t R = 1 + below(12);
                    int32_t nthreads = 1 + (case_id % 8);
                    run_case(case_id++, R, strides[si], ks[ki], nthreads, style, ws);
                }

    /* Argument checks: a zero-row batch and rejected arguments touch nothing. */
    int32_t dummy = 0;
    if (oracle_select(NULL, 1, NULL, NULL, 0, 4, NULL, 1) != 0) ++fails;
    if (oracle_select(NULL, 1, NULL, NULL, 1, 4, NULL, 1) != 1) ++fails;
    if (oracle_select(NULL, 1, NULL, NULL, 1, 0, NULL, 1) != 1) ++fails;
    if (oracle_emit_paged(&dummy, 1, 1, &dummy, 1, 3, &dummy) != 1) ++fails;
    if (oracle_emit_paged_packed(&dummy, 1, 1, &dummy, 1, 6, NULL, NULL, &dummy) != 1) ++fails;
    int32_t neg_start = -1;
    if (oracle_emit_paged_packed(&dummy, 1, 1, &dummy, 1, 1, NULL, &neg_start, &dummy) != 2) ++fails;

    printf("%d cases, %d failures\n", case_id, fails);
    return fails ? 1 : 0;
}
