/*
 * abi_sanitize.c - drives the host side of the C-ABI library built for the
 * host only (no device code) under AddressSanitizer + UndefinedBehavior-
 * Sanitizer. Built and run by tests/test_oracle_sanitized.py, on a machine
 * without a GPU.
 *
 * Every call below is rejected, or accepted as an empty batch, by the
 * argument checks before any HIP call, so no pointer handed in is ever
 * dereferenced: they are host addresses chosen only for their alignment.
 * What this checks: the checks' order and status codes, the plan-size
 * arithmetic at the extremes of num_rows, the status strings, and that none
 * of it reads or writes out of bounds or overflows.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsatopk.h"

static int fails = 0;

#define EXPECT(expr, want)                                                          \
    do {                                                                            \
        int got_ = (int)(expr);                                                     \
        if (got_ != (want)) {                                                       \
            fprintf(stderr, "line %d: %s returned %d, want %d\n", __LINE__, #expr,  \
                    got_, (int)(want));                                             \
            ++fails;                                                                \
        }                                                                           \
    } while (0)

int main(void) {
    static float scores[64] __attribute__((aligned(16)));
    static int32_t ints[64] __attribute__((aligned(16)));
    static unsigned char plan_store[4096] __attribute__((aligned(16)));
    const float* sc = scores;
    const float* sc_mis = scores + 1;   /* 4-byte aligned only */
    int32_t* out = ints;
    void* plan = plan_store;
    void* plan_mis = plan_store + 4;
    const size_t big = (size_t)1 << 40;

    /* status strings: every status has its own text, unknown ones say so */
    for (int s = DSATOPK_OK; s <= DSATOPK_ERR_TOO_LARGE; ++s) {
        const char* t = dsatopk_status_string(s);
        if (!t || !strcmp(t, "unknown status")) {
            fprintf(stderr, "status %d has no text\n", s);
            ++fails;
        }
    }
    if (strcmp(dsatopk_status_string(-1), "unknown status") ||
        strcmp(dsatopk_status_string(99), "unknown status"))
        ++fails;

    /* plan size: 0 for a negative count, grows with rows, no overflow */
    if (dsatopk_plan_bytes(-1) != 0) ++fails;
    size_t prev = 0;
    static const int32_t rows[] = {0, 1, 255, 256, 257, 4096, 262144, 1 << 30, INT32_MAX};
    for (size_t i = 0; i < sizeof(rows) / sizeof(rows[0]); ++i) {
        size_t b = dsatopk_plan_bytes(rows[i]);
        if (b < prev || b % 16 != 0) {
            fprintf(stderr, "plan_bytes(%d) = %zu after %zu\n", rows[i], b, prev);
            ++fails;
        }
        prev = b;
    }

    /* dsatopk_plan: argument checks */
    EXPECT(dsatopk_plan(ints, NULL, -1, 8, plan, big, NULL), DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan(ints, NULL, 4, 0, plan, big, NULL), DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan(ints, NULL, 4, DSATOPK_MAX_K + 1, plan, big, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan(NULL, NULL, 0, 8, NULL, 0, NULL), DSATOPK_OK);
    EXPECT(dsatopk_plan(NULL, NULL, 4, 8, plan, big, NULL), DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan(ints, NULL, 4, 8, NULL, big, NULL), DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan(ints, NULL, 4, 8, plan, dsatopk_plan_bytes(4) - 1, NULL),
           DSATOPK_ERR_PLAN_TOO_SMALL);
    EXPECT(dsatopk_plan(ints, NULL, 4, 8, plan_mis, big, NULL), DSATOPK_ERR_ALIGNMENT);

    /* dsatopk_plan_error: argument checks */
    int32_t err = 0;
    EXPECT(dsatopk_plan_error(NULL, big, &err, NULL), DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan_error(plan, big, NULL, NULL), DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_plan_error(plan, 4, &err, NULL), DSATOPK_ERR_PLAN_TOO_SMALL);

    /* dsatopk_paged */
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, 0, 8, NULL, 0, out, NULL), DSATOPK_OK);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, -1, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, 2, 0, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, 2, DSATOPK_MAX_K + 1, NULL, 0, out,
                         NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(NULL, 64, ints, NULL, ints, 4, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, NULL, NULL, ints, 4, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, 2, 8, NULL, 0, NULL, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 0, ints, NULL, ints, 4, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc_mis, 64, ints, NULL, ints, 4, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_ALIGNMENT);
    EXPECT(dsatopk_paged(sc, 62, ints, NULL, ints, 4, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_ALIGNMENT);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, 2, 8, plan_mis, big, out, NULL),
           DSATOPK_ERR_ALIGNMENT);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 64, 2, 8, plan, dsatopk_plan_bytes(2) - 16,
                         out, NULL),
           DSATOPK_ERR_PLAN_TOO_SMALL);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, NULL, 4, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 0, 64, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 48, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 0, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged(sc, 64, ints, NULL, ints, 4, 1 << 21, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);

    /* dsatopk_paged_packed: the same checks, then table arguments are optional */
    EXPECT(dsatopk_paged_packed(sc, 64, ints, NULL, ints, 4, 3, ints, ints, 2, 8, NULL, 0, out,
                                out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged_packed(sc, 64, ints, NULL, ints, 4, 64, ints, ints, 0, 8, NULL, 0, out,
                                out, NULL),
           DSATOPK_OK);

    /* dsatopk_ragged */
    EXPECT(dsatopk_ragged(sc, 64, ints, NULL, ints, 0, 8, NULL, 0, out, NULL), DSATOPK_OK);
    EXPECT(dsatopk_ragged(sc, 64, ints, NULL, NULL, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_ragged(sc, 64, ints, NULL, ints, 2, 0, NULL, 0, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_ragged(sc_mis, 64, ints, NULL, ints, 2, 8, NULL, 0, out, NULL),
           DSATOPK_ERR_ALIGNMENT);
    EXPECT(dsatopk_ragged(sc, 64, ints, NULL, ints, 2, 8, plan, 16, out, NULL),
           DSATOPK_ERR_PLAN_TOO_SMALL);

    /* dsatopk_paged_noalloc: the size limit comes first */
    EXPECT(dsatopk_paged_noalloc(sc, 64, ints, NULL, ints, 4, 64, DSATOPK_NOALLOC_MAX_ROWS + 1,
                                 8, out, NULL),
           DSATOPK_ERR_TOO_LARGE);
    EXPECT(dsatopk_paged_noalloc(sc, 64, ints, NULL, ints, 4, 64, 0, 8, out, NULL), DSATOPK_OK);
    EXPECT(dsatopk_paged_noalloc(sc, 64, ints, NULL, ints, 4, 5, 2, 8, out, NULL),
           DSATOPK_ERR_INVALID_ARG);
    EXPECT(dsatopk_paged_noalloc(sc_mis, 64, ints, NULL, ints, 4, 64, 2, 8, out, NULL),
           DSATOPK_ERR_ALIGNMENT);

    printf("%d failures\n", fails);
    return fails ? 1 : 0;
}
