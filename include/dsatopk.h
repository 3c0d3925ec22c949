/*
 * dsatopk.h - C ABI of the dsatopk library: per-row windowed top-k selection
 * over fp32 indexer scores with a fused RAGGED or PAGED emit, for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (DeepSeek-V4 DSA indexer top-k transform, as described in
 * the sglang PR digests on prhub.com.cn):
 *
 *   For each row b, with L = max(seq_lens[b], 0) and s = row_starts[b]
 *   (0 when row_starts is NULL), select the k largest scores among
 *   scores[b * score_stride + s + j] for window positions j in [0, L).
 *   Equal scores (IEEE ==, so -0.0 equals +0.0) are ordered by lower
 *   position first. Rows with L <= k select every position 0 .. L-1 and do
 *   not read their scores. Each selected position j is emitted as
 *     RAGGED: j + out_offsets[b]
 *     PAGED:  page_table[b * page_table_stride + j / page_size] * page_size
 *             + j % page_size
 *   into row b of out ([num_rows, k] int32). The first min(k, L) slots of a
 *   row hold the selection in an unspecified order; slots min(k, L) .. k-1
 *   hold -1.
 *   Sources: PR #35175 digest ("RAGGED prefill top-k moved to the v2 JIT
 *   kernel"), section "Key source excerpts": topk_ragged_kernel (window,
 *   trivial path, -1 padding, output = position + out_offsets[b]) and
 *   TopKProblem (emit adds the bias; transform_output maps through the page
 *   table with page_bits = log2(page_size)). PR #26788 digest ("faster top-k
 *   + page-table transform (runtime k <= 2048)"), "Key source excerpts":
 *   plan_topk_v2 / topk_transform_512_v2 signatures, runtime k.
 *
 * Conventions for every call below:
 *   - Pointers named scores, seq_lens, row_starts, out_offsets, page_table,
 *     plan and out are DEVICE pointers. `stream` is a hipStream_t (NULL is
 *     the default stream).
 *   - Calls are asynchronous on `stream`, allocate nothing, never
 *     synchronize the host, and only launch kernels (no memset or copy
 *     nodes), so they may be captured in a HIP graph.
 *   - The caller owns every buffer. `scores` is only read; it is never
 *     written, not even outside the window.
 *   - Host-checkable preconditions are checked before anything is launched;
 *     on error nothing is written and a status other than DSATOPK_OK is
 *     returned. No call aborts or throws.
 *   - The library holds no global state and is safe to call from several
 *     host threads.
 */
#ifndef DSATOPK_H_
#define DSATOPK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (every call returns one of these as an int). */
enum {
    DSATOPK_OK = 0,
    /* k outside [1, DSATOPK_MAX_K]; num_rows < 0; a required pointer is NULL;
       score_stride < 1; page_size not a power of two in [1, 2^20];
       page_table_stride < 1. */
    DSATOPK_ERR_INVALID_ARG = 1,
    /* scores or plan not 16-byte aligned, or score_stride not a multiple of 4. */
    DSATOPK_ERR_ALIGNMENT = 2,
    /* plan_bytes smaller than dsatopk_plan_bytes(num_rows). */
    DSATOPK_ERR_PLAN_TOO_SMALL = 3,
    /* the HIP runtime reported an error (no device, launch failure). */
    DSATOPK_ERR_HIP = 4,
    /* dsatopk_paged_noalloc: num_rows above DSATOPK_NOALLOC_MAX_ROWS. */
    DSATOPK_ERR_TOO_LARGE = 5
};

/* Largest k (runtime value; one build serves every k). The pages bound the
   v2 kernel to 0 < topk <= 2048 (PR #35175 digest, backend dispatch
   condition; PR #26788 digest title). */
#define DSATOPK_MAX_K 2048

/* Longest supported window. Longer windows are a device-side precondition
   violation (see dsatopk_paged). */
#define DSATOPK_MAX_SEQ_LEN 131072

/* Human-readable name of a status code (static string, never NULL). */
const char* dsatopk_status_string(int status);

/* Size in bytes of the plan buffer for `num_rows` rows (0 if num_rows < 0). */
size_t dsatopk_plan_bytes(int32_t num_rows);

/*
 * dsatopk_plan - build the device-side schedule for a batch.
 *
 * Reads seq_lens[num_rows] and row_starts[num_rows] (int32, device;
 * row_starts may be NULL, meaning every window starts at column 0) and
 * writes the plan buffer (device, plan_bytes >= dsatopk_plan_bytes(num_rows),
 * 16-byte aligned): each row's length class (trivial or up to 8192 aligned
 * floats, up to 16384, up to 32768, longer) with the rows of each class
 * listed, and, when the batch has at most 256 rows longer than 32768, a cut
 * of each of them into segments of 8192 floats (4096 when that would give
 * fewer segments than the GPU's 256 CUs), served by one workgroup each,
 * with a zeroed exchange area per row through which the segments merge
 * their histograms. Longer rows of batches with more of them are read
 * whole by one workgroup each. Everything is computed on the device;
 * nothing is read back. The transform calls read the split schedule, and
 * in batches of up to 1024 rows at score strides above 40960 floats the
 * class lists, whose order (longest class first) sets which rows start
 * first; rows go to their kernel by their own length.
 *
 * The plan only schedules: a call given a plan built from different
 * seq_lens / row_starts / k, or no plan at all (NULL), returns the same
 * outputs (every kernel recomputes each row's class and segment count, and
 * a long row that does not match its planned segments is read whole). A
 * plan must come from a dsatopk_plan call with the same num_rows. A plan
 * may be reused by any number of later transform calls (one per layer,
 * say): each call leaves the exchange areas and its work counters zeroed
 * again. Calls that share one plan must not run concurrently.
 *
 * Split rows wait for each other with bounded polls. A wait that gives up
 * (which a correct launch never sees: it takes a segment that cannot run
 * for about a second) sets the plan's error word (dsatopk_plan_error) and
 * leaves that row's outputs all -1 instead of a partial selection; build
 * the plan again before its next use. Plan word 15 (the int32 at byte
 * offset 60) holds the number of polls after which such a wait gives up;
 * dsatopk_plan writes 0, meaning about 2^20. It is exposed for tests that
 * force a wait to give up.
 *
 * Source: PR #26788 digest, "Key source excerpts", plan_topk_v2 (a device
 * plan built from seq_lens and reused by the transform); the layout here is
 * this library's own.
 *
 * Errors: DSATOPK_ERR_INVALID_ARG (num_rows < 0, k outside [1, 2048],
 * NULL seq_lens or plan with num_rows > 0), DSATOPK_ERR_ALIGNMENT (plan not
 * 16-byte aligned), DSATOPK_ERR_PLAN_TOO_SMALL, DSATOPK_ERR_HIP (a launch
 * failed; its own status is checked, not an earlier one).
 * num_rows == 0 is a no-op.
 */
int dsatopk_plan(const int32_t* seq_lens, const int32_t* row_starts, int32_t num_rows, int32_t k,
                 void* plan, size_t plan_bytes, void* stream);

/*
 * dsatopk_plan_error - read a plan's error word.
 *
 * Copies the plan's error word into *error (host memory) after the work
 * already queued on `stream` and synchronizes `stream`: 0 when no split-row
 * wait of the transform calls since the plan was built gave up, 1 when one
 * did (those rows' outputs are all -1; see dsatopk_plan). Unlike the other
 * calls this one waits for the device and must not be captured in a graph.
 * plan is a device pointer from dsatopk_plan, plan_bytes its size.
 *
 * Errors: DSATOPK_ERR_INVALID_ARG (NULL plan or error),
 * DSATOPK_ERR_PLAN_TOO_SMALL (plan_bytes below the 256-byte header),
 * DSATOPK_ERR_HIP (the copy or the synchronization failed).
 */
int dsatopk_plan_error(const void* plan, size_t plan_bytes, int32_t* error, void* stream);

/*
 * dsatopk_paged - top-k with the PAGED emit.
 *
 * Source: PR #26788 digest ("faster top-k + page-table transform (runtime
 * k <= 2048)"), "Key source excerpts": topk_transform_512_v2 takes the
 * scores, seq_lens, the page tables, page_size and the plan and writes the
 * page-mapped indices; PR #35175 digest, TopKProblem::transform_output (the
 * map page_table[j >> page_bits] << page_bits | (j & (page_size - 1)), and
 * -1 for padding).
 *
 *   scores            fp32 [num_rows, score_stride], row-major, 16-B aligned
 *                     base, score_stride % 4 == 0. Read only.
 *   seq_lens          int32 [num_rows]; negative values are read as 0.
 *   row_starts        int32 [num_rows] or NULL (every window starts at
 *                     column 0). Any residue modulo 4 is allowed.
 *   page_table        int32 [num_rows, page_table_stride]; entry
 *                     j / page_size of row b is the physical page of window
 *                     position j.
 *   page_size         power of two in [1, 2^20].
 *   num_rows, k       0 <= num_rows; 1 <= k <= 2048.
 *   plan, plan_bytes  from dsatopk_plan, or NULL / 0. Its exchange areas are
 *                     written during the call and left zeroed.
 *   out               int32 [num_rows, k], written (all of it).
 *
 * Device-side preconditions (not checkable without reading device memory,
 * so not checked): 0 <= row_starts[b]; row_starts[b] + seq_len_b <=
 * score_stride; seq_len_b <= 131072; page_table_stride >= ceil(seq_len_b /
 * page_size); every emitted value < 2^31. NaN scores are outside the
 * contract (the selection stays inside the window, but which NaNs are
 * picked is unspecified).
 *
 * Errors: DSATOPK_ERR_INVALID_ARG, DSATOPK_ERR_ALIGNMENT,
 * DSATOPK_ERR_PLAN_TOO_SMALL, DSATOPK_ERR_HIP. num_rows == 0 is a no-op.
 */
int dsatopk_paged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                  const int32_t* row_starts, const int32_t* page_table,
                  int64_t page_table_stride, int32_t page_size, int32_t num_rows, int32_t k,
                  void* plan, size_t plan_bytes, int32_t* out, void* stream);

/*
 * dsatopk_paged_packed - dsatopk_paged for packed rows, with raw positions
 * beside the paged ones.
 *
 * Packed rows: query rows of one request share that request's page-table
 * row, while their score windows sit at batch-wide columns of the score
 * buffer (sglang/FlashInfer packed PAGED digest, "fix(dsa): use FlashInfer
 * fused top-k for packed PAGED rows": the page table's start for a row is
 * its score window start minus the request's KV start, and a row-to-batch
 * map picks the table row). Raw positions: the transform's optional raw
 * index output (PR #26788 digest, out_raw_indices).
 *
 * Arguments as for dsatopk_paged, plus:
 *   table_rows    int32 [num_rows] (device) or NULL: row b reads page-table
 *                 row table_rows[b] (row b when NULL). The page table may
 *                 then hold fewer rows than num_rows.
 *   table_starts  int32 [num_rows] (device) or NULL: window position j of
 *                 row b is table position table_starts[b] + j (j when
 *                 NULL); out = table[q / page_size] * page_size +
 *                 q % page_size with q that table position.
 *   out_raw       int32 [num_rows, k] or NULL: when given, also written
 *                 (all of it) with the selected window positions j, slot
 *                 for slot with out, and -1 where out holds -1.
 *
 * With table_rows, table_starts and out_raw all NULL this is dsatopk_paged.
 * Device-side preconditions (not checked): table_rows[b] names a row of the
 * page table; 0 <= table_starts[b]; the row's table positions
 * table_starts[b] .. table_starts[b] + seq_len_b - 1 lie inside that row
 * (page_table_stride >= ceil((table_starts[b] + seq_len_b) / page_size)).
 *
 * Errors: as dsatopk_paged.
 */
int dsatopk_paged_packed(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                         const int32_t* row_starts, const int32_t* page_table,
                         int64_t page_table_stride, int32_t page_size,
                         const int32_t* table_rows, const int32_t* table_starts,
                         int32_t num_rows, int32_t k, void* plan, size_t plan_bytes,
                         int32_t* out, int32_t* out_raw, void* stream);

/*
 * dsatopk_ragged - top-k with the RAGGED emit: out = j + out_offsets[b].
 *
 * Arguments as for dsatopk_paged, with out_offsets int32 [num_rows]
 * (device) in place of the page table. With out_offsets == row_starts the
 * outputs are absolute columns of the score row (PR #35175 digest,
 * "Impact": the output is then the token's position in the flattened KV).
 *
 * Errors: as dsatopk_paged.
 */
int dsatopk_ragged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                   const int32_t* row_starts, const int32_t* out_offsets, int32_t num_rows,
                   int32_t k, void* plan, size_t plan_bytes, int32_t* out, void* stream);

/* Largest batch of dsatopk_paged_noalloc (its plan fits 16 MiB). */
#define DSATOPK_NOALLOC_MAX_ROWS 262144

/*
 * dsatopk_paged_noalloc - dsatopk_paged with its plan in the library's own
 * static device memory, for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments as for dsatopk_paged, without the plan: each call builds the
 * batch's plan (dsatopk_plan) in a 16 MiB device array of the library, then
 * runs the PAGED transform with it. Nothing is allocated or freed, by this
 * call or by anything it calls; the caller passes the inputs and out.
 *
 * The array is one per GPU, held by every GPU the library runs on until the
 * process ends, and shared by every call on that GPU: calls that overlap on
 * one GPU (several streams or host threads at once) race on it and must be
 * ordered by the caller. Each call writes the parts of the plan that must
 * start at zero itself. The first call on a device looks the array's
 * address up (hipGetSymbolAddress) with that device current; later calls
 * reuse it.
 *
 * Errors: DSATOPK_ERR_TOO_LARGE (num_rows > DSATOPK_NOALLOC_MAX_ROWS,
 * returned before any HIP call), then as dsatopk_paged. num_rows == 0 is a
 * no-op.
 */
int dsatopk_paged_noalloc(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                          const int32_t* row_starts, const int32_t* page_table,
                          int64_t page_table_stride, int32_t page_size, int32_t num_rows,
                          int32_t k, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSATOPK_H_ */
