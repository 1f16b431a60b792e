/*
 * engram.h -- C ABI of libengram.so: the raw-token hashed n-gram embedding
 * (hash -> row gather -> scatter-add) on one AMD Instinct MI355X (gfx950).
 *
 * Sources the operations follow:
 *   [API] NeMo AutoModel v0.7 API page
 *         "nemo_automodel.components.models.qwen3_8_flash_next.engram"
 *   [PR1] prime-rl release notes v0.9.1.dev179, section "Validation"
 *   [PR2] prime-rl pull request 3434 "feat(models): add native Qwen3.8 Flash
 *         Next", section "Validation"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named d_* are device pointers (HIP device memory of the current
 *   device); pointers named h_* are host pointers.  The caller allocates and
 *   frees every buffer, workspace included.  The library never allocates,
 *   keeps no state between calls and is re-entrant; the one exception is
 *   engram_scatter_add_rowsparse_noalloc, whose workspace is a fixed device
 *   array of the library (see there).
 * - Host arrays are read during the call only (copied into kernel
 *   arguments); the caller may reuse them as soon as the call returns.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   work is enqueued on it and the call returns without waiting: no entry
 *   point synchronises with the host or reads device memory on the host.
 * - Arguments are checked on the host before anything is enqueued; a bad
 *   argument returns an error code and enqueues nothing.  Codes:
 *     ENGRAM_OK         success (work enqueued)
 *     ENGRAM_EINVAL     invalid argument: null required pointer, negative or
 *                       overflowing size, unsupported shape, bad constants
 *     ENGRAM_EALIGN     a device data buffer is not 16-byte aligned
 *     ENGRAM_EWORKSPACE workspace missing or smaller than the query says
 *     ENGRAM_EHIP       the HIP runtime refused a launch
 * - Device-side conditions never abort: a row id of -1 is padding (a zero
 *   row in a gather, skipped in a scatter; the exchange padding of the
 *   [API] page, _validate_padded_received_ids, uses -1 the same way); any
 *   other row id outside [0, table_rows) is treated the same way AND adds
 *   one to *d_err_count when d_err_count is not NULL (an int64 the caller
 *   zeroes; it stays on the device until the caller reads it).
 * - The sorted scatter's kernels wait on one another's published counts
 *   with bounded waits.  Blocks take their tiles in launch order (an atomic
 *   ticket), so every wait is for a block already running and ends; should
 *   one ever expire, the call adds ENGRAM_ERR_STALLED (2^40) to *d_err_count
 *   (when not NULL) instead of hanging, and its results are not valid.
 * - Layouts are row-major and contiguous.  bf16 data is passed as void*.
 * - head_dim, wherever it is taken, is at most 2^30 (the sorted scatter and
 *   its plan: at most 2048); larger values are EINVAL.
 * - A kernel launch holds at most 2^32 - 1 threads (the dispatch packet
 *   counts them in 32 bits).  The hash kernels stride over any number of
 *   tokens; a call whose other kernels would need a larger launch returns
 *   EINVAL before enqueuing anything.  That bounds engram_gather to
 *   n * head_dim <= 8 * 8,589,934,080, engram_lookup(_slice) to n lookups <=
 *   16,777,215 * r (r = 1024 / (head_dim / 8) rows, clamped to [32, 256]),
 *   and the sorted scatter (every call that plans or applies) to n <=
 *   4,294,901,504 at head_dim 40..64, 2,147,450,752 at 72..128 and
 *   1,073,725,376 above 128 (the workspace query returns (size_t)-1 there).
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_ABI_VERSION 3

#define ENGRAM_OK 0
#define ENGRAM_EINVAL (-1)
#define ENGRAM_EALIGN (-2)
#define ENGRAM_EWORKSPACE (-3)
#define ENGRAM_EHIP (-4)

/* Highest n-gram order accepted (the current token counts) and most heads. */
#define ENGRAM_MAX_NGRAM 8
#define ENGRAM_MAX_HEADS 64

/* Scatter-add modes. */
#define ENGRAM_SCATTER_SORTED 0    /* deterministic: sort + segmented sum    */
#define ENGRAM_SCATTER_ATOMIC 1    /* fp32 atomic adds (order not fixed)     */
#define ENGRAM_SCATTER_ROWSPARSE 2 /* workspace query of the row-sparse call */

/* Added to *d_err_count by the sorted scatter: a bounded wait of the plan
 * expired (its results are not valid), or an apply found no complete plan of
 * its n and table_rows in the workspace (it then wrote nothing; U = 0). */
#define ENGRAM_ERR_STALLED ((int64_t)1 << 40)
#define ENGRAM_ERR_NO_PLAN ((int64_t)1 << 41)

/* Bytes of the fixed device array engram_scatter_add_rowsparse_noalloc uses. */
#define ENGRAM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Human-readable text of a status code (static storage). */
const char *engram_status_string(int status);

/* ENGRAM_ABI_VERSION of the built library. */
int engram_abi_version(void);

/*
 * engram_hash -- global table row of every (batch, position, head).
 *
 * Follows [API] Qwen3_8_FlashNextNGramEmbedding (class description and
 * constructor arguments), _hash_input_ids and _shift_right_after_eos.
 * With n = ngram_size, J = heads_per_ngram and H = (n - 1) * J:
 *   - s_0 is the token at (b, t); for k = 1..n-1, s_k is the token k
 *     positions back if the path back to it crosses no EOS (an EOS ends the
 *     segment it closes, so the position right after an EOS starts fresh)
 *     and no change of d_seq_ids, and lies inside the row; otherwise s_k = 0;
 *   - the order-g mix, g = 2..n, is the int64 sum of s_k * multipliers[k]
 *     for k < g, every product and sum wrapping modulo 2^64;
 *   - head h = (g - 2) * J + j (bigram heads first, then trigram, ...) gets
 *     row offsets[h] + (mix mod primes[h]), the remainder taken in [0, p).
 * Arguments:
 *   d_tokens     int64 [batch, seq], raw token ids (any int64 value).
 *   d_seq_ids    int64 [batch, seq] packed segment ids, or NULL.
 *   eos_id       the EOS token id.
 *   h_multipliers int64 [ngram_size]; h_primes, h_offsets int64 [H].
 *   table_rows   rows of the table the ids address: every head must satisfy
 *                primes[h] > 0, offsets[h] >= 0, offsets[h]+primes[h] <=
 *                table_rows.
 *   d_row_ids    int64 [batch, seq, H], written.
 * Errors: EINVAL for ngram_size outside [2, ENGRAM_MAX_NGRAM],
 * heads_per_ngram < 1, H > ENGRAM_MAX_HEADS, a bad prime/offset, a null
 * pointer or a size overflow.  batch * seq == 0 enqueues nothing.
 */
int engram_hash(const int64_t *d_tokens, const int64_t *d_seq_ids,
                int64_t batch, int64_t seq, int32_t ngram_size,
                int32_t heads_per_ngram, int64_t eos_id,
                const int64_t *h_multipliers, const int64_t *h_primes,
                const int64_t *h_offsets, int64_t table_rows,
                int64_t *d_row_ids, void *stream);

/*
 * engram_hash_slice -- the rows of positions [seq_start, seq_end) of every row
 * of a complete sequence: d_row_ids[b, t - seq_start, h] equals what
 * engram_hash gives at (b, t, h) for the whole [batch, global_seq] input.
 *
 * Follows [API] Qwen3_8_FlashNextNGramEmbedding._forward_global_slice: the
 * whole replicated sequence is the input, so a context-parallel slice still
 * sees the tokens before its first position and the EOS resets there; only
 * the requested slice is computed (history is read from before seq_start).
 * Arguments as for engram_hash, with:
 *   d_tokens, d_seq_ids  int64 [batch, global_seq] (d_seq_ids may be NULL).
 *   seq_start, seq_end   the slice, 0 <= seq_start <= seq_end <= global_seq.
 *   d_row_ids            int64 [batch, seq_end - seq_start, H], written.
 * Errors: those of engram_hash, and EINVAL for a slice outside the sequence.
 * An empty slice (or batch 0) enqueues nothing.  Pass the result to
 * engram_gather for the slice's values ([batch, local, H, head_dim]), or use
 * engram_lookup_slice, which does both in one pass.
 */
int engram_hash_slice(const int64_t *d_tokens, const int64_t *d_seq_ids,
                      int64_t batch, int64_t global_seq, int64_t seq_start,
                      int64_t seq_end, int32_t ngram_size,
                      int32_t heads_per_ngram, int64_t eos_id,
                      const int64_t *h_multipliers, const int64_t *h_primes,
                      const int64_t *h_offsets, int64_t table_rows,
                      int64_t *d_row_ids, void *stream);

/*
 * engram_lookup -- the forward in one pass: the rows engram_hash gives for
 * tokens [batch, seq] are gathered straight away, without writing or reading
 * the row ids in between: d_out[b, t, h, :] = d_table[row(b, t, h), :].
 * Follows the sources of engram_hash and engram_gather (the layer's forward
 * hashes, then looks up).  Arguments as for engram_hash, with:
 *   d_table bf16 [table_rows, head_dim]; d_out bf16 [batch, seq, H, head_dim],
 *   written; head_dim a positive multiple of 8; d_table and d_out 16-byte
 *   aligned.
 *   d_row_ids int64 [batch, seq, H], or NULL: when given, the row ids are
 *   written too (the same values engram_hash writes).
 * Hashed rows always lie inside the table (every head is checked to fit), so
 * no id is invalid.  Errors: those of engram_hash and engram_gather.
 * batch * seq == 0 enqueues nothing.
 */
int engram_lookup(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                  int64_t seq, int32_t ngram_size, int32_t heads_per_ngram, int64_t eos_id,
                  const int64_t *h_multipliers, const int64_t *h_primes,
                  const int64_t *h_offsets, const void *d_table, int64_t table_rows,
                  int64_t head_dim, void *d_out, int64_t *d_row_ids, void *stream);

/*
 * engram_lookup_slice -- engram_lookup for positions [seq_start, seq_end) of
 * every row of a complete sequence: one context-parallel rank's forward in
 * one pass.  d_out[b, t - seq_start, h, :] equals what engram_lookup gives at
 * (b, t, h) for the whole [batch, global_seq] input.
 *
 * Follows [API] Qwen3_8_FlashNextNGramEmbedding._forward_global_slice (the
 * whole replicated sequence is hashed, so a slice sees the tokens before its
 * first position and the EOS resets there; only the slice's rows are looked
 * up) and the sources of engram_lookup.  Arguments as for engram_lookup,
 * with:
 *   d_tokens, d_seq_ids  int64 [batch, global_seq] (d_seq_ids may be NULL).
 *   seq_start, seq_end   the slice, 0 <= seq_start <= seq_end <= global_seq.
 *   d_out     bf16 [batch, seq_end - seq_start, H, head_dim], written.
 *   d_row_ids int64 [batch, seq_end - seq_start, H], or NULL.
 * Errors: those of engram_lookup, and EINVAL for a slice outside the
 * sequence.  An empty slice (or batch 0) enqueues nothing.
 */
int engram_lookup_slice(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                        int64_t global_seq, int64_t seq_start, int64_t seq_end,
                        int32_t ngram_size, int32_t heads_per_ngram, int64_t eos_id,
                        const int64_t *h_multipliers, const int64_t *h_primes,
                        const int64_t *h_offsets, const void *d_table, int64_t table_rows,
                        int64_t head_dim, void *d_out, int64_t *d_row_ids, void *stream);

/*
 * engram_gather -- d_out[i, :] = d_table[d_row_ids[i], :] (bitwise bf16 copy).
 *
 * Follows [API] _lookup_ngram_ids and Qwen3_8_FlashNextOwnerShardedEmbedding
 * (with no process group the full table is local and the lookup is a plain
 * embedding lookup).  For the forward of the layer, pass the hash output
 * with n = batch * seq * H: d_out [batch, seq, H, head_dim] is then the
 * page's [batch, sequence, ngram_heads * head_dim] result.
 *   d_row_ids  int64 [n]; d_table bf16 [table_rows, head_dim];
 *   d_out      bf16 [n, head_dim], written (zero rows for -1/invalid ids).
 *   head_dim   a positive multiple of 8; d_table and d_out 16-byte aligned.
 * Errors: EINVAL (null pointer with n > 0, bad head_dim, negative sizes,
 * overflow), EALIGN.  n == 0 enqueues nothing.
 */
int engram_gather(const int64_t *d_row_ids, int64_t n, const void *d_table,
                  int64_t table_rows, int64_t head_dim, void *d_out,
                  int64_t *d_err_count, void *stream);

/*
 * engram_scatter_add_workspace -- bytes of device workspace that
 * engram_scatter_add (mode ENGRAM_SCATTER_SORTED or _ATOMIC) or
 * engram_scatter_add_rowsparse (mode ENGRAM_SCATTER_ROWSPARSE) needs for n
 * ids.  0 means no workspace is needed.  Returns (size_t)-1 for arguments
 * the calls would reject.
 */
size_t engram_scatter_add_workspace(int64_t n, int64_t table_rows,
                                    int64_t head_dim, int32_t mode);

/*
 * engram_scatter_add -- backward of the gather into a dense fp32 gradient
 * table:  for every distinct valid row r among d_row_ids,
 *     d_grad_table[r, :] = fp32(d_grad_table[r, :] + S_r),
 * where S_r is the sum of the bf16 gradient rows d_grads[i, :] with
 * d_row_ids[i] == r.  Rows not referenced are left unchanged.
 *
 * Follows [API] Qwen3_8_FlashNextOwnerShardedEmbedding (the owner alone
 * accumulates a row's gradient), [PR2] Validation (backward gradient
 * aggregation per row) and [PR1] Validation (FP32 reduction defaults).
 *   mode ENGRAM_SCATTER_SORTED: S_r is summed in fp64, rounded once to fp32,
 *     then added with one fp32 add; deterministic run to run.  Needs the
 *     workspace and table_rows < 2^32 - 1, n < 2^32.  The fp64 sum is exact,
 *     and S_r then the same as a sum in any other order, as long as the bits
 *     of a row's terms and partial sums span at most 53 places (bf16 terms
 *     within a factor of about 2^45 of each other, e.g. every N(0, 1)
 *     gradient); past that a row of many terms, which the kernels sum in
 *     interleaved 16-term pieces combined in a fixed order (a short row is
 *     summed in ascending flat index), can round differently from a
 *     sequential sum, in the last bits of an fp64 sum that is then rounded
 *     to fp32; the result is still the same run to run.
 *   mode ENGRAM_SCATTER_ATOMIC: every gradient element is added to the
 *     table with an fp32 atomic add; the order of additions is not fixed.
 *     Needs no workspace.
 *   d_row_ids int64 [n]; d_grads bf16 [n, head_dim]; d_grad_table fp32
 *   [table_rows, head_dim], accumulated in place.  head_dim a positive
 *   multiple of 8, at most 2048; d_grads and d_grad_table 16-byte aligned.
 * Errors: EINVAL, EALIGN, EWORKSPACE.  n == 0 enqueues nothing.
 */
int engram_scatter_add(const int64_t *d_row_ids, int64_t n,
                       const void *d_grads, int64_t head_dim,
                       float *d_grad_table, int64_t table_rows, int32_t mode,
                       void *d_workspace, size_t workspace_bytes,
                       int64_t *d_err_count, void *stream);

/*
 * engram_scatter_add_rowsparse -- the same sums S_r, emitted row-sparse:
 * d_unique_ids[u] (ascending distinct valid rows) and d_unique_grads[u, :]
 * (fp32 S_r, summed in fp64 and rounded once) for u < U, with U written to
 * *d_num_unique.  Deterministic.  Capacity: the caller provides n entries
 * (d_unique_ids int64 [n], d_unique_grads fp32 [n, head_dim]); entries at
 * u >= U are left unchanged.  For tables whose dense fp32 gradient would not
 * fit beside the table (a 200M x 256 table needs 204.8 GB of fp32).
 *   Same limits as the sorted mode of engram_scatter_add; needs the
 *   workspace of mode ENGRAM_SCATTER_ROWSPARSE.
 * Errors: EINVAL, EALIGN, EWORKSPACE.  n == 0 writes U = 0.
 */
int engram_scatter_add_rowsparse(const int64_t *d_row_ids, int64_t n,
                                 const void *d_grads, int64_t head_dim,
                                 int64_t table_rows, int64_t *d_unique_ids,
                                 float *d_unique_grads, int64_t *d_num_unique,
                                 void *d_workspace, size_t workspace_bytes,
                                 int64_t *d_err_count, void *stream);

/*
 * engram_scatter_plan / engram_scatter_apply -- the sorted backward in two
 * steps.  The plan needs only the row ids: it sorts them and gives every
 * distinct valid row its slot, leaving the result in the workspace.  The
 * apply then computes the same sums as engram_scatter_add (sorted mode; pass
 * d_grad_table) or engram_scatter_add_rowsparse (pass the three row-sparse
 * outputs), for one bf16 gradient tensor of those ids.  Splitting them lets
 * a caller run the plan as soon as the hash is done (for example on another
 * stream, beside the forward gather) and reuse one plan for several gradient
 * tensors of the same ids.  The same semantics and citations as the
 * one-call forms apply.
 *   engram_scatter_plan: d_row_ids int64 [n]; the workspace must hold at
 *     least engram_scatter_add_workspace(n, table_rows, head_dim,
 *     ENGRAM_SCATTER_ROWSPARSE) bytes; d_err_count as elsewhere.
 *   engram_scatter_apply: the same n, head_dim, table_rows and workspace as
 *     the plan (made by either plan call), with the plan's work ordered
 *     before it (same stream, or an event).  Exactly one output form:
 *     d_grad_table (dense, accumulated), or all of d_unique_ids /
 *     d_unique_grads / d_num_unique (row-sparse).  The apply does not change
 *     the plan; it may run again on the same plan.
 *   The plan stamps the workspace with its n and table_rows when it
 *   completes, and marks it when a bounded wait expired.  The apply first
 *   checks both on the device: for a workspace that holds no complete plan of
 *   its n and table_rows it writes nothing (a row-sparse apply writes U = 0)
 *   and adds ENGRAM_ERR_NO_PLAN to *d_err_count; for a plan whose wait
 *   expired, ENGRAM_ERR_STALLED.  A complete plan of other ids of the same
 *   sizes cannot be told apart and gives those ids' sums.  Whatever the
 *   workspace holds, the apply reads and writes only inside its buffers.
 * Errors: EINVAL (sizes, output form), EALIGN, EWORKSPACE.  n == 0: the plan
 * enqueues nothing; a row-sparse apply writes U = 0.
 */
int engram_scatter_plan(const int64_t *d_row_ids, int64_t n, int64_t table_rows,
                        int64_t head_dim, void *d_workspace, size_t workspace_bytes,
                        int64_t *d_err_count, void *stream);

/*
 * engram_scatter_plan_tokens -- the plan of the row ids of tokens [batch,
 * seq], computed from the tokens: the same plan engram_scatter_plan makes
 * from engram_hash's output (n = batch * seq * H ids), without the ids being
 * written or read.  Arguments as for engram_hash (the hash) and
 * engram_scatter_plan (table_rows, head_dim, the workspace of n ids).
 * Lets the backward's plan start from the tokens alone, beside a forward
 * done with engram_lookup.  Errors: those of both calls.  Hashed rows are
 * always inside the table, so *d_err_count (when not NULL) only ever receives
 * ENGRAM_ERR_STALLED, should a bounded wait expire; the workspace is then
 * marked, and an apply of it writes nothing.
 */
int engram_scatter_plan_tokens(const int64_t *d_tokens, const int64_t *d_seq_ids,
                               int64_t batch, int64_t seq, int32_t ngram_size,
                               int32_t heads_per_ngram, int64_t eos_id,
                               const int64_t *h_multipliers, const int64_t *h_primes,
                               const int64_t *h_offsets, int64_t table_rows,
                               int64_t head_dim, void *d_workspace, size_t workspace_bytes,
                               int64_t *d_err_count, void *stream);

int engram_scatter_apply(const void *d_grads, int64_t n, int64_t head_dim,
                         int64_t table_rows, float *d_grad_table, int64_t *d_unique_ids,
                         float *d_unique_grads, int64_t *d_num_unique, void *d_workspace,
                         size_t workspace_bytes, int64_t *d_err_count, void *stream);

/*
 * engram_scatter_add_rowsparse_noalloc -- engram_scatter_add_rowsparse
 * without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same sums, outputs, limits and errors as
 * engram_scatter_add_rowsparse; the sorted path's workspace is instead a
 * fixed device array of the library of ENGRAM_NOALLOC_SCRATCH_BYTES bytes
 * (each device the library runs on holds one copy until the process ends).
 * The call allocates nothing.
 *   Size limit: n ids fit when engram_scatter_add_workspace(n, table_rows,
 *   head_dim, ENGRAM_SCATTER_ROWSPARSE) <= ENGRAM_NOALLOC_SCRATCH_BYTES
 *   (2,525,312 ids of a 200M-row table at head_dim 256); larger inputs return
 *   ENGRAM_EWORKSPACE before anything is enqueued.
 *   Every call on a device uses that device's one array, which keeps the last
 *   call's contents (each call clears what it needs cleared): calls that
 *   overlap on one device (other streams, other host threads) race and give
 *   undefined results.  Order them on one stream, or use
 *   engram_scatter_add_rowsparse with a workspace per stream.
 * Errors: those of engram_scatter_add_rowsparse (EWORKSPACE: too many ids),
 * and EHIP if the array's address cannot be found on the current device.
 */
int engram_scatter_add_rowsparse_noalloc(const int64_t *d_row_ids, int64_t n,
                                         const void *d_grads, int64_t head_dim,
                                         int64_t table_rows, int64_t *d_unique_ids,
                                         float *d_unique_grads, int64_t *d_num_unique,
                                         int64_t *d_err_count, void *stream);

/*
 * engram_signsgd_rowsparse -- one SignSGD step on the rows a row-sparse
 * gradient lists: for u < *d_num_unique (read on the device; at most
 * capacity) and r = d_unique_ids[u] in [0, table_rows), every element of
 * row r of the bf16 table becomes
 *     bf16( fp32(w) - lr * sign(d_unique_grads[u, e]) )
 * (the subtraction in fp32, sign(0) = 0, one rounding to bf16 to nearest
 * with ties to even).  Rows not listed keep their values.
 *
 * Follows [PR1] Validation and [PR2] Validation (the RL runs trained with
 * SignSGD, learning rate 1e-6, FP32 optimizer defaults); the pages give no
 * formula, and the one above is the reading taken.
 *   d_unique_ids int64 [capacity], distinct (as engram_scatter_add_rowsparse
 *   writes them; a repeated id would be updated twice, in no fixed order);
 *   d_unique_grads fp32 [capacity, head_dim]; d_num_unique int64 [1];
 *   d_table bf16 [table_rows, head_dim], updated in place.  head_dim a
 *   positive multiple of 8; d_unique_grads and d_table 16-byte aligned.
 *   Ids of -1 are skipped; other ids outside the table are skipped and
 *   counted in *d_err_count (when not NULL).
 * Errors: EINVAL, EALIGN.  capacity == 0 enqueues nothing.
 */
int engram_signsgd_rowsparse(const int64_t *d_unique_ids, const float *d_unique_grads,
                             const int64_t *d_num_unique, int64_t capacity,
                             int64_t head_dim, void *d_table, int64_t table_rows,
                             float lr, int64_t *d_err_count, void *stream);

/*
 * engram_scatter_apply_signsgd -- the backward and the SignSGD step in one
 * pass: for every distinct valid row r of the planned ids, with S_r the
 * fp32 sum engram_scatter_apply would produce (summed in fp64, rounded once),
 *     d_table[r, e] = bf16( fp32(d_table[r, e]) - lr * sign(S_r[e]) ).
 * The same result as engram_scatter_apply (row-sparse) followed by
 * engram_signsgd_rowsparse, without writing or reading the fp32 sums.
 * Citations as for those two calls.
 *   d_grads bf16 [n, head_dim]; d_table bf16 [table_rows, head_dim], updated
 *   in place; lr the learning rate; the workspace holds a plan of the n ids
 *   made by engram_scatter_plan or engram_scatter_plan_tokens (same n,
 *   head_dim and table_rows), ordered before this call, checked on the
 *   device as by engram_scatter_apply (d_err_count likewise).  d_grads and
 *   d_table 16-byte aligned.
 * Errors: EINVAL, EALIGN, EWORKSPACE.  n == 0 enqueues nothing.
 */
int engram_scatter_apply_signsgd(const void *d_grads, int64_t n, int64_t head_dim,
                                 int64_t table_rows, void *d_table, float lr,
                                 void *d_workspace, size_t workspace_bytes,
                                 int64_t *d_err_count, void *stream);

/*
 * engram_ple_conv -- the PLE causal dilated depthwise convolution with zero
 * history per packed segment:
 *     out[b, t, c] = bias[c] + sum_{k < K} w[c, k] * x[b, t - (K-1-k)*dilation, c]
 * where a tap reads 0 before the start of the row (the row starts halo_len
 * positions before x when a halo is given) and when the segment id changes
 * between the tap's position and t.  The sum is accumulated in fp32 from the
 * bias in tap order and rounded once to bf16 (nearest, ties to even).
 *
 * Follows [API] Qwen3_8_FlashNextPLELayer: _causal_short_conv (causal
 * depthwise convolution with zeros as the left history; under context
 * parallelism the preceding (K - 1) * dilation positions come from the
 * previous rank), _segmented_conv (every packed segment convolved as if it
 * began a row), conv_kernel_size (4) and short_conv_dilation (= ngram_size).
 * The tap order (F.conv1d's), fp32 accumulation and the rounding are
 * readings; the pages do not fix them.
 *   d_x bf16 [batch, seq, channels]; d_out bf16 [batch, seq, channels],
 *   written (must not overlap d_x).
 *   d_halo bf16 [batch, halo_len, channels] (the positions just before x),
 *   or NULL with halo_len 0.
 *   d_seq_ids int64 [batch, halo_len + seq] (covering the halo first), or
 *   NULL (no packed segments).
 *   d_weight bf16 [channels, kernel_size]; d_bias bf16 [channels] or NULL.
 *   channels a positive multiple of 8; kernel_size 1..16; dilation >= 1;
 *   d_x, d_halo and d_out 16-byte aligned.  kernel_size 4 with dilation up
 *   to 8 runs the tiled kernel; other shapes a plain one.
 * Errors: EINVAL, EALIGN.  batch * seq == 0 enqueues nothing.
 */
int engram_ple_conv(const void *d_x, const void *d_halo, int64_t halo_len,
                    const int64_t *d_seq_ids, const void *d_weight, const void *d_bias,
                    int64_t batch, int64_t seq, int64_t channels, int32_t kernel_size,
                    int32_t dilation, void *d_out, void *stream);

/*
 * engram_run_ops -- enqueue a list of this library's calls and stream-event
 * operations in one call, in order: what a training loop submits for one
 * step (say, the next batch's plan on a side stream, the forward on the main
 * stream, and later the apply after the plan's event), without a round trip
 * through the caller's language per call.  Each operation is exactly the
 * entry point it names, with that entry point's checks and errors; only the
 * host's per-call cost differs.  The pages count host-side round trips per
 * lookup as the cost to avoid ([API] Qwen3_8_FlashNextEngramTableConfig,
 * strict_validation); with small batches the submission of a step's kernels
 * is what sets its pace.
 *   op ENGRAM_OP_LOOKUP: engram_lookup(d_tokens, d_seq_ids, batch, seq,
 *     ngram_size, heads_per_ngram, eos_id, h_multipliers, h_primes,
 *     h_offsets, d_table, table_rows, head_dim, d_out, d_row_ids, stream).
 *   op ENGRAM_OP_PLAN_TOKENS: engram_scatter_plan_tokens(d_tokens, d_seq_ids,
 *     batch, seq, ngram_size, heads_per_ngram, eos_id, h_multipliers,
 *     h_primes, h_offsets, table_rows, head_dim, d_workspace,
 *     workspace_bytes, d_err_count, stream).
 *   op ENGRAM_OP_APPLY: engram_scatter_apply(d_grads, n, head_dim,
 *     table_rows, d_grad_table, d_unique_ids, d_unique_grads, d_num_unique,
 *     d_workspace, workspace_bytes, d_err_count, stream).
 *   op ENGRAM_OP_APPLY_SIGNSGD: engram_scatter_apply_signsgd(d_grads, n,
 *     head_dim, table_rows, d_table_rw, lr, d_workspace, workspace_bytes,
 *     d_err_count, stream).
 *   op ENGRAM_OP_RECORD: hipEventRecord(event, stream).
 *   op ENGRAM_OP_WAIT: hipStreamWaitEvent(stream, event, 0).
 *   Fields an operation does not name are ignored.  ops[0 .. count) are
 *   read during the call only; every pointer in them must stay valid as the
 *   named entry point requires (device buffers until the work completes).
 *   event is a hipEvent_t the caller created; stream a hipStream_t (NULL:
 *   the null stream).
 * Returns ENGRAM_OK when every operation was enqueued.  Otherwise the
 * status of the first operation that failed (EINVAL, EALIGN, EWORKSPACE,
 * EHIP; EINVAL also for an unknown op code, or a RECORD or WAIT without an
 * event); the operations before it stay enqueued and the later ones are
 * not.  EINVAL with nothing enqueued for count < 0, or ops NULL with
 * count > 0.  *failed_index, when failed_index is not NULL, receives the
 * index of the operation that failed, or -1 (success, or an invalid list).
 */
#define ENGRAM_OP_LOOKUP 1
#define ENGRAM_OP_PLAN_TOKENS 2
#define ENGRAM_OP_APPLY 3
#define ENGRAM_OP_APPLY_SIGNSGD 4
#define ENGRAM_OP_RECORD 5
#define ENGRAM_OP_WAIT 6

typedef struct engram_op {
  int32_t op;                 /* ENGRAM_OP_* */
  int32_t ngram_size;         /* LOOKUP, PLAN_TOKENS */
  int32_t heads_per_ngram;    /* LOOKUP, PLAN_TOKENS */
  float lr;                   /* APPLY_SIGNSGD */
  void *stream;               /* every op: the hipStream_t it is enqueued on */
  void *event;                /* RECORD, WAIT: a hipEvent_t */
  const int64_t *d_tokens;    /* LOOKUP, PLAN_TOKENS */
  const int64_t *d_seq_ids;   /* LOOKUP, PLAN_TOKENS (NULL: no segments) */
  int64_t batch, seq, eos_id; /* LOOKUP, PLAN_TOKENS */
  const int64_t *h_multipliers, *h_primes, *h_offsets; /* LOOKUP, PLAN_TOKENS (host) */
  int64_t table_rows;         /* LOOKUP, PLAN_TOKENS, APPLY, APPLY_SIGNSGD */
  int64_t head_dim;           /* LOOKUP, PLAN_TOKENS, APPLY, APPLY_SIGNSGD */
  const void *d_table;        /* LOOKUP */
  void *d_out;                /* LOOKUP */
  int64_t *d_row_ids;         /* LOOKUP (NULL: not written) */
  void *d_workspace;          /* PLAN_TOKENS, APPLY, APPLY_SIGNSGD */
  size_t workspace_bytes;
  const void *d_grads;        /* APPLY, APPLY_SIGNSGD */
  int64_t n;                  /* APPLY, APPLY_SIGNSGD */
  float *d_grad_table;        /* APPLY (dense output), or NULL */
  int64_t *d_unique_ids;      /* APPLY (row-sparse output), or NULL */
  float *d_unique_grads;
  int64_t *d_num_unique;
  void *d_table_rw;           /* APPLY_SIGNSGD: the bf16 table */
  int64_t *d_err_count;       /* PLAN_TOKENS, APPLY, APPLY_SIGNSGD (or NULL) */
} engram_op;

int engram_run_ops(const engram_op *ops, int64_t count, int64_t *failed_index);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
