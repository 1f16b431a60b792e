/*
 * engram_oracle.c -- plain CPU oracle for the raw-token hashed n-gram
 * embedding (hash -> gather -> scatter-add).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no code, header, table or constant with the HIP path and includes
 * nothing from it.  It is deliberately slow and literal: one token, one head,
 * one element at a time, in the order the pages describe.
 *
 * Sources (the pages this follows; see the citations on each function):
 *   [API]  NeMo AutoModel v0.7 API page
 *          "nemo_automodel.components.models.qwen3_8_flash_next.engram"
 *   [PR1]  prime-rl release notes v0.9.1.dev179 (section "Validation")
 *   [PR2]  prime-rl pull request 3434 "feat(models): add native Qwen3.8 Flash
 *          Next" (section "Validation")
 *
 * Readings where the pages are silent or cut off (each one is a documented
 * choice, and the HIP path implements the same choice independently):
 *   - the n tokens of an order are combined by a wrapping int64 SUM of the
 *     products token * multiplier (the combining operation is not stated);
 *   - the multiplier with index k multiplies the token k positions back
 *     (k = 0 is the current token); order g uses multipliers 0..g-1;
 *   - a history position with no valid token reads FILL = 0;
 *   - an EOS belongs to the segment it ends: the EOS position keeps its own
 *     history, the position after it starts fresh;
 *   - backward: each unique row's contributions are summed in fp64 in
 *     ascending flat index, rounded once to fp32, then added to the fp32
 *     gradient row with one fp32 add;
 *   - optimizer step (SignSGD on the touched rows): fp32(w) - lr * sign(g)
 *     in fp32, rounded once to bf16 (nearest, ties to even), sign(0) = 0.
 *
 * Parity status: every function here is pinned by CPU tests (brute force
 * over exhaustive tiny inputs with an independent big-integer formulation,
 * closed-form unit-multiplier cases written from the pages' EOS and segment
 * rules, degenerate cases, and library routines for gather, scatter and
 * the SignSGD step's fp32 -> bf16 rounding).
 * Parity with the released checkpoint's hash is unpinned: the pages do not
 * fix the combining operation or the fill value, and no checkpoint is here.
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC engram_oracle.c -o libengram_oracle.so
 * The same source built with -fopenmp (the benchmark's all-core CPU
 * baseline) spreads the independent work over threads: tokens of the hash,
 * lookups of the gather, distinct rows of the scatter-add (each row still
 * summed by one thread in ascending flat index, so every result is the same
 * bit for bit).  Without -fopenmp the pragmas are empty and it is serial.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#define ORACLE_FOR_ROWS _Pragma("omp parallel for schedule(dynamic, 1024)")
#define ORACLE_FOR_COUNT _Pragma("omp parallel for schedule(static) reduction(+ : bad)")
#define ORACLE_PARALLEL_FOR _Pragma("omp parallel for schedule(static)")
#else
#define ORACLE_FOR_ROWS
#define ORACLE_FOR_COUNT
#define ORACLE_PARALLEL_FOR
#endif

/* Threads the parallel loops use (1 in a serial build). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Index of the calling thread in [0, oracle_threads()). */
static int oracle_thread(void)
{
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

#define ORACLE_FILL 0
#define ORACLE_MAX_ORDER 8

/* ---------------------------------------------------------------------- */
/* Two's-complement int64 arithmetic without undefined behaviour.  The     */
/* hash relies on signed int64 overflow on purpose ([API],                 */
/* Qwen3_8_FlashNextNGramEmbedding, class description): products and sums  */
/* wrap modulo 2^64.  C leaves signed overflow undefined, so the wrap is   */
/* done on uint64_t and the bits are reinterpreted.                        */
/* ---------------------------------------------------------------------- */
static int64_t bits_to_i64(uint64_t u)
{
    int64_t s;
    memcpy(&s, &u, sizeof s);
    return s;
}

static int64_t wrapping_mul(int64_t a, int64_t b)
{
    return bits_to_i64((uint64_t)a * (uint64_t)b);
}

static int64_t wrapping_add(int64_t a, int64_t b)
{
    return bits_to_i64((uint64_t)a + (uint64_t)b);
}

/* Remainders are taken non-negative ([API], class description): the floor
 * remainder, in [0, p) for p > 0.  C's % truncates toward zero, so a
 * negative result is moved up by p. */
static int64_t positive_remainder(int64_t x, int64_t p)
{
    int64_t r = x % p;
    if (r < 0)
        r += p;
    return r;
}

/* ---------------------------------------------------------------------- */
/* History read ([API], _shift_right_after_eos): an earlier token is only  */
/* read if the way back to it passes no EOS and no packed-segment border.  */
/* Walks back from position t one step at a time.  Stepping from j+1 to j  */
/* crosses a boundary when tok[j] is EOS (an EOS closes the segment before */
/* it, [API] constructor argument eos_token_id, so the position after it   */
/* starts fresh) or when the packed segment IDs of j and j+1 differ (a     */
/* token's history never leaves its own segment, [API] _hash_input_ids,    */
/* argument sequence_ids).  Running off the start of the row also has no   */
/* valid token.  A missing token reads FILL.                               */
/* ---------------------------------------------------------------------- */
static int64_t earlier_token(const int64_t *tok, const int64_t *seg, int64_t t,
                             int shift, int64_t eos_id)
{
    for (int64_t j = t - 1; j >= t - shift; --j) {
        if (j < 0)
            return ORACLE_FILL;
        if (tok[j] == eos_id)
            return ORACLE_FILL;
        if (seg != NULL && seg[j] != seg[j + 1])
            return ORACLE_FILL;
    }
    return tok[t - shift];
}

/* ---------------------------------------------------------------------- */
/* Hash: global row of every (batch, position, head).                      */
/* [API] Qwen3_8_FlashNextNGramEmbedding (class description, constructor   */
/* arguments) and _hash_input_ids: heads come in groups of heads_per_ngram,*/
/* bigrams first, then trigrams, ...; each head reduces its order's mix    */
/* modulo its own prime and adds its own packed-table offset.              */
/* Output layout [batch, seq, H], H = (ngram_size - 1) * heads_per_ngram,  */
/* head index h = (g - 2) * heads_per_ngram + j for order g and member j.  */
/* Returns 0, or -1 on an invalid argument.                                */
/* ---------------------------------------------------------------------- */
int oracle_hash(const int64_t *tokens, const int64_t *seq_ids,
                int64_t batch, int64_t seq, int ngram_size, int heads_per_ngram,
                int64_t eos_id, const int64_t *multipliers,
                const int64_t *primes, const int64_t *offsets,
                int64_t *row_ids)
{
    if (ngram_size < 2 || ngram_size > ORACLE_MAX_ORDER || heads_per_ngram < 1)
        return -1;
    const int64_t H = (int64_t)(ngram_size - 1) * heads_per_ngram;
    for (int64_t h = 0; h < H; ++h)
        if (primes[h] <= 0)
            return -1;

    /* one (b, t) after another: position f = b * seq + t */
    ORACLE_PARALLEL_FOR
    for (int64_t f = 0; f < batch * seq; ++f) {
        const int64_t b = f / seq, t = f % seq;
        const int64_t *tok = tokens + b * seq;
        const int64_t *seg = seq_ids ? seq_ids + b * seq : NULL;
        /* window[k] = token k positions back (k = 0: current token) */
        int64_t window[ORACLE_MAX_ORDER];
        window[0] = tok[t];
        for (int k = 1; k < ngram_size; ++k)
            window[k] = earlier_token(tok, seg, t, k, eos_id);

        for (int g = 2; g <= ngram_size; ++g) {
            /* order-g mix: wrapping sum over k < g of window[k] * m[k] */
            int64_t mix = 0;
            for (int k = 0; k < g; ++k)
                mix = wrapping_add(mix, wrapping_mul(window[k], multipliers[k]));
            for (int j = 0; j < heads_per_ngram; ++j) {
                const int64_t h = (int64_t)(g - 2) * heads_per_ngram + j;
                row_ids[f * H + h] = offsets[h] + positive_remainder(mix, primes[h]);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Gather: out[i, :] = table[row_ids[i], :], a bitwise copy of bf16 rows   */
/* (held here as uint16 bit patterns).  [API] _lookup_ngram_ids and        */
/* Qwen3_8_FlashNextOwnerShardedEmbedding: with no process group the       */
/* complete table is local and the lookup is a plain embedding lookup.     */
/* Row -1 is padding ([API] _validate_padded_received_ids: -1 rows are     */
/* legitimate sender padding) and reads a zero row; any other row outside  */
/* [0, table_rows) also reads a zero row and is counted.                   */
/* Returns the number of such invalid rows.                                */
/* ---------------------------------------------------------------------- */
int64_t oracle_gather(const int64_t *row_ids, int64_t n, const uint16_t *table,
                      int64_t table_rows, int64_t dim, uint16_t *out)
{
    int64_t bad = 0;
    ORACLE_FOR_COUNT
    for (int64_t i = 0; i < n; ++i) {
        const int64_t r = row_ids[i];
        uint16_t *dst = out + i * dim;
        if (r >= 0 && r < table_rows) {
            const uint16_t *src = table + r * dim;
            for (int64_t e = 0; e < dim; ++e)
                dst[e] = src[e];
        } else {
            for (int64_t e = 0; e < dim; ++e)
                dst[e] = 0;
            if (r != -1)
                ++bad;
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------- */
/* Scatter-add (backward of the lookup).                                   */
/* [API] Qwen3_8_FlashNextOwnerShardedEmbedding: the owner alone           */
/* accumulates a row's gradient; [PR2] Validation: backward aggregates     */
/* gradients per row; [PR1] Validation: FP32 reduction defaults.           */
/* For every unique row r among the valid IDs,                             */
/*     S_r = sum over i with row_ids[i] == r, in ascending i, of grad[i],  */
/* accumulated in fp64 (bf16 -> fp64 is exact) and rounded once to fp32.   */
/* Finding the groups uses qsort (a library sort) on (row, i) pairs.       */
/* ---------------------------------------------------------------------- */
typedef struct {
    int64_t row;
    int64_t idx;
} row_ref;

static int compare_row_ref(const void *pa, const void *pb)
{
    const row_ref *a = (const row_ref *)pa;
    const row_ref *b = (const row_ref *)pb;
    if (a->row != b->row)
        return a->row < b->row ? -1 : 1;
    if (a->idx != b->idx)
        return a->idx < b->idx ? -1 : 1;
    return 0;
}

static float bf16_bits_to_float(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Sorted (row, idx) list of the valid IDs; *count receives its length and
 * *bad the number of invalid non-padding IDs.  Caller frees the list. */
static row_ref *sorted_refs(const int64_t *row_ids, int64_t n, int64_t table_rows,
                            int64_t *count, int64_t *bad)
{
    row_ref *refs = (row_ref *)malloc((size_t)(n > 0 ? n : 1) * sizeof(row_ref));
    int64_t m = 0;
    *bad = 0;
    if (refs == NULL)
        return NULL;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t r = row_ids[i];
        if (r >= 0 && r < table_rows) {
            refs[m].row = r;
            refs[m].idx = i;
            ++m;
        } else if (r != -1) {
            ++*bad;
        }
    }
    qsort(refs, (size_t)m, sizeof(row_ref), compare_row_ref);
    *count = m;
    return refs;
}

/* Start of every group of equal rows in the sorted list refs[0, m), and
 * m after the last: starts[0 .. *groups].  Caller frees the list. */
static int64_t *group_starts(const row_ref *refs, int64_t m, int64_t *groups)
{
    int64_t *starts = (int64_t *)malloc((size_t)(m + 1) * sizeof(int64_t));
    int64_t g = 0;
    if (starts == NULL)
        return NULL;
    for (int64_t q = 0; q < m; ++q)
        if (q == 0 || refs[q].row != refs[q - 1].row)
            starts[g++] = q;
    starts[g] = m;
    *groups = g;
    return starts;
}

/* Sum of one group refs[begin, end) (all the same row) into acc[dim]. */
static void sum_group(const row_ref *refs, int64_t begin, int64_t end,
                      const uint16_t *grads, int64_t dim, double *acc)
{
    for (int64_t e = 0; e < dim; ++e)
        acc[e] = 0.0;
    for (int64_t q = begin; q < end; ++q) {
        const uint16_t *g = grads + refs[q].idx * dim;
        for (int64_t e = 0; e < dim; ++e)
            acc[e] += (double)bf16_bits_to_float(g[e]);
    }
}

/* Dense form: grad_table[r, :] = fp32(grad_table[r, :] + fp32(S_r)).
 * Rows not referenced are left untouched.  Returns the invalid-ID count,
 * or -1 if memory ran out. */
int64_t oracle_scatter_add_dense(const int64_t *row_ids, int64_t n,
                                 const uint16_t *grads, int64_t dim,
                                 float *grad_table, int64_t table_rows)
{
    int64_t m = 0, bad = 0, groups = 0;
    row_ref *refs = sorted_refs(row_ids, n, table_rows, &m, &bad);
    int64_t *starts = refs ? group_starts(refs, m, &groups) : NULL;
    /* one fp64 accumulator row per thread */
    double *accs = (double *)malloc((size_t)oracle_threads() * (size_t)(dim > 0 ? dim : 1) *
                                    sizeof(double));
    const int failed = refs == NULL || starts == NULL || accs == NULL;
    if (!failed) {
        ORACLE_FOR_ROWS
        for (int64_t g = 0; g < groups; ++g) {
            double *acc = accs + (int64_t)oracle_thread() * dim;
            sum_group(refs, starts[g], starts[g + 1], grads, dim, acc);
            float *dst = grad_table + refs[starts[g]].row * dim;
            for (int64_t e = 0; e < dim; ++e) {
                const float s = (float)acc[e];
                dst[e] = dst[e] + s;
            }
        }
    }
    free(accs);
    free(starts);
    free(refs);
    return failed ? -1 : bad;
}

/* Row-sparse form: the unique rows in ascending order with their fp32 sums:
 * unique_ids[u], unique_grads[u, :] for u < *num_unique.  Returns the
 * invalid-ID count, or -1 if memory ran out. */
int64_t oracle_scatter_add_rowsparse(const int64_t *row_ids, int64_t n,
                                     const uint16_t *grads, int64_t dim,
                                     int64_t table_rows, int64_t *unique_ids,
                                     float *unique_grads, int64_t *num_unique)
{
    int64_t m = 0, bad = 0, groups = 0;
    row_ref *refs = sorted_refs(row_ids, n, table_rows, &m, &bad);
    int64_t *starts = refs ? group_starts(refs, m, &groups) : NULL;
    /* one fp64 accumulator row per thread */
    double *accs = (double *)malloc((size_t)oracle_threads() * (size_t)(dim > 0 ? dim : 1) *
                                    sizeof(double));
    const int failed = refs == NULL || starts == NULL || accs == NULL;
    if (!failed) {
        /* group u is the u-th distinct row in ascending order */
        ORACLE_FOR_ROWS
        for (int64_t u = 0; u < groups; ++u) {
            double *acc = accs + (int64_t)oracle_thread() * dim;
            sum_group(refs, starts[u], starts[u + 1], grads, dim, acc);
            unique_ids[u] = refs[starts[u]].row;
            for (int64_t e = 0; e < dim; ++e)
                unique_grads[u * dim + e] = (float)acc[e];
        }
        *num_unique = groups;
    }
    free(accs);
    free(starts);
    free(refs);
    return failed ? -1 : bad;
}

/* ---------------------------------------------------------------------- */
/* Row-sparse SignSGD step into the bf16 table.  The RL runs on the pages  */
/* trained with SignSGD at learning rate 1e-6 and the default FP32         */
/* optimizer math ([PR1] Validation; [PR2] Validation).  Reading (the      */
/* pages give no formula): for every listed row r with gradient sum S_r    */
/* (fp32, the row-sparse backward's output), every element becomes         */
/*     w <- bf16( fp32(w) - lr * sign(S_r[e]) )                            */
/* with the subtraction in fp32, sign(0) = 0, and one rounding to bf16,    */
/* to nearest with ties to even.  Rows not listed keep their values.       */
/* The listed ids are taken one after another; ids outside [0, rows) are  */
/* skipped and counted (the return value).                                 */
/* ---------------------------------------------------------------------- */
static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          /* NaN stays a quiet NaN */
    /* round to nearest, ties to even: add just under half of the dropped
     * range, plus one when the kept part is odd, then truncate */
    const uint32_t keep_odd = (u >> 16) & 1u;
    u += 0x7fffu + keep_odd;
    return (uint16_t)(u >> 16);
}

int64_t oracle_signsgd_rowsparse(const int64_t *unique_ids, const float *unique_grads,
                                 int64_t count, int64_t dim, uint16_t *table,
                                 int64_t table_rows, float lr)
{
    int64_t bad = 0;
    for (int64_t u = 0; u < count; ++u) {
        const int64_t r = unique_ids[u];
        if (r < 0 || r >= table_rows) {
            bad += r != -1 ? 1 : 0;
            continue;
        }
        for (int64_t e = 0; e < dim; ++e) {
            const float g = unique_grads[u * dim + e];
            const float sign = g > 0.0f ? 1.0f : (g < 0.0f ? -1.0f : 0.0f);
            const float w = bf16_bits_to_float(table[r * dim + e]);
            const float step = lr * sign;
            const float updated = w - step;
            table[r * dim + e] = float_to_bf16_bits(updated);
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------- */
/* Causal depthwise PLE convolution, zero history per packed segment.     */
/* [API] Qwen3_8_FlashNextPLELayer: _causal_short_conv (a causal depthwise */
/* convolution over [batch, sequence, channels] with zeros as the history  */
/* on the left), _segmented_conv (every packed segment is convolved as if  */
/* it began a fresh row: zeros ahead of it, its own convolution, so no tap */
/* reads another segment), constructor conv_kernel_size (4) and the        */
/* attribute short_conv_dilation (= ngram_size).  Under context            */
/* parallelism the layer receives the preceding (K - 1) * dilation         */
/* positions from the previous rank; `halo` holds them (NULL: none).       */
/* Readings (the pages do not fix them): the taps follow F.conv1d, so      */
/*     out[t, c] = bias[c] + sum_k w[c, k] * x[t - (K - 1 - k) * dilation, c]*/
/* a tap reads 0 before the (halo-extended) row start or across a change   */
/* of segment id between it and t; bf16 data, the sum accumulated in fp32  */
/* from the bias in tap order k = 0 .. K-1, rounded once to bf16 (nearest, */
/* ties to even).                                                          */
/* Layout: x, out bf16 [batch, seq, channels]; halo bf16                   */
/* [batch, halo_len, channels]; seq_ids int64 [batch, halo_len + seq]      */
/* (covering the halo first); weight bf16 [channels, K]; bias bf16         */
/* [channels] or NULL.  Returns 0, or -1 on an invalid argument.           */
/* ---------------------------------------------------------------------- */
int oracle_ple_conv(const uint16_t *x, const uint16_t *halo, int64_t halo_len,
                    const int64_t *seq_ids, const uint16_t *weight, const uint16_t *bias,
                    int64_t batch, int64_t seq, int64_t channels, int kernel_size,
                    int dilation, uint16_t *out)
{
    if (kernel_size < 1 || dilation < 1 || halo_len < 0 || (halo_len > 0 && halo == NULL))
        return -1;
    const int64_t len = halo_len + seq;          /* positions of the extended row */
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t *seg = seq_ids ? seq_ids + b * len : NULL;
        for (int64_t t = 0; t < seq; ++t) {
            const int64_t pos = halo_len + t;    /* t in the extended row */
            for (int64_t c = 0; c < channels; ++c) {
                float acc = bias ? bf16_bits_to_float(bias[c]) : 0.0f;
                for (int k = 0; k < kernel_size; ++k) {
                    const int64_t p = pos - (int64_t)(kernel_size - 1 - k) * dilation;
                    int inside = p >= 0;
                    /* the tap's segment must reach from p to pos unbroken */
                    for (int64_t j = p; inside && seg != NULL && j < pos; ++j)
                        if (seg[j] != seg[j + 1])
                            inside = 0;
                    float v = 0.0f;
                    if (inside)
                        v = p < halo_len
                                ? bf16_bits_to_float(halo[(b * halo_len + p) * channels + c])
                                : bf16_bits_to_float(x[(b * seq + (p - halo_len)) * channels + c]);
                    const float wk = bf16_bits_to_float(weight[c * kernel_size + k]);
                    const float prod = wk * v;
                    acc = acc + prod;
                }
                out[(b * seq + t) * channels + c] = float_to_bf16_bits(acc);
            }
        }
    }
    return 0;
}
