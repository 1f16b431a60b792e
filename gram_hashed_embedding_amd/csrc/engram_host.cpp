// engram_host.cpp -- the extern "C" entry points of libengram.so: argument
// checks on the host, then the launchers of the HIP sources.  Plain C++ (no
// HIP headers), so that the same checks also build for the CPU alone, under
// host sanitizers, with stand-ins for the launchers.
//
// What each entry point computes, and the pages it follows, is stated with
// its declaration in include/engram.h.  Every check here runs before
// anything is enqueued: a bad argument returns an error code and enqueues
// nothing.
#include "engram_host.h"

namespace engram {

int make_hash_params(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                     int64_t stride, int64_t start, int64_t end, int32_t ngram_size,
                     int32_t heads_per_ngram, int64_t eos_id, const int64_t *h_multipliers,
                     const int64_t *h_primes, const int64_t *h_offsets, int64_t table_rows,
                     HashParams *hp, int64_t *tokens_out) {
  if (batch < 0 || stride < 0 || table_rows < 0) return ENGRAM_EINVAL;
  if (start < 0 || end < start || end > stride) return ENGRAM_EINVAL;
  if (ngram_size < 2 || ngram_size > ENGRAM_MAX_NGRAM || heads_per_ngram < 1)
    return ENGRAM_EINVAL;
  const int64_t H = (int64_t)(ngram_size - 1) * heads_per_ngram;
  if (H > ENGRAM_MAX_HEADS) return ENGRAM_EINVAL;
  if (h_multipliers == nullptr || h_primes == nullptr || h_offsets == nullptr)
    return ENGRAM_EINVAL;
  if (!mul_fits(batch, stride, INT64_MAX)) return ENGRAM_EINVAL;
  const int64_t local = end - start;
  const int64_t total = batch * local;
  if (!mul_fits(total, H * 8, INT64_MAX)) return ENGRAM_EINVAL;
  *hp = HashParams{};
  for (int64_t h = 0; h < H; ++h) {
    const int64_t p = h_primes[h], off = h_offsets[h];
    if (p <= 0 || off < 0 || off > table_rows - p) return ENGRAM_EINVAL;
    hp->prime[h] = (uint64_t)p;
    hp->magic[h] = UINT64_MAX / (uint64_t)p;
    hp->offset[h] = off;
  }
  for (int k = 0; k < ngram_size; ++k) hp->mult[k] = (uint64_t)h_multipliers[k];
  *tokens_out = total;
  if (total > 0 && d_tokens == nullptr) return ENGRAM_EINVAL;
  hp->tokens = d_tokens;
  hp->seg = d_seq_ids;
  hp->stride = stride;
  hp->start = start;
  hp->local = local;
  hp->eos = eos_id;
  hp->n = ngram_size;
  hp->J = heads_per_ngram;
  hp->H = (int32_t)H;
  return ENGRAM_OK;
}

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool make_plan(int64_t n, int64_t table_rows, int64_t dim, Plan *p) {
  if (n < 0 || table_rows < 0 || dim <= 0 || dim % 8 != 0 || dim > kMaxSortedDim) return false;
  if (!mul_fits(n, dim * 8, INT64_MAX / 4) || !mul_fits(table_rows, dim * 4, INT64_MAX))
    return false;
  p->num_tiles = (n + kSortTile - 1) / kSortTile;
  p->num_ranges = (n + kRange - 1) / kRange;
  p->slot_tiles = (p->num_ranges + kSlotThreads - 1) / kSlotThreads;
  p->bits = bit_width_u64((uint64_t)table_rows);  // the key table_rows must fit
  if (p->bits < 1) p->bits = 1;
  p->passes = (p->bits + 7) / 8;
  p->per_pass = (p->bits + p->passes - 1) / p->passes;
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  // the plan's scalars first, at the same place whatever n is, so an apply
  // always finds the stamp of the last plan made in the workspace
  p->scalars = take(sizeof(PlanScalars));
  // key / index buffers hold whole ranges (the walkers read 16-byte vectors)
  const size_t nn = (size_t)n;
  static_assert(256 % (kRange * 4) == 0, "256-byte padding covers a whole range");
  p->keys_a = take(nn * 4);
  p->vals_a = take(nn * 4);
  p->keys_b = take(nn * 4);
  p->vals_b = take(nn * 4);
  // look-back words: every sort pass's, then the slot scan's.  A sort in
  // per-head segments has at most one more (ragged) tile per head.
  p->status_words =
      (int64_t)p->passes * (p->num_tiles + ENGRAM_MAX_HEADS) * kMaxBins + p->slot_tiles;
  p->status = take((size_t)p->status_words * 8);
  p->counters = take(kSortCounters * 4);
  p->head_off = take((size_t)p->num_ranges * 4);
  // per chunk of the sorted order: the slot of a long run that leaves it for
  // the next chunk (+1; 0 when none), and two fp64 partial-sum rows (the
  // long run that enters it, the long run that leaves it)
  p->num_chunks = (n + kChunk - 1) / kChunk;
  p->chunk_owner = take((size_t)p->num_chunks * 4);
  p->partials = take((size_t)p->num_chunks * 2 * (size_t)dim * 8);
  p->total = off;
  return true;
}

}  // namespace engram

using namespace engram;

namespace {

// The sorted path's sizes: 32-bit keys and flat indices, and the apply's
// grid inside the launch limit.  That grid (walkers of 2 to 64 lanes per 16
// ids) is the only one of the path that can pass the limit below n = 2^32:
// the plan's kernels take at most about one thread per 4 ids.
bool sorted_fits(const Plan &p, int64_t n, int64_t table_rows, int64_t head_dim) {
  return sorted_limits_ok(n, table_rows) && grid_fits(apply_blocks(p, head_dim), kWalkThreads);
}

int check_sorted(int64_t n, int64_t table_rows, int64_t head_dim, Plan *p) {
  if (!make_plan(n, table_rows, head_dim, p) || !sorted_fits(*p, n, table_rows, head_dim))
    return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

int check_workspace(const Plan &p, const void *ws, size_t bytes) {
  if (ws == nullptr || bytes < p.total || !aligned16(ws)) return ENGRAM_EWORKSPACE;
  return ENGRAM_OK;
}

int hash_window(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch, int64_t stride,
                int64_t start, int64_t end, int32_t ngram_size, int32_t heads_per_ngram,
                int64_t eos_id, const int64_t *h_multipliers, const int64_t *h_primes,
                const int64_t *h_offsets, int64_t table_rows, int64_t *d_row_ids,
                void *stream) {
  HashParams hp;
  int64_t total = 0;
  const int rc = make_hash_params(d_tokens, d_seq_ids, batch, stride, start, end, ngram_size,
                                  heads_per_ngram, eos_id, h_multipliers, h_primes, h_offsets,
                                  table_rows, &hp, &total);
  if (rc != ENGRAM_OK) return rc;
  if (total == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr) return ENGRAM_EINVAL;
  return launch_hash(hp, total, d_row_ids, stream);
}

int lookup_window(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                  int64_t stride, int64_t start, int64_t end, int32_t ngram_size,
                  int32_t heads_per_ngram, int64_t eos_id, const int64_t *h_multipliers,
                  const int64_t *h_primes, const int64_t *h_offsets, const void *d_table,
                  int64_t table_rows, int64_t head_dim, void *d_out, int64_t *d_row_ids,
                  void *stream) {
  if (head_dim <= 0 || head_dim % 8 != 0 || head_dim > kMaxDim) return ENGRAM_EINVAL;
  HashParams hp;
  int64_t tokens = 0;
  const int rc = make_hash_params(d_tokens, d_seq_ids, batch, stride, start, end, ngram_size,
                                  heads_per_ngram, eos_id, h_multipliers, h_primes, h_offsets,
                                  table_rows, &hp, &tokens);
  if (rc != ENGRAM_OK) return rc;
  const int64_t n = tokens * hp.H;
  if (!mul_fits(table_rows, head_dim * 2, INT64_MAX) || !mul_fits(n, head_dim * 2, INT64_MAX))
    return ENGRAM_EINVAL;
  if (n == 0) return ENGRAM_OK;
  if (d_table == nullptr || d_out == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_table) || !aligned16(d_out)) return ENGRAM_EALIGN;
  return launch_lookup(hp, n, d_table, head_dim, d_out, d_row_ids, stream);
}

}  // namespace

extern "C" const char *engram_status_string(int status) {
  switch (status) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_EINVAL: return "invalid argument";
    case ENGRAM_EALIGN: return "device buffer not 16-byte aligned";
    case ENGRAM_EWORKSPACE: return "workspace missing or too small";
    case ENGRAM_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int engram_abi_version(void) { return ENGRAM_ABI_VERSION; }

// ------------------------------------------------------------------ hash ---
extern "C" int engram_hash(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                           int64_t seq, int32_t ngram_size, int32_t heads_per_ngram,
                           int64_t eos_id, const int64_t *h_multipliers,
                           const int64_t *h_primes, const int64_t *h_offsets,
                           int64_t table_rows, int64_t *d_row_ids, void *stream) {
  if (seq < 0) return ENGRAM_EINVAL;
  return hash_window(d_tokens, d_seq_ids, batch, seq, 0, seq, ngram_size, heads_per_ngram,
                     eos_id, h_multipliers, h_primes, h_offsets, table_rows, d_row_ids, stream);
}

extern "C" int engram_hash_slice(const int64_t *d_tokens, const int64_t *d_seq_ids,
                                 int64_t batch, int64_t global_seq, int64_t seq_start,
                                 int64_t seq_end, int32_t ngram_size, int32_t heads_per_ngram,
                                 int64_t eos_id, const int64_t *h_multipliers,
                                 const int64_t *h_primes, const int64_t *h_offsets,
                                 int64_t table_rows, int64_t *d_row_ids, void *stream) {
  return hash_window(d_tokens, d_seq_ids, batch, global_seq, seq_start, seq_end, ngram_size,
                     heads_per_ngram, eos_id, h_multipliers, h_primes, h_offsets, table_rows,
                     d_row_ids, stream);
}

// ---------------------------------------------------------------- gather ---
extern "C" int engram_gather(const int64_t *d_row_ids, int64_t n, const void *d_table,
                             int64_t table_rows, int64_t head_dim, void *d_out,
                             int64_t *d_err_count, void *stream) {
  if (n < 0 || table_rows < 0 || head_dim <= 0 || head_dim % 8 != 0 || head_dim > kMaxDim)
    return ENGRAM_EINVAL;
  if (!mul_fits(table_rows, head_dim * 2, INT64_MAX) || !mul_fits(n, head_dim * 2, INT64_MAX))
    return ENGRAM_EINVAL;
  if (n == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr || d_table == nullptr || d_out == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_table) || !aligned16(d_out)) return ENGRAM_EALIGN;
  return launch_gather(d_row_ids, n, d_table, table_rows, head_dim, d_out, d_err_count, stream);
}

extern "C" int engram_lookup(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                             int64_t seq, int32_t ngram_size, int32_t heads_per_ngram,
                             int64_t eos_id, const int64_t *h_multipliers,
                             const int64_t *h_primes, const int64_t *h_offsets,
                             const void *d_table, int64_t table_rows, int64_t head_dim,
                             void *d_out, int64_t *d_row_ids, void *stream) {
  if (seq < 0) return ENGRAM_EINVAL;
  return lookup_window(d_tokens, d_seq_ids, batch, seq, 0, seq, ngram_size, heads_per_ngram,
                       eos_id, h_multipliers, h_primes, h_offsets, d_table, table_rows, head_dim,
                       d_out, d_row_ids, stream);
}

extern "C" int engram_lookup_slice(const int64_t *d_tokens, const int64_t *d_seq_ids,
                                   int64_t batch, int64_t global_seq, int64_t seq_start,
                                   int64_t seq_end, int32_t ngram_size, int32_t heads_per_ngram,
                                   int64_t eos_id, const int64_t *h_multipliers,
                                   const int64_t *h_primes, const int64_t *h_offsets,
                                   const void *d_table, int64_t table_rows, int64_t head_dim,
                                   void *d_out, int64_t *d_row_ids, void *stream) {
  return lookup_window(d_tokens, d_seq_ids, batch, global_seq, seq_start, seq_end, ngram_size,
                       heads_per_ngram, eos_id, h_multipliers, h_primes, h_offsets, d_table,
                       table_rows, head_dim, d_out, d_row_ids, stream);
}

// --------------------------------------------------------------- scatter ---
extern "C" size_t engram_scatter_add_workspace(int64_t n, int64_t table_rows, int64_t head_dim,
                                               int32_t mode) {
  Plan p;
  if (!make_plan(n, table_rows, head_dim, &p)) return (size_t)-1;
  if (mode == ENGRAM_SCATTER_ATOMIC) return 0;
  if (mode != ENGRAM_SCATTER_SORTED && mode != ENGRAM_SCATTER_ROWSPARSE) return (size_t)-1;
  if (!sorted_fits(p, n, table_rows, head_dim)) return (size_t)-1;
  return p.total;
}

extern "C" int engram_scatter_plan(const int64_t *d_row_ids, int64_t n, int64_t table_rows,
                                   int64_t head_dim, void *d_workspace, size_t workspace_bytes,
                                   int64_t *d_err_count, void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  if (n == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr) return ENGRAM_EINVAL;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  return launch_plan(d_row_ids, nullptr, n, table_rows, p, d_workspace, d_err_count, stream);
}

extern "C" int engram_scatter_plan_tokens(const int64_t *d_tokens, const int64_t *d_seq_ids,
                                          int64_t batch, int64_t seq, int32_t ngram_size,
                                          int32_t heads_per_ngram, int64_t eos_id,
                                          const int64_t *h_multipliers, const int64_t *h_primes,
                                          const int64_t *h_offsets, int64_t table_rows,
                                          int64_t head_dim, void *d_workspace,
                                          size_t workspace_bytes, int64_t *d_err_count,
                                          void *stream) {
  if (seq < 0) return ENGRAM_EINVAL;
  HashParams hp;
  int64_t tokens = 0;
  int rc = make_hash_params(d_tokens, d_seq_ids, batch, seq, 0, seq, ngram_size,
                            heads_per_ngram, eos_id, h_multipliers, h_primes, h_offsets,
                            table_rows, &hp, &tokens);
  if (rc != ENGRAM_OK) return rc;
  if (!mul_fits(tokens, hp.H, INT64_MAX)) return ENGRAM_EINVAL;
  const int64_t n = tokens * hp.H;
  Plan p;
  if ((rc = check_sorted(n, table_rows, head_dim, &p)) != ENGRAM_OK) return rc;
  if (n == 0) return ENGRAM_OK;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  return launch_plan(nullptr, &hp, n, table_rows, p, d_workspace, d_err_count, stream);
}

extern "C" int engram_scatter_apply(const void *d_grads, int64_t n, int64_t head_dim,
                                    int64_t table_rows, float *d_grad_table,
                                    int64_t *d_unique_ids, float *d_unique_grads,
                                    int64_t *d_num_unique, void *d_workspace,
                                    size_t workspace_bytes, int64_t *d_err_count, void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  const bool dense = d_grad_table != nullptr;
  const bool sparse =
      d_unique_ids != nullptr || d_unique_grads != nullptr || d_num_unique != nullptr;
  if (dense == sparse) return ENGRAM_EINVAL;  // exactly one output form
  if (sparse && (d_unique_ids == nullptr || d_unique_grads == nullptr || d_num_unique == nullptr))
    return ENGRAM_EINVAL;
  if (n == 0) return sparse ? launch_write_zero(d_num_unique, stream) : ENGRAM_OK;
  if (d_grads == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || (dense && !aligned16(d_grad_table)) ||
      (sparse && !aligned16(d_unique_grads)))
    return ENGRAM_EALIGN;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  const ApplyOut o = {sparse ? kOutSparse : kOutDense, d_grad_table, d_unique_ids,
                      d_unique_grads, d_num_unique, nullptr, 0.0f};
  return launch_apply(d_grads, n, head_dim, table_rows, p, d_workspace, o, d_err_count, stream);
}

extern "C" int engram_scatter_apply_signsgd(const void *d_grads, int64_t n, int64_t head_dim,
                                            int64_t table_rows, void *d_table, float lr,
                                            void *d_workspace, size_t workspace_bytes,
                                            int64_t *d_err_count, void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  if (n == 0) return ENGRAM_OK;
  if (d_grads == nullptr || d_table == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_table)) return ENGRAM_EALIGN;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  const ApplyOut o = {kOutSignSGD, nullptr, nullptr, nullptr, nullptr, d_table, lr};
  return launch_apply(d_grads, n, head_dim, table_rows, p, d_workspace, o, d_err_count, stream);
}

extern "C" int engram_scatter_add(const int64_t *d_row_ids, int64_t n, const void *d_grads,
                                  int64_t head_dim, float *d_grad_table, int64_t table_rows,
                                  int32_t mode, void *d_workspace, size_t workspace_bytes,
                                  int64_t *d_err_count, void *stream) {
  Plan p;
  if (!make_plan(n, table_rows, head_dim, &p)) return ENGRAM_EINVAL;
  if (mode != ENGRAM_SCATTER_SORTED && mode != ENGRAM_SCATTER_ATOMIC) return ENGRAM_EINVAL;
  if (mode == ENGRAM_SCATTER_SORTED && !sorted_fits(p, n, table_rows, head_dim))
    return ENGRAM_EINVAL;
  if (n == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr || d_grads == nullptr || d_grad_table == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_grad_table)) return ENGRAM_EALIGN;
  if (mode == ENGRAM_SCATTER_ATOMIC)
    return launch_scatter_atomic(d_row_ids, n, d_grads, head_dim, d_grad_table, table_rows,
                                 d_err_count, stream);
  int rc = check_workspace(p, d_workspace, workspace_bytes);
  if (rc != ENGRAM_OK) return rc;
  if ((rc = launch_plan(d_row_ids, nullptr, n, table_rows, p, d_workspace, d_err_count,
                        stream)) != ENGRAM_OK)
    return rc;
  const ApplyOut o = {kOutDense, d_grad_table, nullptr, nullptr, nullptr, nullptr, 0.0f};
  return launch_apply(d_grads, n, head_dim, table_rows, p, d_workspace, o, d_err_count, stream);
}

namespace {

// The row-sparse scatter-add into a checked workspace (the caller's, or the
// library's fixed array).
int rowsparse_into(const int64_t *d_row_ids, int64_t n, const void *d_grads, int64_t head_dim,
                   int64_t table_rows, int64_t *d_unique_ids, float *d_unique_grads,
                   int64_t *d_num_unique, const Plan &p, void *ws, int64_t *d_err_count,
                   void *stream) {
  int rc = launch_plan(d_row_ids, nullptr, n, table_rows, p, ws, d_err_count, stream);
  if (rc != ENGRAM_OK) return rc;
  const ApplyOut o = {kOutSparse, nullptr, d_unique_ids, d_unique_grads, d_num_unique, nullptr,
                      0.0f};
  return launch_apply(d_grads, n, head_dim, table_rows, p, ws, o, d_err_count, stream);
}

// Checks the row-sparse calls share (before any workspace is looked at).
int check_rowsparse(const int64_t *d_row_ids, int64_t n, const void *d_grads,
                    const int64_t *d_unique_ids, const float *d_unique_grads,
                    const int64_t *d_num_unique) {
  if (d_num_unique == nullptr) return ENGRAM_EINVAL;
  if (n == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr || d_grads == nullptr || d_unique_ids == nullptr ||
      d_unique_grads == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_unique_grads)) return ENGRAM_EALIGN;
  return ENGRAM_OK;
}

}  // namespace

extern "C" int engram_scatter_add_rowsparse(const int64_t *d_row_ids, int64_t n,
                                            const void *d_grads, int64_t head_dim,
                                            int64_t table_rows, int64_t *d_unique_ids,
                                            float *d_unique_grads, int64_t *d_num_unique,
                                            void *d_workspace, size_t workspace_bytes,
                                            int64_t *d_err_count, void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  if ((rc = check_rowsparse(d_row_ids, n, d_grads, d_unique_ids, d_unique_grads,
                            d_num_unique)) != ENGRAM_OK)
    return rc;
  if (n == 0) return launch_write_zero(d_num_unique, stream);
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  return rowsparse_into(d_row_ids, n, d_grads, head_dim, table_rows, d_unique_ids,
                        d_unique_grads, d_num_unique, p, d_workspace, d_err_count, stream);
}

extern "C" int engram_scatter_add_rowsparse_noalloc(const int64_t *d_row_ids, int64_t n,
                                                    const void *d_grads, int64_t head_dim,
                                                    int64_t table_rows, int64_t *d_unique_ids,
                                                    float *d_unique_grads,
                                                    int64_t *d_num_unique, int64_t *d_err_count,
                                                    void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  if (p.total > ENGRAM_NOALLOC_SCRATCH_BYTES) return ENGRAM_EWORKSPACE;  // more than the array
  if ((rc = check_rowsparse(d_row_ids, n, d_grads, d_unique_ids, d_unique_grads,
                            d_num_unique)) != ENGRAM_OK)
    return rc;
  if (n == 0) return launch_write_zero(d_num_unique, stream);
  void *ws = static_scratch();
  if (ws == nullptr) return ENGRAM_EHIP;
  return rowsparse_into(d_row_ids, n, d_grads, head_dim, table_rows, d_unique_ids,
                        d_unique_grads, d_num_unique, p, ws, d_err_count, stream);
}

// -------------------------------------------------------------- optimizer --
extern "C" int engram_signsgd_rowsparse(const int64_t *d_unique_ids, const float *d_unique_grads,
                                        const int64_t *d_num_unique, int64_t capacity,
                                        int64_t head_dim, void *d_table, int64_t table_rows,
                                        float lr, int64_t *d_err_count, void *stream) {
  if (capacity < 0 || table_rows < 0 || head_dim <= 0 || head_dim % 8 != 0 || head_dim > kMaxDim)
    return ENGRAM_EINVAL;
  if (!mul_fits(capacity, head_dim * 4, INT64_MAX / 2) ||
      !mul_fits(table_rows, head_dim * 2, INT64_MAX))
    return ENGRAM_EINVAL;
  if (capacity == 0) return ENGRAM_OK;
  if (d_unique_ids == nullptr || d_unique_grads == nullptr || d_num_unique == nullptr ||
      d_table == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned16(d_unique_grads) || !aligned16(d_table)) return ENGRAM_EALIGN;
  return launch_signsgd(d_unique_ids, d_unique_grads, d_num_unique, capacity, head_dim, d_table,
                        table_rows, lr, d_err_count, stream);
}

// ------------------------------------------------------------ convolution --
extern "C" int engram_ple_conv(const void *d_x, const void *d_halo, int64_t halo_len,
                               const int64_t *d_seq_ids, const void *d_weight,
                               const void *d_bias, int64_t batch, int64_t seq, int64_t channels,
                               int32_t kernel_size, int32_t dilation, void *d_out,
                               void *stream) {
  if (batch < 0 || seq < 0 || channels <= 0 || channels % 8 != 0 || halo_len < 0)
    return ENGRAM_EINVAL;
  if (kernel_size < 1 || kernel_size > kConvMaxKernel || dilation < 1) return ENGRAM_EINVAL;
  if (halo_len > 0 && d_halo == nullptr) return ENGRAM_EINVAL;
  if (seq > INT64_MAX / 2 - halo_len || channels > INT64_MAX / 8) return ENGRAM_EINVAL;
  if (!mul_fits(batch, seq + halo_len, INT64_MAX / 8) ||
      !mul_fits(batch * (seq + halo_len), channels * 2, INT64_MAX))
    return ENGRAM_EINVAL;
  if (batch == 0 || seq == 0) return ENGRAM_OK;
  if (d_x == nullptr || d_weight == nullptr || d_out == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_x) || !aligned16(d_out) || (d_halo != nullptr && !aligned16(d_halo)))
    return ENGRAM_EALIGN;
  const ConvCall c = {d_x, d_halo, halo_len, d_seq_ids, d_weight, d_bias, d_out,
                      batch, seq, channels, kernel_size, dilation};
  return launch_ple_conv(c, stream);
}

// ------------------------------------------------------------ the executor --
extern "C" int engram_run_ops(const engram_op *ops, int64_t count, int64_t *failed_index) {
  if (failed_index != nullptr) *failed_index = -1;
  if (count < 0 || (count > 0 && ops == nullptr)) return ENGRAM_EINVAL;
  for (int64_t i = 0; i < count; ++i) {
    const engram_op &o = ops[i];
    int st = ENGRAM_EINVAL;
    switch (o.op) {
      case ENGRAM_OP_LOOKUP:
        st = engram_lookup(o.d_tokens, o.d_seq_ids, o.batch, o.seq, o.ngram_size,
                           o.heads_per_ngram, o.eos_id, o.h_multipliers, o.h_primes, o.h_offsets,
                           o.d_table, o.table_rows, o.head_dim, o.d_out, o.d_row_ids, o.stream);
        break;
      case ENGRAM_OP_PLAN_TOKENS:
        st = engram_scatter_plan_tokens(o.d_tokens, o.d_seq_ids, o.batch, o.seq, o.ngram_size,
                                        o.heads_per_ngram, o.eos_id, o.h_multipliers,
                                        o.h_primes, o.h_offsets, o.table_rows, o.head_dim,
                                        o.d_workspace, o.workspace_bytes, o.d_err_count,
                                        o.stream);
        break;
      case ENGRAM_OP_APPLY:
        st = engram_scatter_apply(o.d_grads, o.n, o.head_dim, o.table_rows, o.d_grad_table,
                                  o.d_unique_ids, o.d_unique_grads, o.d_num_unique,
                                  o.d_workspace, o.workspace_bytes, o.d_err_count, o.stream);
        break;
      case ENGRAM_OP_APPLY_SIGNSGD:
        st = engram_scatter_apply_signsgd(o.d_grads, o.n, o.head_dim, o.table_rows,
                                          o.d_table_rw, o.lr, o.d_workspace, o.workspace_bytes,
                                          o.d_err_count, o.stream);
        break;
      case ENGRAM_OP_RECORD:
        st = o.event != nullptr ? engram::record_event(o.event, o.stream) : ENGRAM_EINVAL;
        break;
      case ENGRAM_OP_WAIT:
        st = o.event != nullptr ? engram::wait_event(o.stream, o.event) : ENGRAM_EINVAL;
        break;
      default:
        break;
    }
    if (st != ENGRAM_OK) {
      if (failed_index != nullptr) *failed_index = i;
      return st;
    }
  }
  return ENGRAM_OK;
}
