// engram_gather.hip -- bf16 row gather for gfx950.
//
// out[i, :] = table[row_ids[i], :], the local embedding lookup of the NeMo
// AutoModel v0.7 API page "qwen3_8_flash_next.engram" (_lookup_ngram_ids;
// Qwen3_8_FlashNextOwnerShardedEmbedding with no process group keeps the
// whole table local and performs a plain lookup).  Row -1 (padding) and
// rows outside the table give zero rows; the latter are counted.
//
// Design.  The work is a random-row copy bound by HBM bandwidth.  A row of
// head_dim bf16 is split into 16-byte chunks; lane i of the grid moves
// chunk i of the flattened [n, head_dim] output, so consecutive lanes read
// consecutive 16-byte pieces of a row (head_dim = 256: 32 lanes per 512-byte
// row, two rows per wavefront instruction) and write one contiguous span of
// the output.  Each lane moves kUnroll = 2 chunks (loads issued before the
// stores); HBM latency on random rows is covered by the number of resident
// wavefronts rather than by deep per-lane unrolling, which measured best on
// MI355X (about 6.2 TB/s, the same as a plain streaming copy; 8 chunks per
// lane was about 4% slower).  Row offsets are
// 64-bit: a 200M x 256 table is 102.4 GB.  Output stores are non-temporal
// so the streaming output does not evict hot (Zipf-frequent) table rows
// from L2 and the Infinity Cache; table loads stay cacheable.
#include "engram_hash_dev.h"

namespace engram {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kUnroll = 2;

// Chunk c of the flattened output -> (lookup i, chunk j of the row).
template <int LOG2_CPR>
__device__ __forceinline__ void split_chunk(int64_t c, int64_t cpr, int64_t &i, int64_t &j) {
  if (LOG2_CPR >= 0) {
    i = c >> LOG2_CPR;
    j = c & ((1 << (LOG2_CPR < 0 ? 0 : LOG2_CPR)) - 1);
  } else {
    i = c / cpr;
    j = c - i * cpr;
  }
}

// One lane's kUnroll chunks.  FULL: every chunk exists, so loads and stores
// are unconditional and the compiler issues all loads, one wait, then all
// stores.  Invalid rows load row 0 (a valid row; requires table_rows > 0)
// and are zeroed afterwards, which keeps the loads branch-free.
template <int LOG2_CPR, bool FULL>
__device__ __forceinline__ void gather_body(const int64_t *__restrict__ ids, int64_t total,
                                            const u32x4 *__restrict__ table, int64_t table_rows,
                                            int64_t cpr, u32x4 *__restrict__ out, int64_t *err,
                                            int64_t base) {
  int64_t row[kUnroll], col[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kGatherThreads;
    int64_t i, j;
    split_chunk<LOG2_CPR>(FULL || c < total ? c : 0, cpr, i, j);
    col[u] = j;
    row[u] = ids[i];
  }
  u32x4 v[kUnroll];
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t r = row[u];
    const bool ok = r >= 0 && r < table_rows;
    v[u] = table[(ok ? r : 0) * cpr + col[u]];
    if (!ok) v[u] = u32x4{0u, 0u, 0u, 0u};
    const bool live = FULL || base + (int64_t)u * kGatherThreads < total;
    bad += (live && col[u] == 0 && !ok && r != -1) ? 1 : 0;
  }
  count_errors(bad, err);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kGatherThreads;
    if (FULL || c < total) __builtin_nontemporal_store(v[u], &out[c]);
  }
}

// LOG2_CPR >= 0: chunks per row is 1 << LOG2_CPR; -1: any chunks per row.
template <int LOG2_CPR>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const int64_t *__restrict__ ids, int64_t n, const u32x4 *__restrict__ table,
    int64_t table_rows, int64_t cpr, u32x4 *__restrict__ out, int64_t *err) {
  const int64_t total = n * cpr;
  const int64_t block0 = (int64_t)blockIdx.x * (kGatherThreads * kUnroll);
  const int64_t base = block0 + threadIdx.x;
  if (block0 + kGatherThreads * kUnroll <= total)
    gather_body<LOG2_CPR, true>(ids, total, table, table_rows, cpr, out, err, base);
  else
    gather_body<LOG2_CPR, false>(ids, total, table, table_rows, cpr, out, err, base);
}

// A table with no rows: every lookup is padding or invalid.
__global__ __launch_bounds__(kGatherThreads) void zero_rows_kernel(const int64_t *ids, int64_t n,
                                                                   int64_t cpr, u32x4 *out,
                                                                   int64_t *err) {
  const int64_t c = (int64_t)blockIdx.x * kGatherThreads + threadIdx.x;
  if (c >= n * cpr) return;
  out[c] = u32x4{0u, 0u, 0u, 0u};
  if (c % cpr == 0) count_errors(ids[c / cpr] != -1 ? 1 : 0, err);
}

// The fused forward (engram_lookup).  A block takes rows_per_block
// consecutive lookups.  Phase 1: its first rows_per_block lanes compute one
// row each from the tokens (lookup_row: the token's history in one round of
// loads, the order mix, a Barrett remainder), so the hash costs one lane per
// row, and keep them in LDS (and write them out when the caller asks).
// Phase 2: every lane moves kLookUnroll 16-byte chunks of those rows (all
// loads before the stores), so a block's kLookChunks chunks take one round
// trip.  The row ids never go through memory.  A block moves about
// kLookChunks chunks: 32 rows at head_dim 256 (measured best there), more
// rows for narrower rows (head_dim 64: 128 rows), at most one per thread.
// Four chunks per lane (one round) against two (two rounds) measured, in one
// process: e2e 265.4 against 269.9 us, full-scale 171.2 against 175.6,
// medium 11.5 against 12.4.  N = ngram_size at compile time, so
// the history takes no more registers than the order needs.  The slice form
// (one context-parallel rank's forward, _forward_global_slice on the same
// page) is the same kernel over a window of positions whose history may
// reach back before it.
constexpr int kLookRows = 32;       // fewest rows per block
constexpr int kLookChunks = 1024;   // 16-byte chunks per block, when rows allow
constexpr int kLookRowsMax = kGatherThreads;
constexpr int kLookUnroll = kLookChunks / kGatherThreads;  // chunks per lane

template <int N>
__global__ __launch_bounds__(kGatherThreads) void lookup_kernel(
    const HashParams h, int64_t n, int rows_per_block, const u32x4 *__restrict__ table,
    int64_t cpr, int log2_cpr, u32x4 *__restrict__ out, int64_t *__restrict__ rows_out) {
  __shared__ int64_t s_row[kLookRowsMax];
  const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
  const int nrows = (int)min((int64_t)rows_per_block, n - row0);
  if ((int)threadIdx.x < nrows) {
    const int64_t r = lookup_row<N>(h, row0 + threadIdx.x);  // inside its head's rows
    s_row[threadIdx.x] = r;
    if (rows_out != nullptr) rows_out[row0 + threadIdx.x] = r;
  }
  __syncthreads();
  const int64_t nchunks = (int64_t)nrows * cpr;
  u32x4 *dst = out + row0 * cpr;
  for (int64_t k0 = threadIdx.x; k0 < nchunks; k0 += (int64_t)kGatherThreads * kLookUnroll) {
    u32x4 v[kLookUnroll];
#pragma unroll
    for (int u = 0; u < kLookUnroll; ++u) {
      const int64_t k = min(k0 + (int64_t)u * kGatherThreads, nchunks - 1);
      const int64_t rl = log2_cpr >= 0 ? k >> log2_cpr : k / cpr;
      v[u] = table[s_row[rl] * cpr + (k - rl * cpr)];
    }
#pragma unroll
    for (int u = 0; u < kLookUnroll; ++u) {
      const int64_t k = k0 + (int64_t)u * kGatherThreads;
      if (k < nchunks) __builtin_nontemporal_store(v[u], &dst[k]);
    }
  }
}

}  // namespace
}  // namespace engram

int engram::launch_gather(const int64_t *d_row_ids, int64_t n, const void *d_table,
                          int64_t table_rows, int64_t head_dim, void *d_out, int64_t *d_err_count,
                          void *stream) {
  const int64_t cpr = head_dim / 8;
  const int64_t total = n * cpr;
  const int64_t per_block = (int64_t)kGatherThreads * kUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  if (!grid_fits(blocks, kGatherThreads)) return ENGRAM_EINVAL;
  const u32x4 *tab = static_cast<const u32x4 *>(d_table);
  u32x4 *out = static_cast<u32x4 *>(d_out);
  hipStream_t s = as_stream(stream);
  if (table_rows == 0) {
    const int64_t zb = (total + kGatherThreads - 1) / kGatherThreads;
    if (!grid_fits(zb, kGatherThreads)) return ENGRAM_EINVAL;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)zb), dim3(kGatherThreads), 0, s,
                       d_row_ids, n, cpr, out, d_err_count);
    return launch_status();
  }
  const dim3 grid((unsigned)blocks), block(kGatherThreads);
  switch (cpr) {
#define ENGRAM_GATHER_CASE(L2)                                                             \
  case (1 << L2):                                                                          \
    hipLaunchKernelGGL(gather_kernel<L2>, grid, block, 0, s, d_row_ids, n, tab, table_rows, \
                       cpr, out, d_err_count);                                             \
    break;
    ENGRAM_GATHER_CASE(0)
    ENGRAM_GATHER_CASE(1)
    ENGRAM_GATHER_CASE(2)
    ENGRAM_GATHER_CASE(3)
    ENGRAM_GATHER_CASE(4)
    ENGRAM_GATHER_CASE(5)
    ENGRAM_GATHER_CASE(6)
    ENGRAM_GATHER_CASE(7)
    ENGRAM_GATHER_CASE(8)
#undef ENGRAM_GATHER_CASE
    default:
      hipLaunchKernelGGL(gather_kernel<-1>, grid, block, 0, s, d_row_ids, n, tab, table_rows,
                         cpr, out, d_err_count);
  }
  return launch_status();
}

// The fused forward over the positions hp describes (a whole row, or one
// context-parallel slice of it), n = tokens * H lookups.
int engram::launch_lookup(const HashParams &hp, int64_t n, const void *d_table,
                          int64_t head_dim, void *d_out, int64_t *d_row_ids, void *stream) {
  const int64_t cpr = head_dim / 8;
  int64_t rows_per_block = kLookChunks / cpr;
  rows_per_block = rows_per_block < kLookRows ? kLookRows : rows_per_block;
  rows_per_block = rows_per_block > kLookRowsMax ? kLookRowsMax : rows_per_block;
  const int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  if (!grid_fits(blocks, kGatherThreads)) return ENGRAM_EINVAL;
  const u32x4 *tab = static_cast<const u32x4 *>(d_table);
  u32x4 *out = static_cast<u32x4 *>(d_out);
  const dim3 grid((unsigned)blocks), block(kGatherThreads);
  hipStream_t s = as_stream(stream);
  int log2_cpr = -1;
  for (int b = 0; b < 62; ++b)
    if (cpr == (int64_t)1 << b) log2_cpr = b;
  switch (hp.n) {
#define ENGRAM_LOOKUP_CASE(N)                                                                 \
  case N:                                                                                     \
    hipLaunchKernelGGL(lookup_kernel<N>, grid, block, 0, s, hp, n, (int)rows_per_block, tab,  \
                       cpr, log2_cpr, out, d_row_ids);                                        \
    break;
    ENGRAM_LOOKUP_CASE(2)
    ENGRAM_LOOKUP_CASE(3)
    ENGRAM_LOOKUP_CASE(4)
    ENGRAM_LOOKUP_CASE(5)
    ENGRAM_LOOKUP_CASE(6)
    ENGRAM_LOOKUP_CASE(7)
    ENGRAM_LOOKUP_CASE(8)
#undef ENGRAM_LOOKUP_CASE
  }
  return launch_status();
}
