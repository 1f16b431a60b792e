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
// the output.  Each lane keeps kUnroll chunks in flight (all loads issued
// before any store) to cover HBM latency on random rows.  Row offsets are
// 64-bit: a 200M x 256 table is 102.4 GB.  Output stores are non-temporal
// so the streaming output does not evict hot (Zipf-frequent) table rows
// from L2 and the Infinity Cache; table loads stay cacheable.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kUnroll = 8;

// LOG2_CPR >= 0: chunks per row is 1 << LOG2_CPR; -1: any chunks per row.
template <int LOG2_CPR>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const int64_t *__restrict__ ids, int64_t n, const u32x4 *__restrict__ table,
    int64_t table_rows, int64_t cpr, u32x4 *__restrict__ out, int64_t *err) {
  const int64_t total = n * cpr;
  const int64_t base = (int64_t)blockIdx.x * (kGatherThreads * kUnroll) + threadIdx.x;

  int64_t row[kUnroll];
  int64_t col[kUnroll];
  bool live[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kGatherThreads;
    live[u] = c < total;
    int64_t i, j;
    if (LOG2_CPR >= 0) {
      i = c >> LOG2_CPR;
      j = c & ((1 << (LOG2_CPR < 0 ? 0 : LOG2_CPR)) - 1);
    } else {
      i = c / cpr;
      j = c - i * cpr;
    }
    col[u] = j;
    row[u] = live[u] ? ids[i] : -1;
  }

  u32x4 v[kUnroll];
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t r = row[u];
    const bool ok = r >= 0 && r < table_rows;
    v[u] = ok ? table[r * cpr + col[u]] : u32x4{0u, 0u, 0u, 0u};
    bad += (live[u] && col[u] == 0 && !ok && r != -1) ? 1 : 0;
  }
  count_errors(bad, err);

#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (live[u]) __builtin_nontemporal_store(v[u], &out[base + (int64_t)u * kGatherThreads]);
  }
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" int engram_gather(const int64_t *d_row_ids, int64_t n, const void *d_table,
                             int64_t table_rows, int64_t head_dim, void *d_out,
                             int64_t *d_err_count, void *stream) {
  if (n < 0 || table_rows < 0 || head_dim <= 0 || head_dim % 8 != 0) return ENGRAM_EINVAL;
  if (!mul_fits(table_rows, head_dim * 2, INT64_MAX) || !mul_fits(n, head_dim * 2, INT64_MAX))
    return ENGRAM_EINVAL;
  if (n == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr || d_table == nullptr || d_out == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_table) || !aligned16(d_out)) return ENGRAM_EALIGN;

  const int64_t cpr = head_dim / 8;
  const int64_t total = n * cpr;
  const int64_t per_block = (int64_t)kGatherThreads * kUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  if (blocks > INT32_MAX) return ENGRAM_EINVAL;

  const u32x4 *tab = static_cast<const u32x4 *>(d_table);
  u32x4 *out = static_cast<u32x4 *>(d_out);
  hipStream_t s = as_stream(stream);
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
