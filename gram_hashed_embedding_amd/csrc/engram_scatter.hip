// engram_scatter.hip -- backward of the row gather for gfx950: per-row sums
// of bf16 gradient rows, written into a dense fp32 gradient table or
// emitted row-sparse.
//
// What is computed follows the NeMo AutoModel v0.7 API page
// "qwen3_8_flash_next.engram" (Qwen3_8_FlashNextOwnerShardedEmbedding: the
// owner alone accumulates a row's gradient), the prime-rl pull request 3434
// Validation section (backward gradient aggregation per row) and the prime-rl
// v0.9.1.dev179 release notes, Validation (FP32 reduction defaults).  The
// pages do not fix the summation order or precision; the reading taken here:
// each row's contributions are summed in fp64, rounded once to fp32, and
// added to the fp32 gradient row with one fp32 add.  Sums of bf16 values are
// exact in fp64 unless their bits span more than 53 places, so the result
// does not depend on the order in which the GPU adds them.
//
// Sorted (deterministic) path, all on the caller's stream:
//  1. LSD radix sort of (row, flat index) pairs, key width = bit width of
//     table_rows, at most 8 bits per pass.  Per pass: an upsweep counts each
//     4096-key tile's digits; a two-kernel scan turns the digit-major count
//     matrix into output offsets; a downsweep ranks every key inside its
//     tile with a wavefront multi-split (one ballot per digit bit yields the
//     mask of lanes holding the same digit, its popcount the stable rank)
//     and scatters keys and indices.  The first pass reads the int64 ids
//     directly: valid rows become 32-bit keys, padding and invalid ids the
//     key table_rows, which sorts last and is dropped.
//  2. Segment heads (first position of each distinct row) are counted per
//     32-position range and scanned: the scan gives every distinct row its
//     output slot u, and U itself.
//  3. Range walkers: a group of head_dim/8 lanes (16 bytes of the row per
//     lane) walks one 32-position range of the sorted order, loading the
//     gradient rows in sorted order (eight in flight per lane) and keeping
//     fp64 sums in registers.  A run that starts and ends inside the range
//     is written once (dense read-modify-write or row-sparse store).  A run
//     cut by a range boundary leaves fp64 partials; a fix-up pass, owned by
//     the range holding the run's first position, adds them in range order
//     and writes the row.  No work item waits on another, and hot rows
//     (hundreds of contributions) are spread over many walkers instead of
//     serialising one.
// Atomic path: one fp32 atomic add per gradient element into the dense
// table (hardware float atomics in L2); order of additions not fixed.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per tile
constexpr int kMaxBins = 256;
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanChunk = kScanThreads * kScanItems;
constexpr int kRange = 32;  // sorted positions per walker
constexpr int kWalkThreads = 256;
constexpr int kWalkUnroll = 8;
constexpr int kAtomicThreads = 256;
constexpr int kAtomicUnroll = 4;

static_assert(kRange == 32, "range_heads_kernel splits each wavefront into two ranges");

// ----------------------------------------------------------------- keys ----
// Valid rows keep their index; -1 (padding) and invalid ids get the key
// table_rows, which sorts after every valid row.  Invalid non-padding ids
// add one to `bad`.
__device__ __forceinline__ uint32_t make_key(int64_t id, int64_t table_rows, int &bad) {
  if (id >= 0 && id < table_rows) return (uint32_t)id;
  bad += id != -1 ? 1 : 0;
  return (uint32_t)table_rows;
}

// ------------------------------------------------------------ block scan ---
// Exclusive scan of one value per thread over a 256-thread block.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t &total) {
  __shared__ uint32_t s_wave[kScanThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / kWave; ++w) {
    const uint32_t t = s_wave[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// Scan, step 1: the sum of every kScanChunk-element chunk.
__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(const uint32_t *in, int64_t m,
                                                                    uint32_t *chunk_sums) {
  const int64_t base = (int64_t)blockIdx.x * kScanChunk;
  uint32_t s = 0;
  for (int i = 0; i < kScanItems; ++i) {
    const int64_t p = base + (int64_t)i * kScanThreads + threadIdx.x;
    if (p < m) s += in[p];
  }
  uint32_t total;
  block_exclusive_scan(s, total);
  if (threadIdx.x == 0) chunk_sums[blockIdx.x] = total;
}

// Scan, step 2: each chunk adds the sums of the chunks before it (at most a
// few hundred) and writes its exclusive prefix.  The last chunk also writes
// the grand total (as uint32 and/or int64) when asked.
__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(
    const uint32_t *in, uint32_t *out, int64_t m, const uint32_t *chunk_sums, uint32_t *total32,
    int64_t *total64) {
  uint32_t carry = 0;
  for (int64_t b = threadIdx.x; b < (int64_t)blockIdx.x; b += kScanThreads) carry += chunk_sums[b];
  uint32_t carry_total;
  block_exclusive_scan(carry, carry_total);

  const int64_t base = (int64_t)blockIdx.x * kScanChunk + (int64_t)threadIdx.x * kScanItems;
  uint32_t v[kScanItems];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    v[i] = base + i < m ? in[base + i] : 0u;
    s += v[i];
  }
  uint32_t block_total;
  uint32_t run = carry_total + block_exclusive_scan(s, block_total);
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    if (base + i < m) out[base + i] = run;
    run += v[i];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    const uint32_t grand = carry_total + block_total;
    if (total32 != nullptr) *total32 = grand;
    if (total64 != nullptr) *total64 = (int64_t)grand;
  }
}

// ------------------------------------------------------------ radix sort ---
template <bool FROM_IDS>
__global__ __launch_bounds__(kSortThreads) void radix_upsweep_kernel(
    const int64_t *ids, const uint32_t *keys, int64_t n, int64_t table_rows, int shift,
    uint32_t mask, uint32_t *counts, int64_t num_tiles, int64_t *err) {
  __shared__ uint32_t hist[kMaxBins];
  const int tid = threadIdx.x;
  for (int d = tid; d <= (int)mask; d += kSortThreads) hist[d] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kSortTile;
  int bad = 0;
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t p = base + (int64_t)i * kSortThreads + tid;
    if (p < n) {
      const uint32_t k = FROM_IDS ? make_key(ids[p], table_rows, bad) : keys[p];
      atomicAdd(&hist[(k >> shift) & mask], 1u);
    }
  }
  if (FROM_IDS) count_errors(bad, err);
  __syncthreads();
  for (int d = tid; d <= (int)mask; d += kSortThreads)
    counts[(int64_t)d * num_tiles + blockIdx.x] = hist[d];
}

// Stable scatter of one tile.  Wave w owns tile positions
// [w * 1024, (w + 1) * 1024), read in 16 rounds of 64 consecutive keys, so
// (wave, round, lane) is the original order.
template <bool FROM_IDS>
__global__ __launch_bounds__(kSortThreads) void radix_downsweep_kernel(
    const int64_t *ids, const uint32_t *keys_in, const uint32_t *vals_in, int64_t n,
    int64_t table_rows, int shift, int bits, const uint32_t *offsets, int64_t num_tiles,
    uint32_t *keys_out, uint32_t *vals_out) {
  __shared__ uint32_t s_hist[kSortWaves][kMaxBins];
  const uint32_t mask = (1u << bits) - 1u;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  for (int d = tid; d < kSortWaves * kMaxBins; d += kSortThreads) (&s_hist[0][0])[d] = 0;
  __syncthreads();

  const int64_t base = (int64_t)blockIdx.x * kSortTile + (int64_t)wave * (kSortItems * kWave);
  const unsigned long long below = (1ull << lane) - 1ull;
  uint32_t key[kSortItems], val[kSortItems], rank[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t p = base + (int64_t)i * kWave + lane;
    const bool valid = p < n;
    int ignored = 0;
    if (FROM_IDS) {
      key[i] = valid ? make_key(ids[p], table_rows, ignored) : 0u;
      val[i] = (uint32_t)p;
    } else {
      key[i] = valid ? keys_in[p] : 0u;
      val[i] = valid ? vals_in[p] : 0u;
    }
    rank[i] = 0;
  }
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t p = base + (int64_t)i * kWave + lane;
    const bool valid = p < n;
    const uint32_t d = (key[i] >> shift) & mask;
    unsigned long long peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (d >> b) & 1u;
      const unsigned long long bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    if (valid) {
      const uint32_t prior = s_hist[wave][d];
      rank[i] = prior + (uint32_t)__popcll(peers & below);
      if ((peers & below) == 0ull) s_hist[wave][d] = prior + (uint32_t)__popcll(peers);
    }
  }
  __syncthreads();
  for (int d = tid; d <= (int)mask; d += kSortThreads) {
    uint32_t run = offsets[(int64_t)d * num_tiles + blockIdx.x];
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = s_hist[w][d];
      s_hist[w][d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t p = base + (int64_t)i * kWave + lane;
    if (p < n) {
      const uint32_t d = (key[i] >> shift) & mask;
      const uint32_t dst = s_hist[wave][d] + rank[i];
      keys_out[dst] = key[i];
      vals_out[dst] = val[i];
    }
  }
}

// --------------------------------------------------------- segment heads ---
__global__ __launch_bounds__(256) void range_heads_kernel(const uint32_t *keys, int64_t n,
                                                          uint32_t sentinel, uint32_t *head_count,
                                                          int64_t num_ranges) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool head = false;
  if (j < n) {
    const uint32_t k = keys[j];
    head = k != sentinel && (j == 0 || keys[j - 1] != k);
  }
  const unsigned long long m = __ballot(head);
  const int lane = __lane_id();
  if ((lane & (kRange - 1)) == 0) {
    const int64_t r = j / kRange;
    const unsigned long long half = lane == 0 ? (m & 0xffffffffull) : (m >> 32);
    if (r < num_ranges) head_count[r] = (uint32_t)__popcll(half);
  }
}

// ---------------------------------------------------------- range walkers --
struct WalkArgs {
  const uint32_t *keys;  // sorted rows (sentinel last)
  const uint32_t *vals;  // flat index of each sorted row
  int64_t n;
  uint32_t sentinel;
  const u32x4 *grads;  // [n, cpr] chunks of 8 bf16
  int64_t cpr;         // head_dim / 8
  int64_t dim;
  const uint32_t *head_count;
  const uint32_t *head_off;
  int64_t num_ranges;
  float *grad_table;     // dense output
  int64_t *unique_ids;   // row-sparse output
  float *unique_grads;
  double *pfirst;  // [num_ranges, dim]: run entering the range from before
  double *plast;   // [num_ranges, dim]: run leaving the range, started in it
};

template <int CPL>
__device__ __forceinline__ void zero_acc(double (&acc)[CPL][8]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.0;
}

template <int CPL>
__device__ __forceinline__ void add_chunk(double (&acc)[CPL][8], const u32x4 (&g)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float f[8];
    unpack_bf16x8(g[c], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] += (double)f[e];
  }
}

template <int L, int CPL>
__device__ __forceinline__ void store_partial(double *buf, int64_t r, const WalkArgs &a, int lane,
                                              const double (&acc)[CPL][8]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t col = lane + (int64_t)c * L;
    if (col < a.cpr) {
      f64x2 *dst = reinterpret_cast<f64x2 *>(buf + r * a.dim + col * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = f64x2{acc[c][2 * e], acc[c][2 * e + 1]};
    }
  }
}

template <int L, int CPL>
__device__ __forceinline__ void add_partial(const double *buf, int64_t r, const WalkArgs &a,
                                            int lane, double (&acc)[CPL][8]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t col = lane + (int64_t)c * L;
    if (col < a.cpr) {
      const f64x2 *src = reinterpret_cast<const f64x2 *>(buf + r * a.dim + col * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f64x2 v = src[e];
        acc[c][2 * e] += v.x;
        acc[c][2 * e + 1] += v.y;
      }
    }
  }
}

// The finished sum of row `key` (distinct-row slot u): one rounding to fp32,
// then one fp32 add into the dense table, or a row-sparse store.
template <int L, int CPL, bool SPARSE>
__device__ __forceinline__ void emit_row(uint32_t key, uint32_t u, const WalkArgs &a, int lane,
                                         const double (&acc)[CPL][8]) {
  if (SPARSE && lane == 0) a.unique_ids[u] = (int64_t)key;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t col = lane + (int64_t)c * L;
    if (col >= a.cpr) continue;
    f32x4 s0 = {(float)acc[c][0], (float)acc[c][1], (float)acc[c][2], (float)acc[c][3]};
    f32x4 s1 = {(float)acc[c][4], (float)acc[c][5], (float)acc[c][6], (float)acc[c][7]};
    if (SPARSE) {
      f32x4 *dst = reinterpret_cast<f32x4 *>(a.unique_grads + (int64_t)u * a.dim + col * 8);
      __builtin_nontemporal_store(s0, dst);
      __builtin_nontemporal_store(s1, dst + 1);
    } else {
      f32x4 *dst = reinterpret_cast<f32x4 *>(a.grad_table + (int64_t)key * a.dim + col * 8);
      const f32x4 g0 = dst[0], g1 = dst[1];
      dst[0] = g0 + s0;
      dst[1] = g1 + s1;
    }
  }
}

template <int L, int CPL, bool SPARSE>
__global__ __launch_bounds__(kWalkThreads) void segment_reduce_kernel(const WalkArgs a) {
  const int lane = threadIdx.x % L;
  const int64_t w = ((int64_t)blockIdx.x * kWalkThreads + threadIdx.x) / L;
  if (w >= a.num_ranges) return;
  const int64_t beg = w * kRange;
  const int64_t end = min(a.n, beg + kRange);
  const uint32_t first = a.keys[beg];
  if (first == a.sentinel) return;  // only padding / invalid ids from here on
  const bool left_open = beg > 0 && a.keys[beg - 1] == first;

  uint32_t u = a.head_off[w];
  uint32_t cur = first;
  bool first_run = true;
  bool done = false;
  double acc[CPL][8];
  zero_acc<CPL>(acc);

  for (int64_t j0 = beg; j0 < end && !done; j0 += kWalkUnroll) {
    uint32_t kk[kWalkUnroll];
    u32x4 g[kWalkUnroll][CPL];
#pragma unroll
    for (int q = 0; q < kWalkUnroll; ++q) kk[q] = j0 + q < end ? a.keys[j0 + q] : a.sentinel;
#pragma unroll
    for (int q = 0; q < kWalkUnroll; ++q) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) g[q][c] = u32x4{0u, 0u, 0u, 0u};
      if (kk[q] != a.sentinel) {
        const int64_t src = (int64_t)a.vals[j0 + q] * a.cpr;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int64_t col = lane + (int64_t)c * L;
          if (col < a.cpr) g[q][c] = a.grads[src + col];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kWalkUnroll; ++q) {
      if (done) continue;
      if (kk[q] == a.sentinel) {
        done = true;
        continue;
      }
      if (kk[q] != cur) {  // a new distinct row starts at j0 + q
        if (first_run && left_open) {
          store_partial<L, CPL>(a.pfirst, w, a, lane, acc);
        } else {
          emit_row<L, CPL, SPARSE>(cur, u, a, lane, acc);
          ++u;
        }
        cur = kk[q];
        first_run = false;
        zero_acc<CPL>(acc);
      }
      add_chunk<CPL>(acc, g[q]);
    }
  }
  const bool right_open = end < a.n && a.keys[end] == cur;
  if (first_run && left_open)
    store_partial<L, CPL>(a.pfirst, w, a, lane, acc);
  else if (right_open)
    store_partial<L, CPL>(a.plast, w, a, lane, acc);
  else
    emit_row<L, CPL, SPARSE>(cur, u, a, lane, acc);
}

// Rows cut by range boundaries: the range holding the row's first position
// adds its own partial and the entering partials of the following ranges,
// in order, and writes the row.
template <int L, int CPL, bool SPARSE>
__global__ __launch_bounds__(kWalkThreads) void segment_fixup_kernel(const WalkArgs a) {
  const int lane = threadIdx.x % L;
  const int64_t w = ((int64_t)blockIdx.x * kWalkThreads + threadIdx.x) / L;
  if (w >= a.num_ranges) return;
  const int64_t end = min(a.n, (w + 1) * kRange);
  const uint32_t heads = a.head_count[w];
  if (heads == 0 || end >= a.n) return;
  const uint32_t key = a.keys[end - 1];
  if (key == a.sentinel || a.keys[end] != key) return;

  double acc[CPL][8];
  zero_acc<CPL>(acc);
  add_partial<L, CPL>(a.plast, w, a, lane, acc);
  for (int64_t q = w + 1; q < a.num_ranges; ++q) {
    add_partial<L, CPL>(a.pfirst, q, a, lane, acc);
    const int64_t qend = min(a.n, (q + 1) * kRange);
    const bool passes_through = a.head_count[q] == 0 && qend < a.n && a.keys[qend] == key;
    if (!passes_through) break;
  }
  emit_row<L, CPL, SPARSE>(key, a.head_off[w] + heads - 1, a, lane, acc);
}

__global__ void write_zero_kernel(int64_t *p) { *p = 0; }

// ---------------------------------------------------------------- atomic ---
template <int LOG2_CPR>
__global__ __launch_bounds__(kAtomicThreads) void scatter_atomic_kernel(
    const int64_t *__restrict__ ids, int64_t n, const u32x4 *__restrict__ grads, int64_t cpr,
    float *grad_table, int64_t table_rows, int64_t *err) {
  const int64_t total = n * cpr;
  const int64_t base = (int64_t)blockIdx.x * (kAtomicThreads * kAtomicUnroll) + threadIdx.x;
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kAtomicUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kAtomicThreads;
    if (c >= total) continue;
    int64_t i, j;
    if (LOG2_CPR >= 0) {
      i = c >> LOG2_CPR;
      j = c & ((1 << (LOG2_CPR < 0 ? 0 : LOG2_CPR)) - 1);
    } else {
      i = c / cpr;
      j = c - i * cpr;
    }
    const int64_t r = ids[i];
    if (r >= 0 && r < table_rows) {
      float f[8];
      unpack_bf16x8(grads[c], f);
      float *dst = grad_table + (r * cpr + j) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) unsafeAtomicAdd(dst + e, f[e]);
    } else {
      bad += (j == 0 && r != -1) ? 1 : 0;
    }
  }
  count_errors(bad, err);
}

// ------------------------------------------------------------------ host ---
struct Plan {
  int64_t num_tiles, num_ranges, scan_chunks;
  int bits, passes, per_pass;
  size_t keys_a, vals_a, keys_b, vals_b, counts, chunk_sums, head_count, head_off, scalars,
      pfirst, plast, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int bit_width_u64(uint64_t x) {
  int b = 0;
  while (x != 0) {
    ++b;
    x >>= 1;
  }
  return b;
}

// Checks shared by every mode; fills the sorted-path workspace plan.
bool make_plan(int64_t n, int64_t table_rows, int64_t dim, Plan *p) {
  if (n < 0 || table_rows < 0 || dim <= 0 || dim % 8 != 0 || dim > 2048) return false;
  if (!mul_fits(n, dim * 8, INT64_MAX / 4) || !mul_fits(table_rows, dim * 4, INT64_MAX))
    return false;
  p->num_tiles = (n + kSortTile - 1) / kSortTile;
  p->num_ranges = (n + kRange - 1) / kRange;
  const int64_t count_len = (int64_t)kMaxBins * p->num_tiles;
  const int64_t longest = count_len > p->num_ranges ? count_len : p->num_ranges;
  p->scan_chunks = (longest + kScanChunk - 1) / kScanChunk;
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
  const size_t nn = (size_t)n;
  p->keys_a = take(nn * 4);
  p->vals_a = take(nn * 4);
  p->keys_b = take(nn * 4);
  p->vals_b = take(nn * 4);
  p->counts = take((size_t)count_len * 4);
  p->chunk_sums = take((size_t)(p->scan_chunks > 0 ? p->scan_chunks : 1) * 4);
  p->head_count = take((size_t)p->num_ranges * 4);
  p->head_off = take((size_t)p->num_ranges * 4);
  p->scalars = take(64);
  p->pfirst = take((size_t)p->num_ranges * (size_t)dim * 8);
  p->plast = take((size_t)p->num_ranges * (size_t)dim * 8);
  p->total = off;
  return true;
}

// The sorted path needs 32-bit keys (table_rows itself is the drop key) and
// 32-bit flat indices.
inline bool sorted_limits_ok(int64_t n, int64_t table_rows) {
  return table_rows < (int64_t)UINT32_MAX && n < (int64_t)UINT32_MAX;
}

void launch_scan(const uint32_t *in, uint32_t *out, int64_t m, uint32_t *chunk_sums,
                 uint32_t *total32, int64_t *total64, hipStream_t s) {
  const unsigned chunks = (unsigned)((m + kScanChunk - 1) / kScanChunk);
  hipLaunchKernelGGL(scan_reduce_kernel, dim3(chunks), dim3(kScanThreads), 0, s, in, m,
                     chunk_sums);
  hipLaunchKernelGGL(scan_apply_kernel, dim3(chunks), dim3(kScanThreads), 0, s, in, out, m,
                     chunk_sums, total32, total64);
}

template <int L, int CPL, bool SPARSE>
void launch_walkers(const WalkArgs &a, hipStream_t s) {
  const int64_t threads = a.num_ranges * L;
  const unsigned blocks = (unsigned)((threads + kWalkThreads - 1) / kWalkThreads);
  hipLaunchKernelGGL((segment_reduce_kernel<L, CPL, SPARSE>), dim3(blocks), dim3(kWalkThreads), 0,
                     s, a);
  hipLaunchKernelGGL((segment_fixup_kernel<L, CPL, SPARSE>), dim3(blocks), dim3(kWalkThreads), 0,
                     s, a);
}

template <bool SPARSE>
void dispatch_walkers(const WalkArgs &a, hipStream_t s) {
  const int64_t cpr = a.cpr;
  if (cpr <= 1) launch_walkers<1, 1, SPARSE>(a, s);
  else if (cpr <= 2) launch_walkers<2, 1, SPARSE>(a, s);
  else if (cpr <= 4) launch_walkers<4, 1, SPARSE>(a, s);
  else if (cpr <= 8) launch_walkers<8, 1, SPARSE>(a, s);
  else if (cpr <= 16) launch_walkers<16, 1, SPARSE>(a, s);
  else if (cpr <= 32) launch_walkers<32, 1, SPARSE>(a, s);
  else if (cpr <= 64) launch_walkers<64, 1, SPARSE>(a, s);
  else if (cpr <= 128) launch_walkers<64, 2, SPARSE>(a, s);
  else launch_walkers<64, 4, SPARSE>(a, s);
}

int sorted_scatter(const int64_t *ids, int64_t n, const void *grads, int64_t dim,
                   int64_t table_rows, bool sparse, float *grad_table, int64_t *unique_ids,
                   float *unique_grads, int64_t *num_unique, void *ws, size_t ws_bytes,
                   int64_t *err, hipStream_t s) {
  Plan p;
  if (!make_plan(n, table_rows, dim, &p) || !sorted_limits_ok(n, table_rows))
    return ENGRAM_EINVAL;
  if (ws == nullptr || ws_bytes < p.total) return ENGRAM_EWORKSPACE;
  char *base = static_cast<char *>(ws);
  uint32_t *keys_a = reinterpret_cast<uint32_t *>(base + p.keys_a);
  uint32_t *vals_a = reinterpret_cast<uint32_t *>(base + p.vals_a);
  uint32_t *keys_b = reinterpret_cast<uint32_t *>(base + p.keys_b);
  uint32_t *vals_b = reinterpret_cast<uint32_t *>(base + p.vals_b);
  uint32_t *counts = reinterpret_cast<uint32_t *>(base + p.counts);
  uint32_t *chunk_sums = reinterpret_cast<uint32_t *>(base + p.chunk_sums);
  uint32_t *head_count = reinterpret_cast<uint32_t *>(base + p.head_count);
  uint32_t *head_off = reinterpret_cast<uint32_t *>(base + p.head_off);
  double *pfirst = reinterpret_cast<double *>(base + p.pfirst);
  double *plast = reinterpret_cast<double *>(base + p.plast);

  // 1. radix sort (ping-pong a <-> b; the first pass reads the ids)
  const uint32_t *src_k = nullptr, *src_v = nullptr;
  uint32_t *dst_k = keys_a, *dst_v = vals_a, *spare_k = keys_b, *spare_v = vals_b;
  const unsigned tiles = (unsigned)p.num_tiles;
  for (int pass = 0; pass < p.passes; ++pass) {
    const int shift = pass * p.per_pass;
    const int width = p.bits - shift < p.per_pass ? p.bits - shift : p.per_pass;
    const uint32_t mask = (1u << width) - 1u;
    const int64_t bins = (int64_t)mask + 1;
    if (pass == 0)
      hipLaunchKernelGGL(radix_upsweep_kernel<true>, dim3(tiles), dim3(kSortThreads), 0, s, ids,
                         nullptr, n, table_rows, shift, mask, counts, p.num_tiles, err);
    else
      hipLaunchKernelGGL(radix_upsweep_kernel<false>, dim3(tiles), dim3(kSortThreads), 0, s,
                         nullptr, src_k, n, table_rows, shift, mask, counts, p.num_tiles,
                         nullptr);
    launch_scan(counts, counts, bins * p.num_tiles, chunk_sums, nullptr, nullptr, s);
    if (pass == 0)
      hipLaunchKernelGGL(radix_downsweep_kernel<true>, dim3(tiles), dim3(kSortThreads), 0, s,
                         ids, nullptr, nullptr, n, table_rows, shift, width, counts,
                         p.num_tiles, dst_k, dst_v);
    else
      hipLaunchKernelGGL(radix_downsweep_kernel<false>, dim3(tiles), dim3(kSortThreads), 0, s,
                         nullptr, src_k, src_v, n, table_rows, shift, width, counts,
                         p.num_tiles, dst_k, dst_v);
    src_k = dst_k;
    src_v = dst_v;
    uint32_t *tk = dst_k, *tv = dst_v;
    dst_k = spare_k;
    dst_v = spare_v;
    spare_k = tk;
    spare_v = tv;
  }

  // 2. distinct-row slots
  const uint32_t sentinel = (uint32_t)table_rows;
  const unsigned head_blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(range_heads_kernel, dim3(head_blocks), dim3(256), 0, s, src_k, n, sentinel,
                     head_count, p.num_ranges);
  launch_scan(head_count, head_off, p.num_ranges, chunk_sums, nullptr,
              sparse ? num_unique : nullptr, s);

  // 3. range walkers + fix-up
  WalkArgs a;
  a.keys = src_k;
  a.vals = src_v;
  a.n = n;
  a.sentinel = sentinel;
  a.grads = static_cast<const u32x4 *>(grads);
  a.cpr = dim / 8;
  a.dim = dim;
  a.head_count = head_count;
  a.head_off = head_off;
  a.num_ranges = p.num_ranges;
  a.grad_table = grad_table;
  a.unique_ids = unique_ids;
  a.unique_grads = unique_grads;
  a.pfirst = pfirst;
  a.plast = plast;
  if (sparse)
    dispatch_walkers<true>(a, s);
  else
    dispatch_walkers<false>(a, s);
  return launch_status();
}

int atomic_scatter(const int64_t *ids, int64_t n, const void *grads, int64_t dim,
                   float *grad_table, int64_t table_rows, int64_t *err, hipStream_t s) {
  const int64_t cpr = dim / 8;
  const int64_t total = n * cpr;
  const int64_t per_block = (int64_t)kAtomicThreads * kAtomicUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  if (blocks > INT32_MAX) return ENGRAM_EINVAL;
  const u32x4 *g = static_cast<const u32x4 *>(grads);
  const dim3 grid((unsigned)blocks), block(kAtomicThreads);
  switch (cpr) {
#define ENGRAM_ATOMIC_CASE(L2)                                                                  \
  case (1 << L2):                                                                               \
    hipLaunchKernelGGL(scatter_atomic_kernel<L2>, grid, block, 0, s, ids, n, g, cpr, grad_table, \
                       table_rows, err);                                                        \
    break;
    ENGRAM_ATOMIC_CASE(0)
    ENGRAM_ATOMIC_CASE(1)
    ENGRAM_ATOMIC_CASE(2)
    ENGRAM_ATOMIC_CASE(3)
    ENGRAM_ATOMIC_CASE(4)
    ENGRAM_ATOMIC_CASE(5)
    ENGRAM_ATOMIC_CASE(6)
    ENGRAM_ATOMIC_CASE(7)
    ENGRAM_ATOMIC_CASE(8)
#undef ENGRAM_ATOMIC_CASE
    default:
      hipLaunchKernelGGL(scatter_atomic_kernel<-1>, grid, block, 0, s, ids, n, g, cpr,
                         grad_table, table_rows, err);
  }
  return launch_status();
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" size_t engram_scatter_add_workspace(int64_t n, int64_t table_rows, int64_t head_dim,
                                               int32_t mode) {
  Plan p;
  if (!make_plan(n, table_rows, head_dim, &p)) return (size_t)-1;
  if (mode == ENGRAM_SCATTER_ATOMIC) return 0;
  if (mode != ENGRAM_SCATTER_SORTED && mode != ENGRAM_SCATTER_ROWSPARSE) return (size_t)-1;
  if (!sorted_limits_ok(n, table_rows)) return (size_t)-1;
  return p.total;
}

extern "C" int engram_scatter_add(const int64_t *d_row_ids, int64_t n, const void *d_grads,
                                  int64_t head_dim, float *d_grad_table, int64_t table_rows,
                                  int32_t mode, void *d_workspace, size_t workspace_bytes,
                                  int64_t *d_err_count, void *stream) {
  Plan p;
  if (!make_plan(n, table_rows, head_dim, &p)) return ENGRAM_EINVAL;
  if (mode != ENGRAM_SCATTER_SORTED && mode != ENGRAM_SCATTER_ATOMIC) return ENGRAM_EINVAL;
  if (mode == ENGRAM_SCATTER_SORTED && !sorted_limits_ok(n, table_rows)) return ENGRAM_EINVAL;
  if (n == 0) return ENGRAM_OK;
  if (d_row_ids == nullptr || d_grads == nullptr || d_grad_table == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_grad_table)) return ENGRAM_EALIGN;
  hipStream_t s = as_stream(stream);
  if (mode == ENGRAM_SCATTER_ATOMIC)
    return atomic_scatter(d_row_ids, n, d_grads, head_dim, d_grad_table, table_rows,
                          d_err_count, s);
  if (!aligned16(d_workspace)) return ENGRAM_EWORKSPACE;
  return sorted_scatter(d_row_ids, n, d_grads, head_dim, table_rows, false, d_grad_table,
                        nullptr, nullptr, nullptr, d_workspace, workspace_bytes, d_err_count, s);
}

extern "C" int engram_scatter_add_rowsparse(const int64_t *d_row_ids, int64_t n,
                                            const void *d_grads, int64_t head_dim,
                                            int64_t table_rows, int64_t *d_unique_ids,
                                            float *d_unique_grads, int64_t *d_num_unique,
                                            void *d_workspace, size_t workspace_bytes,
                                            int64_t *d_err_count, void *stream) {
  Plan p;
  if (!make_plan(n, table_rows, head_dim, &p) || !sorted_limits_ok(n, table_rows))
    return ENGRAM_EINVAL;
  if (d_num_unique == nullptr) return ENGRAM_EINVAL;
  hipStream_t s = as_stream(stream);
  if (n == 0) {
    hipLaunchKernelGGL(write_zero_kernel, dim3(1), dim3(1), 0, s, d_num_unique);
    return launch_status();
  }
  if (d_row_ids == nullptr || d_grads == nullptr || d_unique_ids == nullptr ||
      d_unique_grads == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_unique_grads)) return ENGRAM_EALIGN;
  if (!aligned16(d_workspace)) return ENGRAM_EWORKSPACE;
  return sorted_scatter(d_row_ids, n, d_grads, head_dim, table_rows, true, nullptr, d_unique_ids,
                        d_unique_grads, d_num_unique, d_workspace, workspace_bytes, d_err_count,
                        s);
}
