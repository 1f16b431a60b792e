// engram_sort.hip -- the plan of the sorted scatter-add for gfx950: the
// lookups' row ids sorted, and every distinct row given its output slot.
//
// What the backward computes follows the NeMo AutoModel v0.7 API page
// "qwen3_8_flash_next.engram" (Qwen3_8_FlashNextOwnerShardedEmbedding: the
// owner alone accumulates a row's gradient), the prime-rl pull request 3434
// Validation section (backward gradient aggregation per row) and the prime-rl
// v0.9.1.dev179 release notes, Validation (FP32 reduction defaults).  The
// plan is the part that needs only the row ids (or the tokens they are hashed
// from); engram_apply_*.hip sum the gradients by it.
//
//  1. LSD radix sort of (row, flat index) pairs, key width = bit width of
//     table_rows, at most 8 bits per pass, one kernel per pass: the one-sweep
//     radix sort (one global digit histogram up front, then per pass each
//     tile ranks its keys, publishes its per-digit counts and finds its
//     output offsets by decoupled look-back over earlier tiles' counts).
//     Each 4096-key tile ranks its keys with a wavefront multi-split (one
//     ballot per digit bit yields the mask of lanes holding the same digit,
//     its popcount the stable rank) and writes its keys and indices in
//     coalesced digit runs staged through LDS.  The first pass reads the
//     int64 ids directly: valid rows become 32-bit keys, padding and invalid
//     ids the key table_rows, which sorts last and is dropped.  A plan made
//     from the tokens first hashes them into 32-bit keys (counting the digits
//     as it goes), and its first pass reads those.  When the heads own
//     disjoint row ranges (as when the offsets pack them back to back) every
//     row belongs to one head, so the keys are laid out and sorted per head:
//     one segment per head, in order of offset, each sorted on the bits of its
//     largest remainder (23 bits for 8.3M-row heads instead of the 28 of a
//     200M-row table: 3 passes instead of 4), with look-back inside the
//     segment.  The segments one after another are the same sorted order a
//     sort of all the keys gives.
//  2. Segment heads (first position of each distinct row) are counted per
//     16-position range and scanned in one kernel (decoupled look-back over
//     tiles of ranges): the scan gives every distinct row its output slot u,
//     and U itself.  The same kernel stamps the workspace with the plan's n
//     and table_rows; the apply checks the stamp (and that no wait of the
//     plan expired) before it reads the plan.
#include "engram_hash_dev.h"
#include "engram_scatter_dev.h"

namespace engram {
namespace {

constexpr int kSortWaves = kSortThreads / kWave;
// A sort with fewer tiles than this takes tiles of half the size: twice the
// blocks on a GPU of 256 compute units, and half a tile's serial work each.
constexpr int64_t kSmallSortTiles = 128;
static_assert(kWave % kRange == 0 && kRange % 4 == 0, "ranges tile a wavefront");

// ----------------------------------------------------------------- keys ----
// Valid rows keep their index; -1 (padding) and invalid ids get the key
// table_rows, which sorts after every valid row.  Invalid non-padding ids
// add one to `bad`.
__device__ __forceinline__ uint32_t make_key(int64_t id, int64_t table_rows, int &bad) {
  if (id >= 0 && id < table_rows) return (uint32_t)id;
  bad += id != -1 ? 1 : 0;
  return (uint32_t)table_rows;
}

// Segments of a sort: the keys are sorted within `count` consecutive segments
// of `len` keys each.  A plan from ids, or from tokens whose heads' row ranges
// overlap, has one segment of all n keys.  A plan from tokens whose heads own
// disjoint row ranges sorts each head's keys on their own: segment s holds head
// head[s]'s rows in token order, the heads ordered by row offset, so the
// segments one after another are sorted as a whole.  A key's digits are taken
// from key - base[s] (base[s] = the head's offset), so the sort needs only the
// bits of the largest prime, and a tile's look-back stops at its segment's
// first tile.
struct SortSegs {
  int64_t len;     // keys per segment
  int64_t tiles;   // tiles per segment
  int32_t count;   // segments
  int32_t copies;  // copies of each segment's digit totals
  int32_t stride;  // the key at position t of segment s has flat index t * stride + head[s]
  int32_t pad;
  uint32_t base[ENGRAM_MAX_HEADS];
  uint32_t head[ENGRAM_MAX_HEADS];
};


// ------------------------------------------------------------ block scan ---
// Exclusive scan of one value per thread over an NT-thread block.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t &total) {
  __shared__ uint32_t s_wave[NT / kWave];
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
  for (int w = 0; w < NT / kWave; ++w) {
    const uint32_t t = s_wave[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// ------------------------------------------------------------ radix sort ---
// One-sweep LSD radix sort.  One kernel clears the look-back state, one
// counts every pass's digits over each segment's keys (a segment's digit
// totals of a pass do not depend on the order its keys are in), then one
// kernel per pass: a block takes the next tile by atomic ticket, ranks its
// keys with a wavefront multi-split, publishes its per-digit counts, learns
// the counts of its segment's earlier tiles by decoupled look-back, stages
// the tile in LDS in sorted order and writes it out in coalesced runs.
constexpr uint64_t kFlagAggregate = 1ull << 32;  // count of this tile only
constexpr uint64_t kFlagInclusive = 2ull << 32;  // count of the segment's tiles up to this
constexpr uint32_t kSpinLimit = 1u << 22;        // bound on every look-back wait
constexpr int kLookBatch = 4;                     // predecessor tiles read per look-back step

__global__ __launch_bounds__(256) void sort_clear_kernel(uint64_t *status, int64_t status_len,
                                                         uint32_t *counters, int counters_len,
                                                         PlanScalars *plan) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < status_len) status[i] = 0;
  if (i < counters_len) counters[i] = 0;
  if (i == 0) *plan = PlanScalars{};  // no complete plan until the last kernel stamps it
}

// hist[copy][pass][digit] += number of keys with that digit (digits from bit
// `lo` up).  One block per kSortTile ids, all of a thread's loads in flight
// before any is counted.
__global__ __launch_bounds__(kSortThreads) void sort_histogram_kernel(
    const int64_t *ids, int64_t n, int64_t table_rows, int passes, int per_pass, int bits,
    int lo, uint32_t *hist, int64_t *err) {
  __shared__ uint32_t s_hist[4][kMaxBins];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kSortTile + tid;
  int64_t id[kSortItems];  // loads at clamped positions, so none waits behind a branch
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) id[i] = ids[min(base + (int64_t)i * kSortThreads, n - 1)];
  for (int d = tid; d < 4 * kMaxBins; d += kSortThreads) (&s_hist[0][0])[d] = 0;
  __syncthreads();
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    if (base + (int64_t)i * kSortThreads >= n) continue;
    const uint32_t k = make_key(id[i], table_rows, bad);
    for (int q = 0; q < passes; ++q) {
      const int shift = lo + q * per_pass;
      const int width = bits - shift < per_pass ? bits - shift : per_pass;
      atomicAdd(&s_hist[q][(k >> shift) & ((1u << width) - 1u)], 1u);
    }
  }
  count_errors(bad, err);
  __syncthreads();
  uint32_t *copy = hist + (int64_t)(blockIdx.x % kHistCopies) * 4 * kMaxBins;
  for (int d = tid; d < passes * kMaxBins; d += kSortThreads) {
    const uint32_t c = (&s_hist[0][0])[d];
    if (c != 0) atomicAdd(&copy[d], c);
  }
}

// Where a sort pass takes its input from.
constexpr int kSrcIds = 0;        // int64 row ids (first pass of a plan from ids)
constexpr int kSrcKeys = 1;       // 32-bit keys and flat indices (later passes)
constexpr int kSrcKeysIota = 2;   // 32-bit keys in flat order (first pass of a plan from tokens)

template <int SRC, int ITEMS>
__global__ __launch_bounds__(kSortThreads) void onesweep_kernel(
    const int64_t *ids, const uint32_t *keys_in, const uint32_t *vals_in, const SortSegs sg,
    int64_t table_rows, int shift, int bits, const uint32_t *hist, uint64_t *status,
    uint32_t *ticket, uint32_t *keys_out, uint32_t *vals_out, PlanScalars *plan, int64_t *err) {
  constexpr int TILE = kSortThreads * ITEMS;
  __shared__ uint32_t s_keys[TILE];
  __shared__ uint32_t s_vals[TILE];
  __shared__ uint32_t s_cnt[kSortWaves][kMaxBins];  // per-wave counts -> wave offsets
  __shared__ uint32_t s_local[kMaxBins];            // tile-local start of each digit
  __shared__ uint32_t s_gbase[kMaxBins];            // global position of tile-local 0
  __shared__ uint32_t s_tile;
  const uint32_t mask = (1u << bits) - 1u;
  const int bins = 1 << bits;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  if (tid == 0) s_tile = atomicAdd(ticket, 1u);
  for (int d = tid; d < kSortWaves * kMaxBins; d += kSortThreads) (&s_cnt[0][0])[d] = 0;
  __syncthreads();
  const int64_t tile = s_tile;
  const int64_t seg = tile / sg.tiles;
  const int64_t first = seg * sg.tiles;  // the segment's first tile
  const int64_t seg0 = seg * sg.len;     // and its first key
  const int64_t seg_end = seg0 + sg.len;
  const int64_t tile0 = seg0 + (tile - first) * TILE;
  const int count = (int)min((int64_t)TILE, seg_end - tile0);
  const uint32_t kbase = sg.base[seg];

  // keys of this tile: wave w owns tile positions [w * 1024, (w + 1) * 1024)
  // in 16 rounds of 64, so (wave, round, lane) is the original order; then
  // the segment's digit totals (their latency overlaps the ranking)
  const int64_t base = tile0 + (int64_t)wave * (ITEMS * kWave);
  const unsigned long long below = (1ull << lane) - 1ull;
  // (loads at clamped positions, so none waits behind a branch)
  const uint32_t *seg_hist = hist + seg * 4 * kMaxBins;
  const int64_t copy_stride = (int64_t)sg.count * 4 * kMaxBins;
  uint32_t copies[kHistCopies];
#pragma unroll
  for (int c = 0; c < kHistCopies; ++c)
    copies[c] = c < sg.copies ? seg_hist[c * copy_stride + (tid < bins ? tid : 0)] : 0u;
  uint32_t key[ITEMS], val[ITEMS], rank[ITEMS];
  if (SRC == kSrcIds) {
    int64_t id[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      id[i] = ids[min(base + (int64_t)i * kWave + lane, seg_end - 1)];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t p = base + (int64_t)i * kWave + lane;
      int ignored = 0;
      key[i] = p < seg_end ? make_key(id[i], table_rows, ignored) : 0u;
      val[i] = (uint32_t)p;
    }
  } else {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t p = min(base + (int64_t)i * kWave + lane, seg_end - 1);
      key[i] = keys_in[p];
      val[i] = SRC == kSrcKeysIota ? (uint32_t)((p - seg0) * sg.stride + sg.head[seg])
                                   : vals_in[p];
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (base + (int64_t)i * kWave + lane >= seg_end) key[i] = val[i] = kbase;
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) rank[i] = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t p = base + (int64_t)i * kWave + lane;
    const bool valid = p < seg_end;
    const uint32_t d = ((key[i] - kbase) >> shift) & mask;
    unsigned long long peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (d >> b) & 1u;
      const unsigned long long bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    if (valid) {
      const uint32_t prior = s_cnt[wave][d];
      rank[i] = prior + (uint32_t)__popcll(peers & below);
      if ((peers & below) == 0ull) s_cnt[wave][d] = prior + (uint32_t)__popcll(peers);
    }
  }
  __syncthreads();

  // per digit: tile count, wave offsets; publish the tile's count at once
  uint32_t tile_count = 0;
  if (tid < bins) {
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = s_cnt[w][tid];
      s_cnt[w][tid] = tile_count;
      tile_count += c;
    }
    const uint64_t word = (tile == first ? kFlagInclusive : kFlagAggregate) | tile_count;
    __hip_atomic_store(&status[tile * kMaxBins + tid], word, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // tile-local digit starts, and the segment's digit starts (keys of all
  // smaller digits over the segment's tiles), by block scans over the digits
  uint32_t scan_total;
  const uint32_t local_start =
      block_exclusive_scan<kSortThreads>(tid < bins ? tile_count : 0u, scan_total);
  uint32_t digit_total = 0;
#pragma unroll
  for (int c = 0; c < kHistCopies; ++c) digit_total += tid < bins ? copies[c] : 0u;
  const uint32_t digit_start = block_exclusive_scan<kSortThreads>(digit_total, scan_total);
  // decoupled look-back: the keys of this digit in the segment's earlier tiles
  if (tid < bins) {
    s_local[tid] = local_start;
    uint64_t before = 0;
    bool stalled = false, found = false;
    // look back kLookBatch tiles per step, all loads in flight together
    for (int64_t t = tile - 1; t >= first && !found && !stalled; t -= kLookBatch) {
      uint64_t word[kLookBatch];
#pragma unroll
      for (int j = 0; j < kLookBatch; ++j)
        word[j] = t - j >= first ? __hip_atomic_load(&status[(t - j) * kMaxBins + tid],
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : kFlagInclusive;  // before the segment: nothing
#pragma unroll
      for (int j = 0; j < kLookBatch; ++j) {
        if (found || stalled) continue;
        uint32_t spins = 0;
        while ((word[j] >> 32) == 0) {  // not published yet: wait on this one
          if (++spins == kSpinLimit) break;
          __builtin_amdgcn_s_sleep(1);
          word[j] = __hip_atomic_load(&status[(t - j) * kMaxBins + tid], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
        if ((word[j] >> 32) == 0) {  // the wait expired: give up, flag the call
          stalled = true;
          continue;
        }
        before += word[j] & 0xffffffffull;
        found = (word[j] & kFlagInclusive) != 0;
      }
    }
    if (tile != first)
      __hip_atomic_store(&status[tile * kMaxBins + tid],
                         kFlagInclusive | (uint32_t)(before + tile_count), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (stalled) {
      atomicOr(&plan->stalled, 1u);
      add_mark(err, kStallMark);
    }
    s_gbase[tid] = (uint32_t)seg0 + digit_start + (uint32_t)before;
  }
  __syncthreads();

  // stage in LDS in tile-sorted order, then write digit runs out coalesced
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t p = base + (int64_t)i * kWave + lane;
    if (p < seg_end) {
      const uint32_t d = ((key[i] - kbase) >> shift) & mask;
      const uint32_t at = s_local[d] + s_cnt[wave][d] + rank[i];
      s_keys[at] = key[i];
      s_vals[at] = val[i];
    }
  }
  __syncthreads();
  for (int j = tid; j < count; j += kSortThreads) {
    const uint32_t k = s_keys[j];
    const uint32_t d = ((k - kbase) >> shift) & mask;
    const uint32_t dst = s_gbase[d] + (uint32_t)j - s_local[d];
    keys_out[dst] = k;
    vals_out[dst] = s_vals[j];
  }
}


// ---------------------------------------------------------- plan from tokens
// The first kernel of a plan made from the tokens: the row of every lookup
// is computed as the hash kernel does (64 tokens at a time per block; one
// lane per token computes its order mixes, then the block's 64 * H outputs
// in flat order), written as its 32-bit sort key, and counted into every
// pass's digit histogram.  Hashed rows are always inside the table.
__global__ __launch_bounds__(kSortThreads) void plan_hash_kernel(const HashParams hp,
                                                                 int64_t total_tokens,
                                                                 int passes, int per_pass,
                                                                 int bits, uint32_t *keys,
                                                                 uint32_t *hist) {
  constexpr int kTokens = 64;
  __shared__ uint64_t s_mix[kTokens][ENGRAM_MAX_NGRAM - 1];
  __shared__ uint32_t s_hist[4][kMaxBins];
  const int tid = threadIdx.x;
  for (int d = tid; d < 4 * kMaxBins; d += kSortThreads) (&s_hist[0][0])[d] = 0;
  // (blocks stride over the tokens when there are more than one grid's worth)
  for (int64_t tok0 = (int64_t)blockIdx.x * kTokens; tok0 < total_tokens;
       tok0 += (int64_t)gridDim.x * kTokens) {
    if (tid < kTokens && tok0 + tid < total_tokens) {
      uint64_t mix[ENGRAM_MAX_NGRAM - 1];
      token_mixes(hp, tok0 + tid, mix);
#pragma unroll
      for (int k = 0; k < ENGRAM_MAX_NGRAM - 1; ++k)
        if (k < hp.n - 1) s_mix[tid][k] = mix[k];
    }
    __syncthreads();
    const int ntok = (int)min((int64_t)kTokens, total_tokens - tok0);
    const int nout = ntok * hp.H;
    uint32_t *out = keys + tok0 * hp.H;
    for (int o = tid; o < nout; o += kSortThreads) {
      const int tl = o / hp.H;
      const int h = o - tl * hp.H;
      const uint32_t k = (uint32_t)head_row(hp, s_mix[tl][h / hp.J], h);
      out[o] = k;
      for (int q = 0; q < passes; ++q) {
        const int shift = q * per_pass;
        const int width = bits - shift < per_pass ? bits - shift : per_pass;
        atomicAdd(&s_hist[q][(k >> shift) & ((1u << width) - 1u)], 1u);
      }
    }
    __syncthreads();  // s_mix is rewritten for the next tokens
  }
  uint32_t *copy = hist + (int64_t)(blockIdx.x % kHistCopies) * 4 * kMaxBins;
  for (int d = tid; d < passes * kMaxBins; d += kSortThreads) {
    const uint32_t c = (&s_hist[0][0])[d];
    if (c != 0) atomicAdd(&copy[d], c);
  }
}

// The first kernel of a plan from tokens sorted in per-head segments: a
// block takes kHeadTokens tokens of one head (segment s hashes head head[s];
// a segment is `chunks` blocks), writes each key at its segment's position
// (segment s, token t: s * tokens + t) and counts its digits (of key -
// base[s], from bit `lo` up) into the segment's histograms, one flush per
// block.  A thread takes kHeadItems tokens with all their history loads in
// flight together.
// Blocks of kSortThreads threads, like the sort's, so the plan gets its
// share of the GPU beside a forward running on another stream (blocks of
// 1024 threads wait there for a whole compute unit to drain).  N =
// ngram_size at compile time, as in the fused lookup.
constexpr int kHeadThreads = kSortThreads;
constexpr int kHeadItems = 4;
constexpr int kHeadTokens = kHeadThreads * kHeadItems;

template <int N>
__global__ __launch_bounds__(kHeadThreads) void plan_hash_heads_kernel(
    const HashParams hp, const SortSegs sg, int64_t chunks, int passes, int per_pass, int bits,
    int lo, uint32_t *keys, uint32_t *hist) {
  __shared__ uint32_t s_hist[4][kMaxBins];
  const int tid = threadIdx.x;
  const int64_t seg = blockIdx.x / chunks;
  const int64_t t0 = ((int64_t)blockIdx.x - seg * chunks) * kHeadTokens + tid;
  const int h = (int)sg.head[seg];
  const int order = h / hp.J;  // g - 2
  const uint32_t kbase = sg.base[seg];
  uint32_t *out = keys + seg * sg.len;
  for (int d = tid; d < 4 * kMaxBins; d += kHeadThreads) (&s_hist[0][0])[d] = 0;
  uint64_t mix[kHeadItems][ENGRAM_MAX_NGRAM - 1];
#pragma unroll
  for (int i = 0; i < kHeadItems; ++i)
    token_mixes<N>(hp, min(t0 + (int64_t)i * kHeadThreads, sg.len - 1), mix[i]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHeadItems; ++i) {
    const int64_t t = t0 + (int64_t)i * kHeadThreads;
    if (t >= sg.len) continue;
    uint64_t m = mix[i][0];
#pragma unroll
    for (int k = 1; k < N - 1; ++k) m = order == k ? mix[i][k] : m;
    const uint32_t key = (uint32_t)head_row(hp, m, h);
    out[t] = key;
    for (int q = 0; q < passes; ++q) {
      const int shift = lo + q * per_pass;
      const int width = bits - shift < per_pass ? bits - shift : per_pass;
      atomicAdd(&s_hist[q][((key - kbase) >> shift) & ((1u << width) - 1u)], 1u);
    }
  }
  __syncthreads();
  uint32_t *dst = hist + seg * 4 * kMaxBins;
  for (int d = tid; d < passes * kMaxBins; d += kHeadThreads) {
    const uint32_t c = (&s_hist[0][0])[d];
    if (c != 0) atomicAdd(&dst[d], c);
  }
}

// ---------------------------------------------------- small plan in LDS ---
// A plan from tokens sorted in per-head segments of at most kLdsSortKeys
// keys (a small batch): one block per segment hashes its head's keys, sorts
// them in LDS with the same stable LSD passes as the one-sweep sort (the
// keys in (wave, round, lane) order, ranked by wavefront multi-split, each
// pass's digit offsets by a block scan), and writes the segment's sorted
// keys and flat indices.  The block of segment 0 also clears the slot scan's
// look-back state and the plan's scalars.  One launch does what the clear,
// the hash and one launch per sort pass do for large segments; the slot
// scan follows.  Keys and indices pass through one LDS buffer in turn.
// Measured on MI355X (plan alone, 16 heads): 21.8 against 43.9 us at 1024
// keys per head, 24.2 against 42.9 at 4096, 36.5 against 44.3 at 8192; at
// 16384 keys per head one block per head is slower than the multi-block
// sort (60.4 against 50.8 us), so larger segments take that.
constexpr int kLdsSortThreads = 1024;
constexpr int kLdsSortWaves = kLdsSortThreads / kWave;
constexpr int kLdsSortKeys = kLdsSortThreads * 8;

template <int N, int ITEMS>
__global__ __launch_bounds__(kLdsSortThreads) void plan_heads_lds_kernel(
    const HashParams hp, const SortSegs sg, int passes, int per_pass, int bits,
    uint32_t *keys_out, uint32_t *vals_out, uint64_t *slot_status, int64_t slot_words,
    uint32_t *slot_ticket, PlanScalars *plan) {
  static_assert(kLdsSortThreads * ITEMS <= kLdsSortKeys, "a segment fits the buffer");
  __shared__ uint32_t s_buf[kLdsSortThreads * ITEMS];
  __shared__ uint32_t s_cnt[kLdsSortWaves][kMaxBins];  // per-wave counts -> wave offsets
  __shared__ uint32_t s_local[kMaxBins];               // start of each digit
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t seg = blockIdx.x;
  const int h = (int)sg.head[seg];
  const int order = h / hp.J;  // g - 2
  const uint32_t kbase = sg.base[seg];
  const int len = (int)sg.len;
  if (seg == 0) {
    for (int64_t i = tid; i < slot_words; i += kLdsSortThreads) slot_status[i] = 0;
    if (tid == 0) {
      *slot_ticket = 0;
      *plan = PlanScalars{};  // no complete plan until the slot scan stamps it
    }
  }
  // item i of this thread sits at segment position pos(i): (wave, round, lane)
  auto pos = [&](int i) { return wave * (ITEMS * kWave) + i * kWave + lane; };
  // the keys, B tokens at a time with their history loads in flight, into
  // LDS at their positions (so the history registers are free again before
  // the sort's), then into registers; a key's flat index follows from its
  // position
  constexpr int B = 4;
#pragma unroll
  for (int i0 = 0; i0 < ITEMS; i0 += B) {
    uint64_t mix[B][ENGRAM_MAX_NGRAM - 1];
#pragma unroll
    for (int b = 0; b < B; ++b) token_mixes<N>(hp, min(pos(i0 + b), len - 1), mix[b]);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      uint64_t m = mix[b][0];
#pragma unroll
      for (int k = 1; k < N - 1; ++k) m = order == k ? mix[b][k] : m;
      s_buf[pos(i0 + b)] = (uint32_t)head_row(hp, m, h);
    }
  }
  uint32_t key[ITEMS], val[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    key[i] = s_buf[pos(i)];  // (this thread's own positions: no barrier needed)
    val[i] = (uint32_t)((int64_t)pos(i) * sg.stride + h);
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int q = 0; q < passes; ++q) {
    const int shift = q * per_pass;
    const int width = bits - shift < per_pass ? bits - shift : per_pass;
    const uint32_t mask = (1u << width) - 1u;
    const int bins = 1 << width;
    for (int d = tid; d < kLdsSortWaves * kMaxBins; d += kLdsSortThreads) (&s_cnt[0][0])[d] = 0;
    __syncthreads();
    uint32_t rank[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const bool valid = pos(i) < len;
      const uint32_t d = ((key[i] - kbase) >> shift) & mask;
      unsigned long long peers = __ballot(valid);
      for (int b = 0; b < width; ++b) {
        const bool bit = (d >> b) & 1u;
        const unsigned long long bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      rank[i] = 0;
      if (valid) {
        const uint32_t prior = s_cnt[wave][d];
        rank[i] = prior + (uint32_t)__popcll(peers & below);
        if ((peers & below) == 0ull) s_cnt[wave][d] = prior + (uint32_t)__popcll(peers);
      }
    }
    __syncthreads();
    // per digit: the waves' offsets and the digit's total, then the digits'
    // starts by a block scan
    uint32_t total = 0;
    if (tid < bins) {
      for (int w = 0; w < kLdsSortWaves; ++w) {
        const uint32_t c = s_cnt[w][tid];
        s_cnt[w][tid] = total;
        total += c;
      }
    }
    uint32_t all;
    const uint32_t start = block_exclusive_scan<kLdsSortThreads>(tid < bins ? total : 0u, all);
    if (tid < bins) s_local[tid] = start;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t d = ((key[i] - kbase) >> shift) & mask;
      rank[i] += s_local[d] + s_cnt[wave][d];
    }
    // keys, then flat indices, through LDS into the pass's order
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (pos(i) < len) s_buf[rank[i]] = key[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (pos(i) < len) key[i] = s_buf[pos(i)];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (pos(i) < len) s_buf[rank[i]] = val[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (pos(i) < len) val[i] = s_buf[pos(i)];
    __syncthreads();  // s_buf and s_cnt are rewritten by the next pass
  }
  const int64_t seg0 = seg * sg.len;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (pos(i) < len) {
      keys_out[seg0 + pos(i)] = key[i];
      vals_out[seg0 + pos(i)] = val[i];
    }
  }
}

// ------------------------------------------- buckets after a top pass ---
// Two plans sort in two steps: a per-head plan of more than kLdsSortKeys
// keys a head on 17 to 24 bits (buckets on its low 16 bits), and a plan of
// at most kIdBucketKeys ids (buckets on all but the top bits of the keys,
// 9 to 24 bits).  First one one-sweep pass on the top bits (stable, so every
// bucket -- the keys of one segment whose top digit is equal -- holds its
// keys in flat order), then this kernel sorts each bucket on the low bits,
// in place, with two or three stable LSD passes of at most 8 bits.  One
// block per (segment, top digit): the bucket's start is the sum of the
// segment's top-digit counts below it (over the histogram's copies).  A
// bucket of at most 256 * ITEMS keys is sorted in LDS (the keys in (wave,
// round, lane) order, as few rounds as it needs, ranked by wavefront
// multi-split, each pass's digit starts by a block scan), read and written
// once.  A larger one (a hot row's run) is sorted through global memory by
// the same block: per pass, its digit totals, then tile after tile ranked as
// above and written at its digits' running offsets, into the segment's
// scratch copy and back.  The result is the order the full LSD sort gives:
// stable passes over all bits, low first.
constexpr int kBucketLow = 16;  // bits a per-head plan's buckets are sorted on
constexpr int kBucketMaxLow = 24;
constexpr int64_t kIdBucketKeys = 262144;  // most ids sorted by buckets
// A per-head plan's buckets: blocks of 256 threads holding 8 keys each (many
// small buckets); a plan of ids': 1024 threads holding 4 (fewer, larger
// buckets, each sorted by more waves).  Both hold up to 2048 or 4096 keys in
// LDS, and have at least one thread per digit of a pass of at most 8 bits.
constexpr int kBucketThreads = 256;
constexpr int kBucketItems = 8;
constexpr int kIdBucketThreads = 1024;
constexpr int kIdBucketItems = 4;

// Ranks of one tile's keys by digit ((key - kbase) >> shift) & mask.  Item
// i (i < rounds) of a thread sits at tile position (wave * rounds + i) * 64
// + lane, and positions below `count` hold keys.  rank[i] receives the
// item's place among its wave's keys of its digit, s_cnt[w][d] the start of
// wave w's keys of digit d among the tile's, and (threads below `bins`)
// *total the tile's count of digit tid.  Ends with a barrier.
template <int NT, int ITEMS>
__device__ __forceinline__ void bucket_tile_ranks(const uint32_t (&key)[ITEMS], int count,
                                                  int rounds, uint32_t kbase, int shift, int width,
                                                  uint32_t (&s_cnt)[(NT / kWave)][kMaxBins],
                                                  uint32_t (&rank)[ITEMS],
                                                  uint32_t *total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t mask = (1u << width) - 1u;
  const int bins = 1 << width;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int d = tid; d < (NT / kWave) * kMaxBins; d += NT) (&s_cnt[0][0])[d] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    rank[i] = 0;
    if (i < rounds) {  // (block-uniform)
      const bool valid = (wave * rounds + i) * kWave + lane < count;
      const uint32_t d = ((key[i] - kbase) >> shift) & mask;
      unsigned long long peers = __ballot(valid);
      for (int b = 0; b < width; ++b) {
        const bool bit = (d >> b) & 1u;
        const unsigned long long bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      if (valid) {
        const uint32_t prior = s_cnt[wave][d];
        rank[i] = prior + (uint32_t)__popcll(peers & below);
        if ((peers & below) == 0ull) s_cnt[wave][d] = prior + (uint32_t)__popcll(peers);
      }
    }
  }
  __syncthreads();
  if (tid < bins) {
    uint32_t t = 0;
    for (int w = 0; w < (NT / kWave); ++w) {
      const uint32_t c = s_cnt[w][tid];
      s_cnt[w][tid] = t;
      t += c;
    }
    *total = t;
  }
  __syncthreads();
}

template <int NT, int ITEMS>
__global__ __launch_bounds__(NT) void bucket_sort_kernel(
    const SortSegs sg, int top_bits, int low_bits, const uint32_t *hist, uint32_t *keys,
    uint32_t *vals, uint32_t *tmp_keys, uint32_t *tmp_vals) {
  static_assert(NT >= kMaxBins && NT % kWave == 0, "a thread per digit, whole waves");
  constexpr int kBucketKeys = NT * ITEMS;  // the LDS buffer's pairs
  __shared__ uint2 s_buf[kBucketKeys];  // (key, flat index) pairs
  __shared__ uint32_t s_cnt[(NT / kWave)][kMaxBins];
  __shared__ uint32_t s_start[kMaxBins];  // start of each digit (tile, or bucket's running)
  __shared__ uint32_t s_bucket[2];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t seg = blockIdx.x >> top_bits;
  const int top = (int)(blockIdx.x & ((1u << top_bits) - 1u));
  uint32_t all;
  // the top pass's digit totals, summed over the histogram's copies
  uint32_t c = 0;
  if (tid < (1 << top_bits))
    for (int cp = 0; cp < sg.copies; ++cp)
      c += hist[((int64_t)cp * sg.count + seg) * 4 * kMaxBins + tid];
  const uint32_t before = block_exclusive_scan<NT>(c, all);
  if (tid == top) {
    s_bucket[0] = before;
    s_bucket[1] = c;
  }
  __syncthreads();
  const int64_t b0 = seg * sg.len + s_bucket[0];
  const uint32_t m = s_bucket[1];
  if (m < 2) return;  // (block-uniform)
  const uint32_t kbase = sg.base[seg];
  // the low bits in npass LSD passes of w bits (the last one narrower)
  const int npass = (low_bits + 7) / 8;
  const int w = (low_bits + npass - 1) / npass;
  // rounds of 64 keys a wave: as few as the tile needs, so a small bucket's
  // keys are spread over all the waves
  int rounds = ITEMS;
  auto pos = [&](int i) { return (wave * rounds + i) * kWave + lane; };
  uint32_t key[ITEMS], val[ITEMS], rank[ITEMS];
  uint32_t total = 0;
  if (m <= (uint32_t)kBucketKeys) {
    rounds = (int)((m + NT - 1) / NT);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (i >= rounds) break;
      const int64_t q = b0 + min((uint32_t)pos(i), m - 1);
      key[i] = keys[q];
      val[i] = vals[q];
    }
    for (int pass = 0; pass < npass; ++pass) {
      const int shift = pass * w;
      const int width = low_bits - shift < w ? low_bits - shift : w;
      bucket_tile_ranks<NT, ITEMS>(key, (int)m, rounds, kbase, shift, width, s_cnt, rank, &total);
      const uint32_t start = block_exclusive_scan<NT>(tid < (1 << width) ? total
                                                                                      : 0u, all);
      if (tid < (1 << width)) s_start[tid] = start;
      __syncthreads();
      const uint32_t mask = (1u << width) - 1u;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (i >= rounds) break;
        const uint32_t d = ((key[i] - kbase) >> shift) & mask;
        rank[i] += s_start[d] + s_cnt[wave][d];
      }
      // keys with their flat indices through LDS into the pass's order
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (i >= rounds) break;
        if ((uint32_t)pos(i) < m) s_buf[rank[i]] = uint2{key[i], val[i]};
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (i >= rounds) break;
        if ((uint32_t)pos(i) < m) {
          const uint2 kv = s_buf[pos(i)];
          key[i] = kv.x;
          val[i] = kv.y;
        }
      }
      __syncthreads();  // s_buf, s_cnt and s_start are rewritten by the next pass
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (i >= rounds) break;
      if ((uint32_t)pos(i) < m) {
        keys[b0 + pos(i)] = key[i];
        vals[b0 + pos(i)] = val[i];
      }
    }
    return;
  }
  // a bucket larger than the LDS buffer: each pass from one copy of the
  // bucket's positions to the other (keys -> scratch -> keys).  A pass whose
  // keys all share one digit keeps their order and is skipped (a bucket of
  // one hot row needs no pass at all); after an odd number of passes the
  // bucket is copied back.
  bool in_tmp = false;
  for (int pass = 0; pass < npass; ++pass) {
    const uint32_t *src_k = in_tmp ? tmp_keys : keys, *src_v = in_tmp ? tmp_vals : vals;
    uint32_t *dst_k = in_tmp ? keys : tmp_keys, *dst_v = in_tmp ? vals : tmp_vals;
    const int shift = pass * w;
    const int width = low_bits - shift < w ? low_bits - shift : w;
    const uint32_t mask = (1u << width) - 1u;
    const int bins = 1 << width;
    // the bucket's digit totals, kBucketKeys keys a round with every load in
    // flight, then each digit's start; a bucket of one row (every key alike)
    // is already in order
    if (tid < kMaxBins) s_start[tid] = 0;
    __syncthreads();
    const uint32_t first = src_k[b0];
    bool differs = false;
    for (uint32_t p0 = 0; p0 < m; p0 += kBucketKeys) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const uint32_t q = p0 + (uint32_t)(i * NT + tid);
        key[i] = q < m ? src_k[b0 + q] : first;
      }
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (p0 + (uint32_t)(i * NT + tid) < m) {
          atomicAdd(&s_start[((key[i] - kbase) >> shift) & mask], 1u);
          differs = differs || key[i] != first;
        }
      }
    }
    if (!__syncthreads_or(differs)) break;  // (only at the first pass: the keys do not change)
    const uint32_t cnt = tid < bins ? s_start[tid] : 0u;
    if (__syncthreads_or(cnt == m)) continue;  // one digit: the pass keeps the order
    const uint32_t start = block_exclusive_scan<NT>(cnt, all);
    if (tid < kMaxBins) s_start[tid] = start;
    __syncthreads();
    for (uint32_t t0 = 0; t0 < m; t0 += kBucketKeys) {
      const int count = (int)min((uint32_t)kBucketKeys, m - t0);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t q = b0 + t0 + min(pos(i), count - 1);
        key[i] = src_k[q];
        val[i] = src_v[q];
      }
      bucket_tile_ranks<NT, ITEMS>(key, count, rounds, kbase, shift, width, s_cnt, rank, &total);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (pos(i) < count) {
          const uint32_t d = ((key[i] - kbase) >> shift) & mask;
          const int64_t q = b0 + s_start[d] + s_cnt[wave][d] + rank[i];
          dst_k[q] = key[i];
          dst_v[q] = val[i];
        }
      }
      __syncthreads();  // every read of s_start and s_cnt is done
      if (tid < bins) s_start[tid] += total;
      __syncthreads();
    }
    in_tmp = !in_tmp;
  }
  if (in_tmp) {
    for (uint32_t p0 = 0; p0 < m; p0 += kBucketKeys) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const uint32_t q = p0 + (uint32_t)(i * NT + tid);
        key[i] = q < m ? tmp_keys[b0 + q] : 0u;
        val[i] = q < m ? tmp_vals[b0 + q] : 0u;
      }
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const uint32_t q = p0 + (uint32_t)(i * NT + tid);
        if (q < m) {
          keys[b0 + q] = key[i];
          vals[b0 + q] = val[i];
        }
      }
    }
  }
}

// ------------------------------------------------------------ row slots ---
// Slot of every range's first distinct row: the number of distinct-row heads
// (first positions of a valid row) in all earlier ranges; the last tile also
// writes U, the number of distinct valid rows, and the plan's stamp.  One thread per range, a tile
// of kSlotThreads ranges per block (taken by atomic ticket): heads counted
// from the range's keys, a block scan, then the tile's offset by decoupled
// look-back, wavefront 0 reading 64 earlier tiles' published words at a time.
__global__ __launch_bounds__(kSlotThreads) void range_slots_kernel(
    const uint32_t *keys, int64_t n, uint32_t sentinel, int64_t num_ranges, uint64_t *status,
    uint32_t *ticket, uint32_t *head_off, PlanScalars *plan, int64_t *err) {
  __shared__ uint32_t s_tile, s_prefix;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  if (tid == 0) s_tile = atomicAdd(ticket, 1u);
  __syncthreads();
  const int64_t tile = s_tile;
  const int64_t r = tile * kSlotThreads + tid;
  uint32_t heads = 0;
  if (r < num_ranges) {
    const int64_t beg = r * kRange;
    const int cnt = (int)min((int64_t)kRange, n - beg);
    uint32_t prev = beg > 0 ? keys[beg - 1] : sentinel;
    const u32x4 *kp = reinterpret_cast<const u32x4 *>(keys + beg);
#pragma unroll
    for (int i = 0; i < kRange / 4; ++i) {
      const u32x4 k4 = kp[i];
      const uint32_t k[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        heads += (4 * i + e < cnt && k[e] != sentinel && k[e] != prev) ? 1u : 0u;
        prev = k[e];
      }
    }
  }
  uint32_t tile_total;
  const uint32_t local = block_exclusive_scan<kSlotThreads>(heads, tile_total);
  if (tid < kWave) {
    if (tid == 0)
      __hip_atomic_store(&status[tile], (tile == 0 ? kFlagInclusive : kFlagAggregate) | tile_total,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t before = 0;
    bool stalled = false;
    for (int64_t t0 = tile - 1; t0 >= 0;) {
      // lane l reads tile t0 - l; tiles before 0 read as an empty inclusive
      const int64_t t = t0 - lane;
      uint64_t word = t >= 0 ? __hip_atomic_load(&status[t], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : kFlagInclusive;
      unsigned long long incl, need;
      uint32_t spins = 0;
      for (;;) {  // wait for every word up to the nearest inclusive one
        incl = __ballot((word & kFlagInclusive) != 0);
        const int upto = incl != 0ull ? __ffsll((long long)incl) - 1 : kWave - 1;
        need = upto == kWave - 1 ? ~0ull : ((2ull << upto) - 1ull);
        const unsigned long long pending = __ballot((word >> 32) == 0) & need;
        if (pending == 0ull) break;
        if (++spins == kSpinLimit) {
          stalled = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        if ((pending >> lane) & 1ull)
          word = __hip_atomic_load(&status[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (stalled) break;
      uint64_t c = ((need >> lane) & 1ull) ? (word & 0xffffffffull) : 0ull;
#pragma unroll
      for (int d = kWave / 2; d > 0; d >>= 1) c += __shfl_xor(c, d, kWave);
      before += c;
      if (incl != 0ull) break;
      t0 -= kWave;
    }
    if (tid == 0) {
      if (tile != 0)
        __hip_atomic_store(&status[tile], kFlagInclusive | (uint32_t)(before + tile_total),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (stalled) {
        atomicOr(&plan->stalled, 1u);
        add_mark(err, kStallMark);
      }
      s_prefix = (uint32_t)before;
    }
  }
  __syncthreads();
  if (r < num_ranges) head_off[r] = s_prefix + local;
  if (tile == (int64_t)gridDim.x - 1 && tid == 0) {  // U, and the stamp of a complete plan
    plan->unique = s_prefix + tile_total;
    plan->n = (uint64_t)n;
    plan->table_rows = (uint64_t)sentinel;
  }
}


// How a plan sorts: one segment of all n keys, or one per head.
struct SortLayout {
  SortSegs sg;
  int64_t num_tiles;
  int bits, passes, per_pass;
  int items;  // keys per thread of a sort tile
};

// Tiles of a layout: half-size tiles for a small sort (when its look-back
// words still fit the workspace), full-size ones otherwise.
void size_tiles(const Plan &p, SortLayout *L) {
  auto per_segment = [L](int64_t tile) { return (L->sg.len + tile - 1) / tile; };
  L->items = kSortItems;
  int64_t per = per_segment(kSortTile);
  if ((int64_t)L->sg.count * per < kSmallSortTiles) {
    const int64_t half = per_segment(kSortTile / 2);
    if ((int64_t)L->passes * L->sg.count * half * kMaxBins + p.slot_tiles <= p.status_words) {
      L->items = kSortItems / 2;
      per = half;
    }
  }
  L->sg.tiles = per;
  L->num_tiles = (int64_t)L->sg.count * per;
}

SortLayout whole_sort(const Plan &p, int64_t n) {
  SortLayout L = {};
  L.sg.len = n;
  L.sg.count = 1;
  L.sg.copies = kHistCopies;
  L.sg.stride = 1;
  L.bits = p.bits;
  L.passes = p.passes;
  L.per_pass = p.per_pass;
  size_tiles(p, &L);
  return L;
}

// Per-head segments for a plan from tokens: possible when the heads' row
// ranges [offset, offset + prime) do not overlap (then every row belongs to
// one head, and the heads ordered by offset are sorted segment after
// segment), and used when the layout fits the workspace of n keys.
bool head_sort(const HashParams &hp, int64_t tokens, const Plan &p, SortLayout *out) {
  int order[ENGRAM_MAX_HEADS];
  for (int h = 0; h < hp.H; ++h) order[h] = h;
  for (int i = 1; i < hp.H; ++i)  // heads by row offset (at most 64)
    for (int j = i; j > 0 && hp.offset[order[j]] < hp.offset[order[j - 1]]; --j) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  uint64_t widest = 1;
  for (int i = 0; i < hp.H; ++i) {
    const int h = order[i];
    if (i + 1 < hp.H && hp.offset[h] + (int64_t)hp.prime[h] > hp.offset[order[i + 1]])
      return false;
    widest = hp.prime[h] > widest ? hp.prime[h] : widest;
  }
  SortLayout L = {};
  L.sg.len = tokens;
  L.sg.count = hp.H;
  L.sg.copies = 1;
  L.sg.stride = hp.H;
  for (int i = 0; i < hp.H; ++i) {
    L.sg.base[i] = (uint32_t)hp.offset[order[i]];
    L.sg.head[i] = (uint32_t)order[i];
  }
  L.bits = bit_width_u64(widest - 1);  // digits of key - offset < prime
  if (L.bits < 1) L.bits = 1;
  L.passes = (L.bits + 7) / 8;
  L.per_pass = (L.bits + L.passes - 1) / L.passes;
  size_tiles(p, &L);
  if (L.passes > p.passes ||
      (int64_t)L.passes * L.num_tiles * kMaxBins + p.slot_tiles > p.status_words)
    return false;
  *out = L;
  return true;
}

// One sort pass's buffers and digit, for launch_pass.
struct PassArgs {
  const int64_t *ids;
  const uint32_t *keys_in, *vals_in;
  int64_t table_rows;
  int shift, width;
  const uint32_t *hist;
  uint64_t *status;
  uint32_t *ticket, *keys_out, *vals_out;
  PlanScalars *plan;
  int64_t *err;
};

template <int ITEMS>
void launch_pass(int src, const SortLayout &L, const PassArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)L.num_tiles), block(kSortThreads);
  if (src == kSrcIds)
    hipLaunchKernelGGL((onesweep_kernel<kSrcIds, ITEMS>), grid, block, 0, s, a.ids, nullptr,
                       nullptr, L.sg, a.table_rows, a.shift, a.width, a.hist, a.status, a.ticket,
                       a.keys_out, a.vals_out, a.plan, a.err);
  else if (src == kSrcKeysIota)
    hipLaunchKernelGGL((onesweep_kernel<kSrcKeysIota, ITEMS>), grid, block, 0, s, nullptr,
                       a.keys_in, nullptr, L.sg, a.table_rows, a.shift, a.width, a.hist, a.status,
                       a.ticket, a.keys_out, a.vals_out, a.plan, a.err);
  else
    hipLaunchKernelGGL((onesweep_kernel<kSrcKeys, ITEMS>), grid, block, 0, s, nullptr, a.keys_in,
                       a.vals_in, L.sg, a.table_rows, a.shift, a.width, a.hist, a.status,
                       a.ticket, a.keys_out, a.vals_out, a.plan, a.err);
}


}  // namespace
}  // namespace engram

// Plan: sort the row ids and give every distinct row its slot (U and the
// plan's stamp are left in the workspace scalars).  Needs only the ids: given (ids), or computed
// from the tokens (hp, when ids is null).
int engram::launch_plan(const int64_t *ids, const HashParams *hp, int64_t n, int64_t table_rows,
                        const Plan &p, void *ws, int64_t *err, void *stream) {
  hipStream_t s = as_stream(stream);
  const Views v = views_of(p, ws);
  uint32_t *tickets = v.counters;              // [4], then the slot scan's
  uint32_t *hist = v.counters + kTicketWords;  // [copy][segment][4][kMaxBins]
  SortLayout L = whole_sort(p, n);
  const bool heads = ids == nullptr && head_sort(*hp, n / hp->H, p, &L);
  // one sort pass on the top bits, then each bucket on the rest: per-head
  // segments too large for the LDS plan, on 17 to 24 bits (the low 16 bits
  // in the buckets); and at most kIdBucketKeys ids, about 512 a bucket, on
  // 9 to 24 bits below the top digit
  int top_bits = 0;
  if (heads && L.sg.len > kLdsSortKeys && L.bits > kBucketLow && L.bits <= kBucketLow + 8)
    top_bits = L.bits - kBucketLow;
  if (ids != nullptr && n > kSortTile && n <= kIdBucketKeys) {
    const int want = bit_width_u64((uint64_t)(n - 1) / 512);  // about 512 ids a bucket
    const int top = want < 8 ? want : 8;
    if (L.bits - top >= 9 && L.bits - top <= kBucketMaxLow) top_bits = top;
  }
  const bool buckets = top_bits > 0;
  const int low_bits = L.bits - top_bits;
  if (buckets) L.passes = 1;
  const int64_t sort_words = (int64_t)L.passes * L.num_tiles * kMaxBins;
  const int64_t status_len = sort_words + p.slot_tiles;
  const int64_t counters_len = kTicketWords + (int64_t)L.sg.copies * L.sg.count * 4 * kMaxBins;
  const int64_t clear_len = status_len > counters_len ? status_len : counters_len;
  // every grid inside the launch limit, checked before anything is enqueued
  // (below n = 2^32 they all are; the token hash of a flat plan strides)
  const int64_t head_chunks = (L.sg.len + kHeadTokens - 1) / kHeadTokens;
  if (!grid_fits(p.num_tiles, kSortThreads) || !grid_fits(L.num_tiles, kSortThreads) ||
      !grid_fits(p.slot_tiles, kSlotThreads) || !grid_fits((clear_len + 255) / 256, 256) ||
      !grid_fits(L.sg.count * head_chunks, kHeadThreads))
    return ENGRAM_EINVAL;
  if (heads && L.sg.len <= kLdsSortKeys) {
    // small segments: one kernel sorts every head's keys in LDS, into the
    // buffers the apply reads (those the last pass of a sort would fill)
    uint32_t *const keys_dst = p.passes % 2 == 1 ? v.keys_a : v.keys_b;
    uint32_t *const vals_dst = p.passes % 2 == 1 ? v.vals_a : v.vals_b;
    const int items = L.sg.len <= 4 * kLdsSortThreads ? 4 : 8;
    const dim3 grid((unsigned)L.sg.count), block(kLdsSortThreads);
    switch (hp->n * 100 + items) {
#define ENGRAM_PLAN_LDS_CASE(N, I)                                                             \
  case N * 100 + I:                                                                            \
    hipLaunchKernelGGL((plan_heads_lds_kernel<N, I>), grid, block, 0, s, *hp, L.sg, L.passes,   \
                       L.per_pass, L.bits, keys_dst, vals_dst, v.status,                       \
                       p.slot_tiles, tickets + kSlotTicketAt, v.scalars);                      \
    break;
#define ENGRAM_PLAN_LDS_N(N) ENGRAM_PLAN_LDS_CASE(N, 4) ENGRAM_PLAN_LDS_CASE(N, 8)
      ENGRAM_PLAN_LDS_N(2)
      ENGRAM_PLAN_LDS_N(3)
      ENGRAM_PLAN_LDS_N(4)
      ENGRAM_PLAN_LDS_N(5)
      ENGRAM_PLAN_LDS_N(6)
      ENGRAM_PLAN_LDS_N(7)
      ENGRAM_PLAN_LDS_N(8)
#undef ENGRAM_PLAN_LDS_N
#undef ENGRAM_PLAN_LDS_CASE
    }
    hipLaunchKernelGGL(range_slots_kernel, dim3((unsigned)p.slot_tiles), dim3(kSlotThreads), 0,
                       s, v.sorted_keys, n, (uint32_t)table_rows, p.num_ranges, v.status,
                       tickets + kSlotTicketAt, v.head_off, v.scalars, err);
    return launch_status();
  }
  hipLaunchKernelGGL(sort_clear_kernel, dim3((unsigned)((clear_len + 255) / 256)), dim3(256), 0,
                     s, v.status, status_len, v.counters, (int)counters_len, v.scalars);
  // The passes alternate between the two key/index buffers and end in the
  // pair the apply reads; the keys a plan from tokens hashes go to the other
  // buffer of the first pass.
  const bool end_in_a = p.passes % 2 == 1;
  uint32_t *const last_k = end_in_a ? v.keys_a : v.keys_b,
                 *const last_v = end_in_a ? v.vals_a : v.vals_b;
  uint32_t *const other_k = end_in_a ? v.keys_b : v.keys_a,
                 *const other_v = end_in_a ? v.vals_b : v.vals_a;
  auto out_k = [&](int pass) { return (L.passes - 1 - pass) % 2 == 0 ? last_k : other_k; };
  auto out_v = [&](int pass) { return (L.passes - 1 - pass) % 2 == 0 ? last_v : other_v; };
  uint32_t *const hashed = out_k(0) == last_k ? other_k : last_k;
  if (ids != nullptr) {  // one block per kSortTile ids, whatever the sort's tiles
    hipLaunchKernelGGL(sort_histogram_kernel, dim3((unsigned)p.num_tiles), dim3(kSortThreads), 0,
                       s, ids, n, table_rows, L.passes, buckets ? top_bits : L.per_pass, L.bits,
                       buckets ? low_bits : 0, hist, err);
  } else if (heads) {
    const int64_t chunks = head_chunks;
    const dim3 grid((unsigned)(L.sg.count * chunks));
    switch (hp->n) {
#define ENGRAM_PLAN_HEADS_CASE(N)                                                             \
  case N:                                                                                     \
    hipLaunchKernelGGL(plan_hash_heads_kernel<N>, grid, dim3(kHeadThreads), 0, s, *hp, L.sg,    \
                       chunks, L.passes, buckets ? top_bits : L.per_pass, L.bits,             \
                       buckets ? low_bits : 0, hashed, hist);                                 \
    break;
      ENGRAM_PLAN_HEADS_CASE(2)
      ENGRAM_PLAN_HEADS_CASE(3)
      ENGRAM_PLAN_HEADS_CASE(4)
      ENGRAM_PLAN_HEADS_CASE(5)
      ENGRAM_PLAN_HEADS_CASE(6)
      ENGRAM_PLAN_HEADS_CASE(7)
      ENGRAM_PLAN_HEADS_CASE(8)
#undef ENGRAM_PLAN_HEADS_CASE
    }
  } else {  // keys in flat order
    const int64_t tokens = n / hp->H;
    const int64_t need = (tokens + 63) / 64, most = kMaxGridItems / kSortThreads;
    hipLaunchKernelGGL(plan_hash_kernel, dim3((unsigned)(need < most ? need : most)),
                       dim3(kSortThreads), 0, s, *hp, tokens, L.passes, L.per_pass, L.bits,
                       hashed, hist);
  }
  for (int pass = 0; pass < L.passes; ++pass) {
    const int shift = buckets ? low_bits : pass * L.per_pass;
    const int width = buckets ? top_bits
                              : (L.bits - shift < L.per_pass ? L.bits - shift : L.per_pass);
    const PassArgs a = {ids, pass == 0 ? hashed : out_k(pass - 1),
                        pass == 0 ? nullptr : out_v(pass - 1), table_rows, shift, width,
                        hist + pass * kMaxBins, v.status + (int64_t)pass * L.num_tiles * kMaxBins,
                        tickets + pass, out_k(pass), out_v(pass), v.scalars, err};
    const int src = pass > 0 ? kSrcKeys : (ids != nullptr ? kSrcIds : kSrcKeysIota);
    if (L.items == kSortItems)
      launch_pass<kSortItems>(src, L, a, s);
    else
      launch_pass<kSortItems / 2>(src, L, a, s);
  }
  if (buckets) {  // the top pass wrote the pair the apply reads; the other is scratch
    if (ids != nullptr)
      hipLaunchKernelGGL((bucket_sort_kernel<kIdBucketThreads, kIdBucketItems>),
                         dim3(1u << top_bits), dim3(kIdBucketThreads), 0, s, L.sg, top_bits,
                         low_bits, hist, last_k, last_v, other_k, other_v);
    else
      hipLaunchKernelGGL((bucket_sort_kernel<kBucketThreads, kBucketItems>),
                         dim3((unsigned)(L.sg.count << top_bits)), dim3(kBucketThreads), 0, s,
                         L.sg, top_bits, low_bits, hist, last_k, last_v, other_k, other_v);
  }
  // distinct-row slots
  hipLaunchKernelGGL(range_slots_kernel, dim3((unsigned)p.slot_tiles), dim3(kSlotThreads), 0, s,
                     v.sorted_keys, n, (uint32_t)table_rows, p.num_ranges, v.status + sort_words,
                     tickets + kSlotTicketAt, v.head_off, v.scalars, err);
  return launch_status();
}
