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
//     table_rows, at most 8 bits per pass, one kernel per pass ("one-sweep"):
//     each 4096-key tile ranks its keys with a wavefront multi-split (one
//     ballot per digit bit yields the mask of lanes holding the same digit,
//     its popcount the stable rank), finds its output offsets by decoupled
//     look-back over earlier tiles' published digit counts, and writes its
//     keys and indices in coalesced digit runs staged through LDS.  The
//     first pass reads the int64 ids directly: valid rows become 32-bit
//     keys, padding and invalid ids the key table_rows, which sorts last and
//     is dropped.  A plan made from the tokens first hashes them into 32-bit
//     keys (counting the digits as it goes), and its first pass reads those.
//     When the heads own disjoint row ranges (as when the offsets pack them
//     back to back) every row belongs to one head, so the
//     keys are laid out and sorted per head: one segment per head, in order
//     of offset, each sorted on the bits of its largest remainder (23 bits
//     for 8.3M-row heads instead of the 28 of a 200M-row table: 3 passes
//     instead of 4), with look-back inside the segment.  The segments one
//     after another are the same sorted order a sort of all the keys gives.
//  2. Segment heads (first position of each distinct row) are counted per
//     16-position range and scanned in one kernel (decoupled look-back over
//     tiles of ranges): the scan gives every distinct row its output slot u,
//     and U itself.
//  3. Range walkers: a group of head_dim/4 lanes (one 4-value quad of the
//     row per lane, up to a whole wavefront) takes one 16-position range of
//     the sorted order, issues all its loads at once (keys, flat indices,
//     then the gradient rows) and sums runs in fp64 registers.  A run that
//     starts and ends inside the range is written once (dense
//     read-modify-write, row-sparse store, or the SignSGD step on the bf16
//     table row); a run cut by the range's end but ending in the next range
//     is finished by the same walker.  Runs longer than that (hot rows,
//     found from three sorted keys per range) are summed whole by the
//     leading blocks of the same launch, a block per run, its walkers taking
//     interleaved ranges of the run and adding their sums in a fixed order.
//     No work item waits on another, and hot rows (hundreds of
//     contributions) do not serialise a walker.
// Atomic path: one fp32 atomic add per gradient element into the dense
// table (hardware float atomics in L2); order of additions not fixed.
#include <mutex>

#include "engram_hash_dev.h"

namespace engram {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per tile (and per histogram block)
// A sort with fewer tiles than this takes tiles of half the size: twice the
// blocks on a GPU of 256 compute units, and half a tile's serial work each.
constexpr int64_t kSmallSortTiles = 128;
constexpr int kMaxBins = 256;
constexpr int kSlotThreads = 256;  // ranges per tile of the slot scan
constexpr int kRange = 16;  // sorted positions per walker
constexpr int kWalkThreads = 256;
constexpr int kAtomicThreads = 256;
constexpr int kAtomicUnroll = 4;

constexpr int64_t kLongBlocks = 1024;  // most blocks that sum long runs
constexpr int64_t kXcds = 8;           // XCDs of an MI355X (blocks go to them in turn)
// Gradient tensors larger than this are read with non-temporal loads: half
// the MI355X's 256 MB Infinity Cache, so a tensor that could still be cached
// when the apply runs is read normally.
constexpr int64_t kStreamGradBytes = int64_t(128) << 20;
constexpr int64_t kLongSpan = 64;      // fewest ranges per long-run block
// Global digit totals are kept in kHistCopies copies (a block adds to copy
// blockIdx % kHistCopies) so the histogram's atomics do not all meet on the
// same few hundred words; readers add the copies.
constexpr int kHistCopies = 8;
// counters: 4 pass tickets and the slot scan's ticket (8 words), then the
// digit totals, [copy][segment][pass][digit]: kHistCopies copies of one
// segment for a sort of the whole key array, or one copy per segment for a
// sort of per-head segments.
constexpr int kTicketWords = 8;
constexpr int kSlotTicketAt = 4;
constexpr int kHistSets = kHistCopies > ENGRAM_MAX_HEADS ? kHistCopies : ENGRAM_MAX_HEADS;
constexpr int kSortCounters = kTicketWords + kHistSets * 4 * kMaxBins;
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
constexpr int64_t kStallMark = int64_t(1) << 40;  // added to err when a wait expires
constexpr int kLookBatch = 4;                     // predecessor tiles read per look-back step

__global__ __launch_bounds__(256) void sort_clear_kernel(uint64_t *status, int64_t status_len,
                                                         uint32_t *counters, int counters_len) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < status_len) status[i] = 0;
  if (i < counters_len) counters[i] = 0;
}

// hist[copy][pass][digit] += number of keys with that digit.  One block per
// kSortTile ids, all of a thread's loads in flight before any is counted.
__global__ __launch_bounds__(kSortThreads) void sort_histogram_kernel(
    const int64_t *ids, int64_t n, int64_t table_rows, int passes, int per_pass, int bits,
    uint32_t *hist, int64_t *err) {
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
      const int shift = q * per_pass;
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
    uint32_t *ticket, uint32_t *keys_out, uint32_t *vals_out, int64_t *err) {
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
    if (stalled && err != nullptr)
      atomicAdd(reinterpret_cast<unsigned long long *>(err), (unsigned long long)kStallMark);
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
// is computed as the hash kernel does (64 tokens per block; one lane per
// token computes its order mixes, then the block's 64 * H outputs in flat
// order), written as its 32-bit sort key, and counted into every pass's
// digit histogram.  Hashed rows are always inside the table.
__global__ __launch_bounds__(kSortThreads) void plan_hash_kernel(const HashParams hp,
                                                                 int64_t total_tokens,
                                                                 int passes, int per_pass,
                                                                 int bits, uint32_t *keys,
                                                                 uint32_t *hist) {
  constexpr int kTokens = 64;
  __shared__ uint64_t s_mix[kTokens][ENGRAM_MAX_NGRAM - 1];
  __shared__ uint32_t s_hist[4][kMaxBins];
  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * kTokens;
  for (int d = tid; d < 4 * kMaxBins; d += kSortThreads) (&s_hist[0][0])[d] = 0;
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
  __syncthreads();
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
// base[s]) into the segment's histograms, one flush per block.  A thread
// takes kHeadItems tokens with all their history loads in flight together.
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
    uint32_t *keys, uint32_t *hist) {
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
      const int shift = q * per_pass;
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

// ------------------------------------------------------------ row slots ---
// Slot of every range's first distinct row: the number of distinct-row heads
// (first positions of a valid row) in all earlier ranges; the last tile also
// writes U, the number of distinct valid rows.  One thread per range, a tile
// of kSlotThreads ranges per block (taken by atomic ticket): heads counted
// from the range's keys, a block scan, then the tile's offset by decoupled
// look-back, wavefront 0 reading 64 earlier tiles' published words at a time.
__global__ __launch_bounds__(kSlotThreads) void range_slots_kernel(
    const uint32_t *keys, int64_t n, uint32_t sentinel, int64_t num_ranges, uint64_t *status,
    uint32_t *ticket, uint32_t *head_off, uint32_t *total, int64_t *err) {
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
      if (stalled && err != nullptr)
        atomicAdd(reinterpret_cast<unsigned long long *>(err), (unsigned long long)kStallMark);
      s_prefix = (uint32_t)before;
    }
  }
  __syncthreads();
  if (r < num_ranges) head_off[r] = s_prefix + local;
  if (tile == (int64_t)gridDim.x - 1 && tid == 0) *total = s_prefix + tile_total;
}

// ---------------------------------------------------------- range walkers --
// Lane layout.  A walker is L lanes.  A row of head_dim values is split into
// quads of 4 values (8 bytes of bf16 input, 16 bytes of fp32 output); lane
// l owns quads l, l + L, ..., l + (Q - 1) * L (Q = quads per lane).  Every
// load instruction of a walker thus reads L consecutive 8-byte pieces, and
// every store instruction writes L consecutive 16-byte pieces: whole
// cache lines, so no partially written line reaches HBM.
struct WalkArgs {
  const uint32_t *keys;  // sorted rows (sentinel last), padded to whole ranges
  const uint32_t *vals;  // flat index of each sorted row
  int64_t n;
  uint32_t sentinel;
  const uint2 *grads;  // [n, dim / 4] quads of 4 bf16
  bool stream_grads;   // read the gradient rows with non-temporal loads
  int64_t quads;       // dim / 4
  int64_t dim;
  const uint32_t *head_off;  // slot of each range's first distinct row
  int64_t num_ranges;
  float *grad_table;    // dense output
  int64_t *unique_ids;  // row-sparse output
  float *unique_grads;
  uint2 *table;         // SignSGD output: the bf16 table, [rows, dim / 4] quads
  float lr;
  uint32_t long_blocks;  // leading blocks of the grid: they sum the long runs
  int64_t long_span;     // ranges each of those blocks looks after
  const uint32_t *unique_total;  // U, from the plan
  int64_t *num_unique;           // row-sparse output count
};

template <int Q>
__device__ __forceinline__ void zero_acc(double (&acc)[Q][4]) {
#pragma unroll
  for (int k = 0; k < Q; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[k][e] = 0.0;
}

template <int Q>
__device__ __forceinline__ void add_quads(double (&acc)[Q][4], const uint2 (&g)[Q]) {
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    acc[k][0] += (double)bf16_lo(g[k].x);
    acc[k][1] += (double)bf16_hi(g[k].x);
    acc[k][2] += (double)bf16_lo(g[k].y);
    acc[k][3] += (double)bf16_hi(g[k].y);
  }
}

template <int Q>
__device__ __forceinline__ void add_quads_if(double (&acc)[Q][4], const uint2 (&g)[Q], bool live) {
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    acc[k][0] += live ? (double)bf16_lo(g[k].x) : 0.0;
    acc[k][1] += live ? (double)bf16_hi(g[k].x) : 0.0;
    acc[k][2] += live ? (double)bf16_lo(g[k].y) : 0.0;
    acc[k][3] += live ? (double)bf16_hi(g[k].y) : 0.0;
  }
}

// What the apply writes for each distinct row r with sum S_r.
constexpr int kOutDense = 0;    // grad_table[r] += fp32(S_r)
constexpr int kOutSparse = 1;   // unique_ids[u] = r, unique_grads[u] = fp32(S_r)
constexpr int kOutSignSGD = 2;  // table[r] = bf16(fp32(table[r]) - lr * sign(fp32(S_r)))

// This lane's quads of row idx of a [rows, quads] array of 4-value quads.
template <int L, int Q, bool EXACT>
__device__ __forceinline__ void load_quads(const uint2 *base, uint32_t idx, int64_t quads,
                                           int lane, uint2 (&g)[Q]) {
  const uint2 *row = base + (int64_t)idx * quads;
#pragma unroll
  for (int k = 0; k < Q; ++k)
    g[k] = EXACT ? row[lane + k * L] : row[min((int64_t)lane + (int64_t)k * L, quads - 1)];
}

// This lane's fp32 quads of row idx of the dense gradient table.
template <int L, int Q, bool EXACT>
__device__ __forceinline__ void load_grad_row(const WalkArgs &a, uint32_t idx, int lane,
                                              f32x4 (&g)[Q]) {
  const f32x4 *row = reinterpret_cast<const f32x4 *>(a.grad_table + (int64_t)idx * a.dim);
#pragma unroll
  for (int k = 0; k < Q; ++k)
    g[k] = EXACT ? row[lane + k * L] : row[min((int64_t)lane + (int64_t)k * L, a.quads - 1)];
}

// This lane's quads of one gradient row.  Every gradient row is read exactly
// once; when the gradients are far larger than the caches (NT, chosen once per
// launch from stream_grads) the loads are non-temporal, so they do not displace
// the lines that are reused (keys, indices, the rows being written).  A
// gradient tensor small enough to stay cached (just written by the layer
// above, say) is read normally.
template <int L, int Q, bool EXACT, bool NT>
__device__ __forceinline__ void load_row(const WalkArgs &a, uint32_t idx, int lane,
                                         uint2 (&g)[Q]) {
  if constexpr (!NT) {
    load_quads<L, Q, EXACT>(a.grads, idx, a.quads, lane, g);
    return;
  }
  const u32x2 *row = reinterpret_cast<const u32x2 *>(a.grads) + (int64_t)idx * a.quads;
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const u32x2 t = __builtin_nontemporal_load(
        EXACT ? &row[lane + k * L] : &row[min((int64_t)lane + (int64_t)k * L, a.quads - 1)]);
    g[k] = uint2{t.x, t.y};
  }
}

// Keys and flat indices of one range as 16-byte vectors.
__device__ __forceinline__ void load_range(const uint32_t *keys, const uint32_t *vals,
                                           int64_t beg, uint32_t (&kk)[kRange],
                                           uint32_t (&vv)[kRange]) {
  const u32x4 *kp = reinterpret_cast<const u32x4 *>(keys + beg);
  const u32x4 *vp = reinterpret_cast<const u32x4 *>(vals + beg);
#pragma unroll
  for (int i = 0; i < kRange / 4; ++i) {
    const u32x4 k4 = kp[i], v4 = vp[i];
    kk[4 * i] = k4.x; kk[4 * i + 1] = k4.y; kk[4 * i + 2] = k4.z; kk[4 * i + 3] = k4.w;
    vv[4 * i] = v4.x; vv[4 * i + 1] = v4.y; vv[4 * i + 2] = v4.z; vv[4 * i + 3] = v4.w;
  }
}

// Flat indices of one range as 16-byte vectors.
__device__ __forceinline__ void load_vals(const uint32_t *vals, int64_t beg,
                                          uint32_t (&vv)[kRange]) {
  const u32x4 *vp = reinterpret_cast<const u32x4 *>(vals + beg);
#pragma unroll
  for (int i = 0; i < kRange / 4; ++i) {
    const u32x4 v4 = vp[i];
    vv[4 * i] = v4.x; vv[4 * i + 1] = v4.y; vv[4 * i + 2] = v4.z; vv[4 * i + 3] = v4.w;
  }
}

// A run is long when it starts in range c and still holds position
// 16 (c + 2): it covers the whole of range c + 1 and reaches beyond.  Given
// the keys at 16 c - 1 (`before`), 16 c + 15 (`k15`) and 16 (c + 2) (`far`),
// whether range c's last run is long.
__device__ __forceinline__ bool last_run_long(int64_t c, int64_t n, uint32_t sentinel,
                                              uint32_t before, uint32_t k15, uint32_t far) {
  return (c + 2) * kRange < n && k15 != sentinel && far == k15 && (c == 0 || before != k15);
}

// The finished sum of row `key` (distinct-row slot u): one rounding to fp32,
// then one fp32 add into the dense table (gt: this lane's quads of the fp32
// row, loaded earlier), a row-sparse store, or the SignSGD step on the bf16
// table row (w: this lane's quads of that row, loaded earlier).
template <int L, int Q, int OUT>
__device__ __forceinline__ void emit_row(uint32_t key, uint32_t u, const WalkArgs &a, int lane,
                                         const double (&acc)[Q][4], const uint2 (&w)[Q],
                                         const f32x4 (&gt)[Q]) {
  if (OUT == kOutSparse && lane == 0) a.unique_ids[u] = (int64_t)key;
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int64_t qd = lane + (int64_t)k * L;
    if (qd >= a.quads) continue;
    const f32x4 sum = {(float)acc[k][0], (float)acc[k][1], (float)acc[k][2], (float)acc[k][3]};
    if (OUT == kOutSparse) {
      f32x4 *dst = reinterpret_cast<f32x4 *>(a.unique_grads + (int64_t)u * a.dim) + qd;
      __builtin_nontemporal_store(sum, dst);
    } else if (OUT == kOutDense) {
      f32x4 *dst = reinterpret_cast<f32x4 *>(a.grad_table + (int64_t)key * a.dim) + qd;
      *dst = (Q == 1 ? gt[k] : *dst) + sum;  // wide rows are read here, not prefetched
    } else {
      const uint32_t b0 = signsgd_bf16(bf16_lo(w[k].x), sum.x, a.lr);
      const uint32_t b1 = signsgd_bf16(bf16_hi(w[k].x), sum.y, a.lr);
      const uint32_t b2 = signsgd_bf16(bf16_lo(w[k].y), sum.z, a.lr);
      const uint32_t b3 = signsgd_bf16(bf16_hi(w[k].y), sum.w, a.lr);
      a.table[(int64_t)key * a.quads + qd] = uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
  }
}

// One walker over one kRange-position range of the sorted order.  Run
// ownership: the walker holding a run's first position owns it, unless the
// run is long (then a long-run block sums it whole).  Positions of a run
// that entered from the previous range are never summed here: that run is
// either long or was finished by its owner.  Every load of the positions the
// walker sums is issued up front and unconditionally (keys and flat indices
// as 16-byte vectors, then one gradient row per position; other positions
// read row 0 and are ignored), so a walker costs two memory round trips;
// only then are runs summed and written.  A run that crosses into the next
// range (and, not being long, ends there) is finished by its owner, which
// then reads the next range's keys and the continuation rows.
template <int L, int Q, int OUT, bool EXACT, bool NT>
__device__ __forceinline__ void walk_range(const WalkArgs &a, int64_t blk) {
  const int lane = threadIdx.x % L;
  const int64_t w = (blk * kWalkThreads + threadIdx.x) / L;
  if (w >= a.num_ranges) return;
  const int64_t beg = w * kRange;
  const int cnt = (int)min((int64_t)kRange, a.n - beg);

  uint32_t kk[kRange], vv[kRange];
  load_range(a.keys, a.vals, beg, kk, vv);
  const int64_t end = beg + cnt;
  const uint32_t before = a.keys[beg > 0 ? beg - 1 : 0];
  const uint32_t after = a.keys[end < a.n ? end : a.n - 1];
  const uint32_t far = a.keys[min(beg + 2 * kRange, a.n - 1)];
  const bool last_long = last_run_long(w, a.n, a.sentinel, before, kk[kRange - 1], far);
  int live_count = 0;
#pragma unroll
  for (int q = 0; q < kRange; ++q) {
    if (q >= cnt) kk[q] = a.sentinel;
    live_count += kk[q] != a.sentinel ? 1 : 0;  // sentinels sort last
  }
  // [lead, tail): the positions this walker sums.  lead skips the run that
  // entered from before; a long last run (it started here) ends the span.
  const bool left_open = beg > 0 && live_count > 0 && before == kk[0];
  int lead = 0;
#pragma unroll
  for (int q = 0; q < kRange; ++q) lead += (left_open && lead == q && kk[q] == kk[0]) ? 1 : 0;
  uint32_t klast = kk[0];
#pragma unroll
  for (int q = 1; q < kRange; ++q) klast = q < live_count ? kk[q] : klast;
  int tail = 0;
#pragma unroll
  for (int q = 0; q < kRange; ++q)
    tail += (q < live_count && !(last_long && kk[q] == klast)) ? 1 : 0;

  // The output row of every run that starts in [lead, tail), loaded beside
  // the gradient rows, so no write waits on a read (other positions re-read
  // the first key's row): the bf16 table row (SignSGD) or the fp32 gradient
  // table row (dense, rows up to 256 values: wider fp32 rows would not fit
  // in registers 16 at a time).
  constexpr bool kPrefetchDense = OUT == kOutDense && Q == 1;
  uint2 tw[OUT == kOutSignSGD ? kRange : 1][Q];
  f32x4 tg[kPrefetchDense ? kRange : 1][Q];
  uint2 cw[Q];   // the current run's bf16 table row
  f32x4 cg[Q];   // the current run's fp32 gradient table row
  if constexpr (OUT == kOutSignSGD || kPrefetchDense) {
    if (tail > lead) {
#pragma unroll
      for (int q = 0; q < kRange; ++q) {
        const bool head = q >= lead && q < tail && (q == lead || kk[q] != kk[q > 0 ? q - 1 : 0]);
        if constexpr (OUT == kOutSignSGD)
          load_quads<L, Q, EXACT>(a.table, head ? kk[q] : kk[0], a.quads, lane, tw[q]);
        else
          load_grad_row<L, Q, EXACT>(a, head ? kk[q] : kk[0], lane, tg[q]);
      }
    }
  }

  // gradient rows in flight together (rows wider than 512 values: Q / 2
  // batches, to bound registers)
  constexpr int B = Q > 2 ? kRange / (Q / 2) : kRange;
  uint32_t u = a.head_off[w];  // slot of the first run that starts here
  uint32_t cur = a.sentinel;
  bool started = false;
  double acc[Q][4];
  zero_acc<Q>(acc);
#pragma unroll
  for (int b0 = 0; b0 < kRange; b0 += B) {
    uint2 g[B][Q];
#pragma unroll
    for (int qq = 0; qq < B; ++qq) {
      const int q = b0 + qq;
      load_row<L, Q, EXACT, NT>(a, (q >= lead && q < tail) ? vv[q] : 0u, lane, g[qq]);
    }
#pragma unroll
    for (int qq = 0; qq < B; ++qq) {
      const int q = b0 + qq;
      const bool live = q >= lead && q < tail;
      const bool head = live && (!started || kk[q] != cur);  // a distinct row starts at beg + q
      if (head && started) {
        emit_row<L, Q, OUT>(cur, u, a, lane, acc, cw, cg);
        ++u;
        zero_acc<Q>(acc);
      }
      if (head) {
        if constexpr (OUT == kOutSignSGD) {
#pragma unroll
          for (int k = 0; k < Q; ++k) cw[k] = tw[q][k];
        }
        if constexpr (kPrefetchDense) {
#pragma unroll
          for (int k = 0; k < Q; ++k) cg[k] = tg[q][k];
        }
        cur = kk[q];
        started = true;
      }
      // the row is used on every path, so its load stays with the others
      // (issued in order, consumed in order as each one arrives)
      add_quads_if<Q>(acc, g[qq], live);
    }
  }
  if (!started) return;
  // the last run continues into the next range (this range is full, the
  // next one starts at end); not being long, it ends there
  if (!last_long && live_count == kRange && end < a.n && after == cur) {
    const int ncnt = (int)min((int64_t)kRange, a.n - end);
    uint32_t nk[kRange], nv[kRange];
    load_range(a.keys, a.vals, end, nk, nv);
    int m = 0;  // continuation length
#pragma unroll
    for (int q = 0; q < kRange; ++q) m += (m == q && q < ncnt && nk[q] == cur) ? 1 : 0;
    for (int q0 = 0; q0 < m; q0 += 4) {
      uint2 g[4][Q];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        load_row<L, Q, EXACT, NT>(a, q0 + b < m ? nv[q0 + b] : 0u, lane, g[b]);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (q0 + b < m) add_quads<Q>(acc, g[b]);
    }
  }
  emit_row<L, Q, OUT>(cur, u, a, lane, acc, cw, cg);
}

// One long run: the run that starts in range c0 and reaches range c0 + 2.
template <int L, int Q, int OUT, bool EXACT, bool NT>
__device__ __forceinline__ void long_run(const WalkArgs &a, int64_t c0,
                                         double (&s_part)[kWalkThreads / L][L * 4]) {
  constexpr int G = kWalkThreads / L;  // walkers per block
  const int lane = threadIdx.x % L, g = threadIdx.x / L, wl = __lane_id();
  const int64_t r0 = c0 * kRange;
  const uint32_t u = a.head_off[c0 + 1] - 1;  // the last head of c0 (c0 + 2 exists)
  const uint32_t key = a.keys[r0 + kRange - 1];
  uint2 tw[Q];   // SignSGD: the run's bf16 table row
  f32x4 tg[Q];   // dense: the run's fp32 gradient table row
  if constexpr (OUT == kOutSignSGD) load_quads<L, Q, EXACT>(a.table, key, a.quads, lane, tw);
  if constexpr (OUT == kOutDense && Q == 1) load_grad_row<L, Q, EXACT>(a, key, lane, tg);
  // start: range c0 is sorted, so the run begins after its smaller keys
  int64_t start = r0;
  const u32x4 *kp = reinterpret_cast<const u32x4 *>(a.keys + r0);
#pragma unroll
  for (int j = 0; j < kRange / 4; ++j) {
    const u32x4 k4 = kp[j];
    start += (k4.x != key) + (k4.y != key) + (k4.z != key) + (k4.w != key);
  }
  // stop: the first position past r0 + 2 * kRange (which holds key) whose
  // key differs, 4 * kWave positions per step, each wavefront on its own
  int64_t stop = -1;
  for (int64_t p0 = r0 + 2 * kRange + 1; stop < 0; p0 += 4 * kWave) {
    int leave_at = 4;  // first of this lane's 4 positions past the run
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      const int64_t p = p0 + 4 * wl + e;
      leave_at = (p >= a.n || a.keys[p] != key) ? e : leave_at;
    }
    const unsigned long long leave = __ballot(leave_at < 4);
    if (leave != 0ull) {
      const int src = __ffsll((long long)leave) - 1;
      stop = p0 + 4 * src + __shfl(leave_at, src, kWave);
    }
  }
  const int64_t c1 = (stop - 1) / kRange;  // range of the run's last position
  double acc[Q][4];
  zero_acc<Q>(acc);
  uint32_t vv[kRange];
  if (Q == 1 && c0 + g <= c1) load_vals(a.vals, (c0 + g) * kRange, vv);
  if constexpr (Q == 1) {
    // a whole range of rows in flight, the next range's indices fetched
    // while they arrive
#pragma unroll 1
    for (int64_t c = c0 + g; c <= c1; c += G) {
      uint2 rows[kRange][Q];
#pragma unroll
      for (int q = 0; q < kRange; ++q) {
        const int64_t p = c * kRange + q;
        load_row<L, Q, EXACT, NT>(a, (p >= start && p < stop) ? vv[q] : 0u, lane, rows[q]);
      }
      if (c + G <= c1) load_vals(a.vals, (c + G) * kRange, vv);
#pragma unroll
      for (int q = 0; q < kRange; ++q) {
        const int64_t p = c * kRange + q;
        add_quads_if<Q>(acc, rows[q], p >= start && p < stop);
      }
    }
  } else {
    // wide rows: batches of kRange / Q rows, one batch at a time (a loop the
    // compiler keeps rolled, so it cannot hoist every batch's loads at once)
    constexpr int B = kRange / Q > 0 ? kRange / Q : 1;
#pragma unroll 1
    for (int64_t p0 = (c0 + g) * kRange; p0 <= c1 * kRange; p0 += (int64_t)G * kRange) {
#pragma unroll 1
      for (int b0 = 0; b0 < kRange; b0 += B) {
        uint32_t idx[B];
#pragma unroll
        for (int qq = 0; qq < B; ++qq) idx[qq] = a.vals[p0 + b0 + qq];
        uint2 rows[B][Q];
#pragma unroll
        for (int qq = 0; qq < B; ++qq) {
          const int64_t p = p0 + b0 + qq;
          load_row<L, Q, EXACT, NT>(a, (p >= start && p < stop) ? idx[qq] : 0u, lane, rows[qq]);
        }
#pragma unroll
        for (int qq = 0; qq < B; ++qq) {
          const int64_t p = p0 + b0 + qq;
          add_quads_if<Q>(acc, rows[qq], p >= start && p < stop);
        }
      }
    }
  }
  // walker 0 adds the other walkers' sums in walker order
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    if (g > 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_part[g][lane * 4 + e] = acc[k][e];
    __syncthreads();
    if (g == 0)
#pragma unroll 1
      for (int h = 1; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] += s_part[h][lane * 4 + e];
    __syncthreads();
  }
  if (g == 0) emit_row<L, Q, OUT>(key, u, a, lane, acc, tw, tg);
}

// Long runs (hot rows, longer than a range).  Block b checks which of the
// ranges [b * long_span, (b + 1) * long_span) end in a long run (three keys
// per range) and sums those runs in range order, the whole block on one run:
// the run's end is found by a scan of the keys, the block's G walkers sum the
// run's ranges c0 + g, c0 + g + G, ... (each range's indices fetched one
// range ahead, its rows all in flight), and walker 0 adds the walkers' sums
// in walker order before writing the row.  Fixed assignment and fixed order keep the result
// deterministic.
template <int L, int Q, int OUT, bool EXACT, bool NT>
__device__ __forceinline__ void long_runs(const WalkArgs &a) {
  __shared__ double s_part[kWalkThreads / L][L * 4];
  __shared__ uint32_t s_list[kWalkThreads];
  __shared__ int s_wave_count[kWalkThreads / kWave];
  const int wl = __lane_id(), wave = threadIdx.x / kWave;
  const int64_t first = (int64_t)blockIdx.x * a.long_span;
  const int64_t last = min(a.num_ranges, first + a.long_span);
  for (int64_t b0 = first; b0 < last; b0 += kWalkThreads) {
    // this stretch's flagged ranges, in range order
    const int64_t r = b0 + threadIdx.x;
    bool flagged = false;
    if (r < last) {
      const int64_t at = r * kRange;
      flagged = last_run_long(r, a.n, a.sentinel, a.keys[at > 0 ? at - 1 : 0],
                              a.keys[min(at + kRange - 1, a.n - 1)],
                              a.keys[min(at + 2 * kRange, a.n - 1)]);
    }
    const unsigned long long bal = __ballot(flagged);
    if (wl == 0) s_wave_count[wave] = __popcll(bal);
    __syncthreads();
    int at = __popcll(bal & ((1ull << wl) - 1ull)), count = 0;
#pragma unroll
    for (int v = 0; v < kWalkThreads / kWave; ++v) {
      at += v < wave ? s_wave_count[v] : 0;
      count += s_wave_count[v];
    }
    if (flagged) s_list[at] = (uint32_t)r;
    __syncthreads();
    for (int i = 0; i < count; ++i) long_run<L, Q, OUT, EXACT, NT>(a, s_list[i], s_part);
    __syncthreads();  // s_list and s_wave_count are rewritten for the next stretch
  }
}

// The apply kernel: blocks [0, long_blocks) sum the long runs, the rest are
// range walkers, kWalkThreads / L walkers per block.
template <int L, int Q, int OUT, bool EXACT, bool NT>
__global__ __launch_bounds__(kWalkThreads) void segment_reduce_kernel(const WalkArgs a) {
  if (OUT == kOutSparse && blockIdx.x == 0 && threadIdx.x == 0)
    *a.num_unique = (int64_t)*a.unique_total;
  if (blockIdx.x < a.long_blocks) {
    long_runs<L, Q, OUT, EXACT, NT>(a);
  } else {
    // Walker blocks take their ranges stripe by stripe: the GPU hands
    // consecutive blocks to its kXcds XCDs in turn, so the blocks of stripe
    // blk % kXcds all run on one XCD, which then walks one contiguous part
    // of the sorted order (the keys at its range boundaries and the runs
    // that cross into the next range stay in that XCD's L2).  The blocks
    // past the last whole stripe keep their order.
    const int64_t nb = (int64_t)gridDim.x - a.long_blocks;
    const int64_t blk = (int64_t)blockIdx.x - a.long_blocks;
    const int64_t full = nb / kXcds * kXcds;
    walk_range<L, Q, OUT, EXACT, NT>(a, blk < full ? blk % kXcds * (nb / kXcds) + blk / kXcds
                                                   : blk);
  }
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
  int64_t num_tiles, num_ranges, slot_tiles;
  int bits, passes, per_pass;
  int64_t status_words;  // look-back words the workspace holds
  size_t keys_a, vals_a, keys_b, vals_b, status, counters, head_off,
      scalars, total;
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
  p->scalars = take(64);
  p->total = off;
  return true;
}

// The sorted path needs 32-bit keys (table_rows itself is the drop key) and
// 32-bit flat indices.
inline bool sorted_limits_ok(int64_t n, int64_t table_rows) {
  return table_rows < (int64_t)UINT32_MAX && n < (int64_t)UINT32_MAX;
}

template <int L, int Q, int OUT>
void launch_walkers(const WalkArgs &a, hipStream_t s) {
  const int64_t threads = a.num_ranges * L;
  const unsigned blocks =
      a.long_blocks + (unsigned)((threads + kWalkThreads - 1) / kWalkThreads);
  const bool exact = a.quads == (int64_t)Q * L;
  if (exact && a.stream_grads)
    hipLaunchKernelGGL((segment_reduce_kernel<L, Q, OUT, true, true>), dim3(blocks),
                       dim3(kWalkThreads), 0, s, a);
  else if (exact)
    hipLaunchKernelGGL((segment_reduce_kernel<L, Q, OUT, true, false>), dim3(blocks),
                       dim3(kWalkThreads), 0, s, a);
  else if (a.stream_grads)
    hipLaunchKernelGGL((segment_reduce_kernel<L, Q, OUT, false, true>), dim3(blocks),
                       dim3(kWalkThreads), 0, s, a);
  else
    hipLaunchKernelGGL((segment_reduce_kernel<L, Q, OUT, false, false>), dim3(blocks),
                       dim3(kWalkThreads), 0, s, a);
}

// One quad (4 values) per lane: a walker is quads lanes wide, up to a whole
// wavefront (head_dim 256: one 64-lane walker per wavefront, each load
// instruction one 512-byte bf16 row, each store one 1 KB fp32 row); wider
// rows give each lane 2, 4 or 8 quads.
template <int OUT>
void dispatch_walkers(const WalkArgs &a, hipStream_t s) {
  const int64_t q = a.quads;
  if (q <= 2) launch_walkers<2, 1, OUT>(a, s);
  else if (q <= 4) launch_walkers<4, 1, OUT>(a, s);
  else if (q <= 8) launch_walkers<8, 1, OUT>(a, s);
  else if (q <= 16) launch_walkers<16, 1, OUT>(a, s);
  else if (q <= 32) launch_walkers<32, 1, OUT>(a, s);
  else if (q <= 64) launch_walkers<64, 1, OUT>(a, s);
  else if (q <= 128) launch_walkers<64, 2, OUT>(a, s);
  else if (q <= 256) launch_walkers<64, 4, OUT>(a, s);
  else launch_walkers<64, 8, OUT>(a, s);
}

// Workspace views shared by the plan and the apply.
struct Views {
  uint32_t *keys_a, *vals_a, *keys_b, *vals_b;
  uint64_t *status;
  uint32_t *counters, *head_off, *scalars;
  const uint32_t *sorted_keys, *sorted_vals;  // where the last sort pass leaves them
};

Views views_of(const Plan &p, void *ws) {
  char *base = static_cast<char *>(ws);
  Views v;
  v.keys_a = reinterpret_cast<uint32_t *>(base + p.keys_a);
  v.vals_a = reinterpret_cast<uint32_t *>(base + p.vals_a);
  v.keys_b = reinterpret_cast<uint32_t *>(base + p.keys_b);
  v.vals_b = reinterpret_cast<uint32_t *>(base + p.vals_b);
  v.status = reinterpret_cast<uint64_t *>(base + p.status);
  v.counters = reinterpret_cast<uint32_t *>(base + p.counters);
  v.head_off = reinterpret_cast<uint32_t *>(base + p.head_off);
  v.scalars = reinterpret_cast<uint32_t *>(base + p.scalars);
  // passes alternate a -> b -> a ...: an odd pass count ends in a
  v.sorted_keys = (p.passes % 2 == 1) ? v.keys_a : v.keys_b;
  v.sorted_vals = (p.passes % 2 == 1) ? v.vals_a : v.vals_b;
  return v;
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
  int64_t *err;
};

template <int ITEMS>
void launch_pass(int src, const SortLayout &L, const PassArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)L.num_tiles), block(kSortThreads);
  if (src == kSrcIds)
    hipLaunchKernelGGL((onesweep_kernel<kSrcIds, ITEMS>), grid, block, 0, s, a.ids, nullptr,
                       nullptr, L.sg, a.table_rows, a.shift, a.width, a.hist, a.status, a.ticket,
                       a.keys_out, a.vals_out, a.err);
  else if (src == kSrcKeysIota)
    hipLaunchKernelGGL((onesweep_kernel<kSrcKeysIota, ITEMS>), grid, block, 0, s, nullptr,
                       a.keys_in, nullptr, L.sg, a.table_rows, a.shift, a.width, a.hist, a.status,
                       a.ticket, a.keys_out, a.vals_out, a.err);
  else
    hipLaunchKernelGGL((onesweep_kernel<kSrcKeys, ITEMS>), grid, block, 0, s, nullptr, a.keys_in,
                       a.vals_in, L.sg, a.table_rows, a.shift, a.width, a.hist, a.status,
                       a.ticket, a.keys_out, a.vals_out, a.err);
}

// Plan: sort the row ids and give every distinct row its slot (U is left
// in the workspace scalars).  Needs only the ids: given (ids), or computed
// from the tokens (hp, when ids is null).
int plan_sorted(const int64_t *ids, const HashParams *hp, int64_t n, int64_t table_rows,
                const Plan &p, void *ws, int64_t *err, hipStream_t s) {
  const Views v = views_of(p, ws);
  uint32_t *tickets = v.counters;              // [4], then the slot scan's
  uint32_t *hist = v.counters + kTicketWords;  // [copy][segment][4][kMaxBins]
  SortLayout L = whole_sort(p, n);
  const bool heads = ids == nullptr && head_sort(*hp, n / hp->H, p, &L);
  const int64_t sort_words = (int64_t)L.passes * L.num_tiles * kMaxBins;
  const int64_t status_len = sort_words + p.slot_tiles;
  const int64_t counters_len = kTicketWords + (int64_t)L.sg.copies * L.sg.count * 4 * kMaxBins;
  const int64_t clear_len = status_len > counters_len ? status_len : counters_len;
  hipLaunchKernelGGL(sort_clear_kernel, dim3((unsigned)((clear_len + 255) / 256)), dim3(256), 0,
                     s, v.status, status_len, v.counters, (int)counters_len);
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
                       s, ids, n, table_rows, L.passes, L.per_pass, L.bits, hist, err);
  } else if (heads) {
    const int64_t chunks = (L.sg.len + kHeadTokens - 1) / kHeadTokens;
    const dim3 grid((unsigned)(L.sg.count * chunks));
    switch (hp->n) {
#define ENGRAM_PLAN_HEADS_CASE(N)                                                             \
  case N:                                                                                     \
    hipLaunchKernelGGL(plan_hash_heads_kernel<N>, grid, dim3(kHeadThreads), 0, s, *hp, L.sg,    \
                       chunks, L.passes, L.per_pass, L.bits, hashed, hist);                   \
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
    hipLaunchKernelGGL(plan_hash_kernel, dim3((unsigned)((tokens + 63) / 64)),
                       dim3(kSortThreads), 0, s, *hp, tokens, L.passes, L.per_pass, L.bits,
                       hashed, hist);
  }
  for (int pass = 0; pass < L.passes; ++pass) {
    const int shift = pass * L.per_pass;
    const int width = L.bits - shift < L.per_pass ? L.bits - shift : L.per_pass;
    const PassArgs a = {ids, pass == 0 ? hashed : out_k(pass - 1),
                        pass == 0 ? nullptr : out_v(pass - 1), table_rows, shift, width,
                        hist + pass * kMaxBins, v.status + (int64_t)pass * L.num_tiles * kMaxBins,
                        tickets + pass, out_k(pass), out_v(pass), err};
    const int src = pass > 0 ? kSrcKeys : (ids != nullptr ? kSrcIds : kSrcKeysIota);
    if (L.items == kSortItems)
      launch_pass<kSortItems>(src, L, a, s);
    else
      launch_pass<kSortItems / 2>(src, L, a, s);
  }
  // distinct-row slots
  hipLaunchKernelGGL(range_slots_kernel, dim3((unsigned)p.slot_tiles), dim3(kSlotThreads), 0, s,
                     v.sorted_keys, n, (uint32_t)table_rows, p.num_ranges, v.status + sort_words,
                     tickets + kSlotTicketAt, v.head_off, v.scalars, err);
  return launch_status();
}

// Outputs of an apply; the ones the output mode does not use are null.
struct ApplyOut {
  int mode;  // kOutDense, kOutSparse or kOutSignSGD
  float *grad_table;
  int64_t *unique_ids;
  float *unique_grads;
  int64_t *num_unique;
  void *table;  // bf16
  float lr;
};

// Apply: the per-row sums of one gradient tensor, given the plan of its ids.
int apply_sorted(const void *grads, int64_t n, int64_t dim, int64_t table_rows, const Plan &p,
                 void *ws, const ApplyOut &o, hipStream_t s) {
  const Views v = views_of(p, ws);
  WalkArgs a;
  a.keys = v.sorted_keys;
  a.vals = v.sorted_vals;
  a.n = n;
  a.sentinel = (uint32_t)table_rows;
  a.grads = static_cast<const uint2 *>(grads);
  a.stream_grads = n * dim * 2 > kStreamGradBytes;
  a.quads = dim / 4;
  a.dim = dim;
  a.head_off = v.head_off;
  a.num_ranges = p.num_ranges;
  a.grad_table = o.grad_table;
  a.unique_ids = o.unique_ids;
  a.unique_grads = o.unique_grads;
  a.table = static_cast<uint2 *>(o.table);
  a.lr = o.lr;
  // long-run blocks: at most kLongBlocks, each looking after at least
  // kLongSpan ranges (a long run spans 3 ranges or more)
  int64_t lb = p.num_ranges >= 3 ? (p.num_ranges + kLongSpan - 1) / kLongSpan : 0;
  lb = lb < kLongBlocks ? lb : kLongBlocks;
  a.long_blocks = (uint32_t)lb;
  a.long_span = lb > 0 ? (p.num_ranges + lb - 1) / lb : 0;
  a.unique_total = v.scalars;
  a.num_unique = o.num_unique;
  if (o.mode == kOutSparse)
    dispatch_walkers<kOutSparse>(a, s);
  else if (o.mode == kOutDense)
    dispatch_walkers<kOutDense>(a, s);
  else
    dispatch_walkers<kOutSignSGD>(a, s);
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

// ------------------------------------------------------- static scratch ---
// The workspace of engram_scatter_add_rowsparse_noalloc: a fixed device
// array of the library (each device holds its own copy from the time the
// library's code is loaded on it until the process ends), for callers that
// cannot allocate.  Host code never uses the array's name as a device
// address: the address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
constexpr size_t kStaticScratchBytes = ENGRAM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint64_t scratch[kStaticScratchBytes / sizeof(uint64_t)];

struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t rc = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch`, or null.
void *static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot &slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    void *p = nullptr;
    slot.rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    slot.ptr = slot.rc == hipSuccess ? p : nullptr;
  });
  return slot.ptr;
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

// Shared argument checks; fills the plan.  Returns ENGRAM_OK or an error.
static int check_sorted(int64_t n, int64_t table_rows, int64_t head_dim, Plan *p) {
  if (!make_plan(n, table_rows, head_dim, p) || !sorted_limits_ok(n, table_rows))
    return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

static int check_workspace(const Plan &p, const void *ws, size_t bytes) {
  if (ws == nullptr || bytes < p.total || !aligned16(ws)) return ENGRAM_EWORKSPACE;
  return ENGRAM_OK;
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
  return plan_sorted(d_row_ids, nullptr, n, table_rows, p, d_workspace, d_err_count,
                     as_stream(stream));
}

extern "C" int engram_scatter_apply(const void *d_grads, int64_t n, int64_t head_dim,
                                    int64_t table_rows, float *d_grad_table,
                                    int64_t *d_unique_ids, float *d_unique_grads,
                                    int64_t *d_num_unique, void *d_workspace,
                                    size_t workspace_bytes, void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  const bool dense = d_grad_table != nullptr;
  const bool sparse =
      d_unique_ids != nullptr || d_unique_grads != nullptr || d_num_unique != nullptr;
  if (dense == sparse) return ENGRAM_EINVAL;  // exactly one output form
  if (sparse && (d_unique_ids == nullptr || d_unique_grads == nullptr || d_num_unique == nullptr))
    return ENGRAM_EINVAL;
  hipStream_t s = as_stream(stream);
  if (n == 0) {
    if (sparse) {
      hipLaunchKernelGGL(write_zero_kernel, dim3(1), dim3(1), 0, s, d_num_unique);
      return launch_status();
    }
    return ENGRAM_OK;
  }
  if (d_grads == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || (dense && !aligned16(d_grad_table)) ||
      (sparse && !aligned16(d_unique_grads)))
    return ENGRAM_EALIGN;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  const ApplyOut o = {sparse ? kOutSparse : kOutDense, d_grad_table, d_unique_ids,
                      d_unique_grads, d_num_unique, nullptr, 0.0f};
  return apply_sorted(d_grads, n, head_dim, table_rows, p, d_workspace, o, s);
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
  int rc = check_workspace(p, d_workspace, workspace_bytes);
  if (rc != ENGRAM_OK) return rc;
  if ((rc = plan_sorted(d_row_ids, nullptr, n, table_rows, p, d_workspace, d_err_count, s)) !=
      ENGRAM_OK)
    return rc;
  const ApplyOut o = {kOutDense, d_grad_table, nullptr, nullptr, nullptr, nullptr, 0.0f};
  return apply_sorted(d_grads, n, head_dim, table_rows, p, d_workspace, o, s);
}

extern "C" int engram_scatter_add_rowsparse(const int64_t *d_row_ids, int64_t n,
                                            const void *d_grads, int64_t head_dim,
                                            int64_t table_rows, int64_t *d_unique_ids,
                                            float *d_unique_grads, int64_t *d_num_unique,
                                            void *d_workspace, size_t workspace_bytes,
                                            int64_t *d_err_count, void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
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
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  if ((rc = plan_sorted(d_row_ids, nullptr, n, table_rows, p, d_workspace, d_err_count, s)) !=
      ENGRAM_OK)
    return rc;
  const ApplyOut o = {kOutSparse, nullptr, d_unique_ids, d_unique_grads, d_num_unique, nullptr,
                      0.0f};
  return apply_sorted(d_grads, n, head_dim, table_rows, p, d_workspace, o, s);
}

extern "C" int engram_scatter_apply_signsgd(const void *d_grads, int64_t n, int64_t head_dim,
                                            int64_t table_rows, void *d_table, float lr,
                                            void *d_workspace, size_t workspace_bytes,
                                            void *stream) {
  Plan p;
  int rc = check_sorted(n, table_rows, head_dim, &p);
  if (rc != ENGRAM_OK) return rc;
  if (n == 0) return ENGRAM_OK;
  if (d_grads == nullptr || d_table == nullptr) return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_table)) return ENGRAM_EALIGN;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  const ApplyOut o = {kOutSignSGD, nullptr, nullptr, nullptr, nullptr, d_table, lr};
  return apply_sorted(d_grads, n, head_dim, table_rows, p, d_workspace, o, as_stream(stream));
}

extern "C" int engram_scatter_plan_tokens(const int64_t *d_tokens, const int64_t *d_seq_ids,
                                          int64_t batch, int64_t seq, int32_t ngram_size,
                                          int32_t heads_per_ngram, int64_t eos_id,
                                          const int64_t *h_multipliers, const int64_t *h_primes,
                                          const int64_t *h_offsets, int64_t table_rows,
                                          int64_t head_dim, void *d_workspace,
                                          size_t workspace_bytes, void *stream) {
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
  if ((tokens + 63) / 64 > INT32_MAX) return ENGRAM_EINVAL;
  if ((rc = check_workspace(p, d_workspace, workspace_bytes)) != ENGRAM_OK) return rc;
  return plan_sorted(nullptr, &hp, n, table_rows, p, d_workspace, nullptr, as_stream(stream));
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
  if (d_num_unique == nullptr) return ENGRAM_EINVAL;
  if (p.total > kStaticScratchBytes) return ENGRAM_EWORKSPACE;  // more ids than the array plans
  hipStream_t s = as_stream(stream);
  if (n == 0) {
    hipLaunchKernelGGL(write_zero_kernel, dim3(1), dim3(1), 0, s, d_num_unique);
    return launch_status();
  }
  if (d_row_ids == nullptr || d_grads == nullptr || d_unique_ids == nullptr ||
      d_unique_grads == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned16(d_grads) || !aligned16(d_unique_grads)) return ENGRAM_EALIGN;
  void *ws = static_scratch();
  if (ws == nullptr) return ENGRAM_EHIP;
  if ((rc = plan_sorted(d_row_ids, nullptr, n, table_rows, p, ws, d_err_count, s)) != ENGRAM_OK)
    return rc;
  const ApplyOut o = {kOutSparse, nullptr, d_unique_ids, d_unique_grads, d_num_unique, nullptr,
                      0.0f};
  return apply_sorted(d_grads, n, head_dim, table_rows, p, ws, o, s);
}
