// engram_apply_dev.h -- the apply of the sorted scatter-add for gfx950, as
// device code: one kernel per output form (dense fp32 table, row-sparse, or
// the SignSGD step on the bf16 table), each built in its own translation unit
// (engram_apply_dense.hip, engram_apply_sparse.hip, engram_apply_signsgd.hip).
//
// What is computed follows the NeMo AutoModel v0.7 API page
// "qwen3_8_flash_next.engram" (Qwen3_8_FlashNextOwnerShardedEmbedding: the
// owner alone accumulates a row's gradient), the prime-rl pull request 3434
// Validation section and the prime-rl v0.9.1.dev179 release notes,
// Validation (FP32 reduction defaults).  The pages do not fix the summation
// order or precision; the reading taken here: each row's contributions are
// summed in fp64, rounded once to fp32, and added to the fp32 gradient row
// with one fp32 add.  Sums of bf16 values are exact in fp64 while the bits
// of the terms and of every partial sum span at most 53 places; then the
// result does not depend on the order of the additions.  Past that (terms
// whose magnitudes differ by more than about 2^45) the kernels' order,
// which differs from a sequential sum's, can round differently.
//
// Range walkers: a group of head_dim/4 lanes (one 4-value quad of the row
// per lane, up to a whole wavefront) takes one 16-position range of the
// sorted order, issues all its loads at once (keys, flat indices, then the
// gradient rows) and sums runs in fp64 registers.  A run that starts and
// ends inside the range is written once (dense read-modify-write, row-sparse
// store, or the SignSGD step on the bf16 table row); a run cut by the
// range's end but ending in the next range is finished by the same walker.
// Runs longer than that (hot rows, found from three sorted keys per range)
// are summed by the leading blocks of the same launch in aligned chunks of
// kChunk sorted positions: the block of a chunk sums each long run that
// starts there, its walkers taking interleaved 16-position pieces and adding
// their sums in a fixed order.  A long run that ends in its first chunk or
// the next is written at once; one that spans three chunks or more leaves an
// fp64 partial-sum row in each chunk it touches, and a second launch
// (combine_kernel) adds those in chunk order.  No work item waits on another,
// hot rows do not serialise a walker, and a row that holds a large share of
// all positions (a padding row) is spread over as many blocks as it has
// chunks.
#pragma once

#include "engram_scatter_dev.h"

namespace engram {

// (kWalkThreads, kLongBlocks and walker_lanes, the launch's shape, are in
// engram_host.h, where the entry points check the grid before any launch.)
constexpr int64_t kCombineBlocks = 256;  // most blocks of the second launch
constexpr int64_t kXcds = 8;           // XCDs of an MI355X (blocks go to them in turn)
// Gradient tensors larger than this are read with non-temporal loads: half
// the MI355X's 256 MB Infinity Cache, so a tensor that could still be cached
// when the apply runs is read normally.
constexpr int64_t kStreamGradBytes = int64_t(128) << 20;

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
  uint32_t *chunk_owner;   // per chunk: slot + 1 of the long run that leaves it, or 0
  double *partials;        // per chunk: [2, dim] fp64 rows (run entering, run leaving)
  int64_t num_chunks;
  uint32_t long_blocks;    // leading blocks of the grid: they sum long runs by chunk
  uint32_t long_group;     // consecutive chunks a long block takes at a time
  const PlanScalars *plan;  // U, the stall flag and the stamp, from the plan
  int64_t *num_unique;      // row-sparse output count
  int64_t *err;             // error counter, or null
};

// Enqueue the apply for one output form (one translation unit each).
void walk_dense(const WalkArgs &a, hipStream_t s);
void walk_sparse(const WalkArgs &a, hipStream_t s);
void walk_signsgd(const WalkArgs &a, hipStream_t s);

namespace {

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

// A table row index read from the plan, kept inside the table (a plan the
// stamp vouches for never needs it; a damaged workspace then still reads
// valid rows, and emit_row drops what it would write).
__device__ __forceinline__ uint32_t table_row(const WalkArgs &a, uint32_t key) {
  return key < a.sentinel ? key : a.sentinel - 1;
}

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
  idx = (int64_t)idx < a.n ? idx : (uint32_t)(a.n - 1);  // inside the gradients, whatever the plan
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
  // a row outside the table, or a slot past the output, cannot come from a
  // plan of these ids: write nothing and count it
  if (key >= a.sentinel || (OUT == kOutSparse && (int64_t)u >= a.n)) {
    if (lane == 0) add_mark(a.err, kNoPlanMark);
    return;
  }
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
        const uint32_t row = table_row(a, head ? kk[q] : kk[0]);
        if constexpr (OUT == kOutSignSGD)
          load_quads<L, Q, EXACT>(a.table, row, a.quads, lane, tw[q]);
        else
          load_grad_row<L, Q, EXACT>(a, row, lane, tg[q]);
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

// Walker 0 adds the other walkers' sums to its own, in walker order (through
// LDS, one quad of the row at a time).
template <int L, int Q>
__device__ __forceinline__ void block_combine(double (&acc)[Q][4],
                                              double (&s_part)[kWalkThreads / L][L * 4]) {
  constexpr int G = kWalkThreads / L;
  const int lane = threadIdx.x % L, g = threadIdx.x / L;
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
}

// The partial-sum row of chunk j, side 0 (the long run entering the chunk)
// or 1 (the long run leaving it).
__device__ __forceinline__ f64x2 *partial_row(const WalkArgs &a, int64_t j, int side) {
  return reinterpret_cast<f64x2 *>(a.partials + (2 * j + side) * a.dim);
}

// Walker 0's sum into a partial-sum row (fp64, exactly as held).
template <int L, int Q>
__device__ __forceinline__ void store_partial(const WalkArgs &a, f64x2 *row, int lane,
                                              const double (&acc)[Q][4]) {
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int64_t qd = lane + (int64_t)k * L;
    if (qd >= a.quads) continue;
    row[2 * qd] = f64x2{acc[k][0], acc[k][1]};
    row[2 * qd + 1] = f64x2{acc[k][2], acc[k][3]};
  }
}

// Long-run blocks hold kGroupChunks chunks at a time in LDS: the keys of
// each chunk with the two ranges before and after it, which the tests read
// (positions P0 - kHalo .. P1 + kHalo - 1; 0xFFFFFFFF before the first
// position, the drop key past the last), the flat indices, and per range
// the chunk offsets of its first and last distinct-row starts and the slot
// of its last distinct row.  Keys and indices arrive as 16-byte vectors.
constexpr int kChunkRanges = (int)(kChunk / kRange);
constexpr int kGroupChunks = kLongGroup;
constexpr int kHalo = 2 * kRange;
constexpr int kChunkKeys = kHalo + (int)kChunk + kHalo;

template <int L>
struct LongLds {
  double part[kWalkThreads / L][L * 4];
  alignas(16) uint32_t keys[kGroupChunks][kChunkKeys];
  // indices; one row more, for the chunk after the group's last
  alignas(16) uint32_t vals[kGroupChunks + 1][kChunk];
  uint32_t slot[kGroupChunks][kChunkRanges];
  uint32_t far_before[kGroupChunks];  // key at P0 - kChunk - 1 (0xFFFFFFFF: none)
  uint32_t far_after[kGroupChunks];   // key at P0 + 2 kChunk (the drop key: none)
  unsigned long long end_next;        // end of a run in the next chunk
  uint16_t first[kGroupChunks][kChunkRanges];
  uint16_t last[kGroupChunks][kChunkRanges];
  uint32_t has_start[kGroupChunks];  // bit r: range r holds a distinct-row start
  uint32_t flagged[kGroupChunks];    // bit r: range r's last run is long
  uint32_t enters[kGroupChunks];     // a long run enters the chunk
};

// The sum of chunk offsets [s, e) of one row (flat indices from LDS) by the
// whole block: walker g takes offsets s + 16 g .. s + 16 g + 15, then
// s + 16 (g + G) ..., all 16 rows in flight at once (wide rows: in batches);
// walker 0 then adds the walkers' sums in walker order.  The order of every
// addition depends only on [s, e).  Walker 0's acc holds the sum on return.
template <int L, int Q, bool EXACT, bool NT>
__device__ __forceinline__ void block_sum_lds(const WalkArgs &a, const uint32_t *vals, int s,
                                              int e, double (&acc)[Q][4],
                                              double (&part)[kWalkThreads / L][L * 4]) {
  constexpr int G = kWalkThreads / L;
  constexpr int B = Q == 1 ? kRange : (kRange / Q > 0 ? kRange / Q : 1);  // rows in flight
  const int lane = threadIdx.x % L, g = threadIdx.x / L;
  zero_acc<Q>(acc);
#pragma unroll 1
  for (int b = s + kRange * g; b < e; b += kRange * G) {
#pragma unroll 1
    for (int b0 = 0; b0 < kRange; b0 += B) {
      uint2 rows[B][Q];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int o = b + b0 + q;
        load_row<L, Q, EXACT, NT>(a, o < e ? vals[o] : 0u, lane, rows[q]);
      }
#pragma unroll
      for (int q = 0; q < B; ++q) add_quads_if<Q>(acc, rows[q], b + b0 + q < e);
    }
  }
  block_combine<L, Q>(acc, part);
}

// Chunks [j0, j0 + cnt) into LDS (cnt <= kGroupChunks), then the tests of
// every range of them: one round of loads for the whole group.  The key and
// index buffers hold whole ranges, so a 16-byte vector that starts before
// n is inside them (its positions past n read as the drop key).
template <int L>
__device__ __forceinline__ void load_group(const WalkArgs &a, int64_t j0, int cnt,
                                           LongLds<L> &s) {
  const int tid = threadIdx.x;
  constexpr int kKeyVecs = kChunkKeys / 4, kValVecs = (int)kChunk / 4;
  constexpr int kKeyIters = (kGroupChunks * kKeyVecs + kWalkThreads - 1) / kWalkThreads;
  constexpr int kValIters = (kGroupChunks * kValVecs + kWalkThreads - 1) / kWalkThreads;
  static_assert(kGroupChunks * kChunkRanges <= kWalkThreads, "one thread per range");
  static_assert(kHalo % 4 == 0 && kChunkKeys % 4 == 0, "whole vectors");
  const u32x4 *kv = reinterpret_cast<const u32x4 *>(a.keys);
  const u32x4 *vv = reinterpret_cast<const u32x4 *>(a.vals);
  u32x4 kx[kKeyIters] = {}, vx[kValIters] = {};
#pragma unroll
  for (int it = 0; it < kKeyIters; ++it) {
    const int i = tid + it * kWalkThreads, k = i / kKeyVecs;
    const int64_t p = (j0 + k) * kChunk - kHalo + 4 * (i - k * kKeyVecs);
    if (i < cnt * kKeyVecs && p >= 0 && p < a.n) kx[it] = kv[p / 4];
  }
#pragma unroll
  for (int it = 0; it < kValIters; ++it) {
    const int i = tid + it * kWalkThreads, k = i / kValVecs;
    const int64_t p = (j0 + k) * kChunk + 4 * (i - k * kValVecs);
    if (i < cnt * kValVecs && p < a.n) vx[it] = vv[p / 4];
  }
#pragma unroll
  for (int it = 0; it < kKeyIters; ++it) {
    const int i = tid + it * kWalkThreads, k = i / kKeyVecs, o = 4 * (i - k * kKeyVecs);
    const int64_t p = (j0 + k) * kChunk - kHalo + o;
    if (i < cnt * kKeyVecs) {
      u32x4 v = kx[it];
      const uint32_t pre = 0xFFFFFFFFu;
      v.x = p < 0 ? pre : (p < a.n ? v.x : a.sentinel);
      v.y = p < 0 ? pre : (p + 1 < a.n ? v.y : a.sentinel);
      v.z = p < 0 ? pre : (p + 2 < a.n ? v.z : a.sentinel);
      v.w = p < 0 ? pre : (p + 3 < a.n ? v.w : a.sentinel);
      *reinterpret_cast<u32x4 *>(&s.keys[k][o]) = v;
    }
  }
#pragma unroll
  for (int it = 0; it < kValIters; ++it) {
    const int i = tid + it * kWalkThreads, k = i / kValVecs, o = 4 * (i - k * kValVecs);
    if (i < cnt * kValVecs) *reinterpret_cast<u32x4 *>(&s.vals[k][o]) = vx[it];
  }
  {
    const int k = tid / kChunkRanges, r = tid % kChunkRanges;
    const int64_t c = (j0 + k) * kChunkRanges + r;  // this thread's range
    const int64_t P0 = (j0 + k) * kChunk;
    if (k < cnt && c + 1 < a.num_ranges) s.slot[k][r] = a.head_off[c + 1] - 1;
    if (k < cnt && r == 1)
      s.far_before[k] = P0 >= kChunk + 1 ? a.keys[P0 - kChunk - 1] : 0xFFFFFFFFu;
    if (k < cnt && r == 2) s.far_after[k] = P0 + 2 * kChunk < a.n ? a.keys[P0 + 2 * kChunk] : a.sentinel;
  }
  __syncthreads();
  // per range: distinct-row starts (key differs from the one before) and the
  // walkers' long-run test; the first thread of a chunk tests the run that
  // enters it
  const int k = tid / kChunkRanges, r = tid % kChunkRanges;
  bool has = false, flag = false, enter = false;
  if (k < cnt) {
    const int64_t c = (j0 + k) * kChunkRanges + r, P0 = (j0 + k) * kChunk;
    const uint32_t *kk = &s.keys[k][kHalo + r * kRange];  // kk[q]: position 16 c + q
    int first = kRange, last = -1;
#pragma unroll
    for (int q = 0; q < kRange; ++q) {
      const bool st = kk[q] != kk[q - 1];
      first = (st && first == kRange) ? q : first;
      last = st ? q : last;
    }
    s.first[k][r] = (uint16_t)(r * kRange + first);
    s.last[k][r] = (uint16_t)(r * kRange + (last < 0 ? 0 : last));
    has = first < kRange;
    flag = last_run_long(c, a.n, a.sentinel, kk[-1], kk[kRange - 1], kk[2 * kRange]);
    if (r == 0) {
      const uint32_t *k0 = &s.keys[k][kHalo];  // k0[o]: position P0 + o
      enter = P0 > 0 && k0[0] != a.sentinel && k0[-1] == k0[0] &&
              (k0[-kRange - 1] == k0[0] || (P0 + kRange < a.n && k0[kRange] == k0[0]));
    }
  }
  const unsigned long long hb = __ballot(has), fb = __ballot(flag), eb = __ballot(enter);
  if (tid % 64 == 0 && tid / kChunkRanges < kGroupChunks) {
    const int k0 = tid / kChunkRanges;  // chunks k0 and k0 + 1 share this wavefront
    s.has_start[k0] = (uint32_t)hb;
    s.flagged[k0] = (uint32_t)fb;
    s.enters[k0] = (uint32_t)(eb & 1u);
    if (k0 + 1 < kGroupChunks) {
      s.has_start[k0 + 1] = (uint32_t)(hb >> 32);
      s.flagged[k0 + 1] = (uint32_t)(fb >> 32);
      s.enters[k0 + 1] = (uint32_t)((eb >> 32) & 1u);
    }
  }
  __syncthreads();
}

// The end of a run of `key` that holds P1 = (j + 1) * kChunk and ends in
// chunk j + 1 (not past P1 + kChunk), as an offset from P1, with chunk j + 1's
// flat indices put in LDS row k + 1 beside it.  When the group holds chunk
// j + 1 (k + 1 < cnt) both come from LDS; else one round of loads.
template <int L>
__device__ __forceinline__ int next_chunk_end(const WalkArgs &a, int64_t j, int k, int cnt,
                                              uint32_t key, LongLds<L> &s) {
  if (k + 1 < cnt) {
    const uint32_t has = s.has_start[k + 1];  // (no start at its offset 0: the run holds it)
    return has != 0 ? (int)s.first[k + 1][__ffs((int)has) - 1]
                    : (int)min(kChunk, a.n - (j + 1) * kChunk);
  }
  const int tid = threadIdx.x;
  const int64_t P1 = (j + 1) * kChunk;
  if (tid == 0) s.end_next = (unsigned long long)min(kChunk, a.n - P1);
  __syncthreads();
  static_assert(kChunk == 2 * kWalkThreads, "two positions a thread");
  const int o = 2 * tid;
  const int64_t p = P1 + o;
  if (p < a.n) {  // the buffers hold whole ranges: p + 1 is inside them
    const uint2 kk = *reinterpret_cast<const uint2 *>(a.keys + p);
    const uint2 vv = *reinterpret_cast<const uint2 *>(a.vals + p);
    s.vals[k + 1][o] = vv.x;
    s.vals[k + 1][o + 1] = vv.y;
    const int e = kk.x != key ? o : (p + 1 < a.n && kk.y != key ? o + 1 : -1);
    if (e >= 0) atomicMin(&s.end_next, (unsigned long long)e);
  }
  __syncthreads();
  return (int)s.end_next;
}

// One chunk of long-run work: positions [P0, P1) = [j * kChunk, ...) of the
// sorted order, held in LDS slot k of a group of cnt.  The long runs there
// are the one entering from the previous chunk and those starting in the
// chunk's ranges that a walker leaves out.  The block sums each run's
// positions; a run's end is the first distinct-row start after it (from the
// per-range starts).  A run that ends in this chunk or the next is summed
// whole by the chunk it starts in and written out at once (its output row
// read while the sum's loads are in flight).  A run that spans three chunks
// or more is split: every chunk it touches sums its own part into an fp64
// partial row (side 0: the run entering the chunk; side 1: the run leaving
// it, whose slot (+1) goes to chunk_owner[j], 0 when none) for the second
// launch.  The chunks on both sides of a boundary agree on which runs are
// split from the keys at P0 - kChunk - 1, P1 and P0 + 2 kChunk.  Block-uniform
// control flow throughout (every value it branches on comes from LDS after a
// barrier).
template <int L, int Q, int OUT, bool EXACT, bool NT>
__device__ __forceinline__ void long_chunk(const WalkArgs &a, int64_t j, int k, int cnt,
                                           LongLds<L> &s) {
  const int lane = threadIdx.x % L, g = threadIdx.x / L;
  const int64_t P0 = j * kChunk;
  const int len = (int)min(kChunk, a.n - P0);
  const bool more = P0 + len < a.n;  // a chunk follows
  const uint32_t has = s.has_start[k];
  const uint32_t *kk = &s.keys[k][kHalo];  // kk[o]: position P0 + o
  // the end (chunk offset) of a run that holds no distinct-row start in
  // ranges r and up: the first start there, else the chunk's end
  auto end_from = [&](int r) -> int {
    const uint32_t m = r < kChunkRanges ? has >> r : 0u;
    return m != 0 ? (int)s.first[k][r + __ffs((int)m) - 1] : len;
  };
  uint32_t owner = 0;  // slot + 1 of the split run that leaves the chunk
  double acc[Q][4];
  if (s.enters[k] != 0) {
    // split when it started two chunks back or more, or leaves this chunk
    // too; else the chunk before sums it whole
    const uint32_t ekey = kk[0];
    if (s.far_before[k] == ekey || (more && kk[len] == ekey)) {
      block_sum_lds<L, Q, EXACT, NT>(a, s.vals[k], 0, end_from(0), acc, s.part);
      if (g == 0) store_partial<L, Q>(a, partial_row(a, j, 0), lane, acc);
    }
  }
  for (uint32_t m = s.flagged[k]; m != 0; m &= m - 1) {
    const int r = __ffs((int)m) - 1;
    const int start = s.last[k][r];
    const uint32_t key = kk[start];
    int end = end_from(r + 2);  // the run holds range r + 2's first position
    const bool leaves = end == len && more && kk[len] == key;
    const bool split = leaves && s.far_after[k] == key;
    const uint32_t slot = s.slot[k][r];
    uint2 tw[Q];   // SignSGD: the run's bf16 table row
    f32x4 tg[Q];   // dense: the run's fp32 gradient table row
    if (!split && g == 0) {
      if constexpr (OUT == kOutSignSGD)
        load_quads<L, Q, EXACT>(a.table, table_row(a, key), a.quads, lane, tw);
      if constexpr (OUT == kOutDense && Q == 1)
        load_grad_row<L, Q, EXACT>(a, table_row(a, key), lane, tg);
    }
    if (leaves && !split) end = len + next_chunk_end<L>(a, j, k, cnt, key, s);
    // (offsets past len index LDS row k + 1: the next chunk's indices)
    block_sum_lds<L, Q, EXACT, NT>(a, s.vals[k], start, end, acc, s.part);
    if (g == 0) {
      if (split)
        store_partial<L, Q>(a, partial_row(a, j, 1), lane, acc);
      else
        emit_row<L, Q, OUT>(key, slot, a, lane, acc, tw, tg);
    }
    if (split) owner = slot + 1;
  }
  if (threadIdx.x == 0) a.chunk_owner[j] = owner;
}

// Long runs (hot rows, longer than a range), chunk by chunk.  Long block l
// of nlong takes the groups of a.long_group consecutive chunks l, l + nlong,
// l + 2 nlong, ... (a.long_group <= kGroupChunks), so a stretch of hot
// chunks (a padding row) is spread over all long blocks.
template <int L, int Q, int OUT, bool EXACT, bool NT>
__device__ __forceinline__ void long_chunks(const WalkArgs &a, int64_t l, int64_t nlong) {
  static_assert(kChunkRanges == 32 && kWalkThreads % 64 == 0,
                "a chunk's ranges are one half of a wavefront");
  __shared__ LongLds<L> s;
  const int64_t per = a.long_group;
  for (int64_t j0 = l * per; j0 < a.num_chunks; j0 += nlong * per) {
    const int cnt = (int)min(per, a.num_chunks - j0);
    load_group<L>(a, j0, cnt, s);
#pragma unroll 1
    for (int k = 0; k < cnt; ++k) long_chunk<L, Q, OUT, EXACT, NT>(a, j0 + k, k, cnt, s);
    __syncthreads();  // the group's LDS is rewritten next
  }
}

// Whether the workspace holds a complete plan of these n and table_rows,
// none of whose waits expired.  If not, nothing is written, and with
// `report` block 0 says so (U = 0 for the row-sparse output, and the mark in
// the error counter; the apply's second launch leaves that to the first).
template <int OUT>
__device__ __forceinline__ bool plan_ok(const WalkArgs &a, bool report) {
  const PlanScalars *pl = a.plan;
  const bool stalled = pl->stalled != 0;
  if (!stalled && pl->n == (uint64_t)a.n && pl->table_rows == (uint64_t)a.sentinel) return true;
  if (report && blockIdx.x == 0 && threadIdx.x == 0) {
    if (OUT == kOutSparse) *a.num_unique = 0;
    add_mark(a.err, stalled ? kStallMark : kNoPlanMark);
  }
  return false;
}

// The apply kernel: blocks [0, long_blocks) sum the long runs chunk by chunk
// (first, so that no long run is left for the end of the launch), the rest
// are range walkers, kWalkThreads / L walkers per block.
template <int L, int Q, int OUT, bool EXACT, bool NT>
__global__ __launch_bounds__(kWalkThreads) void segment_reduce_kernel(const WalkArgs a) {
  if (!plan_ok<OUT>(a, true)) return;
  if (OUT == kOutSparse && blockIdx.x == 0 && threadIdx.x == 0)
    *a.num_unique = (int64_t)a.plan->unique;
  if (blockIdx.x < a.long_blocks) {
    long_chunks<L, Q, OUT, EXACT, NT>(a, blockIdx.x, a.long_blocks);
    return;
  }
  // Walker blocks take their ranges stripe by stripe: the GPU hands
  // consecutive blocks to its kXcds XCDs in turn, so the blocks of stripe
  // blk % kXcds all run on one XCD, which then walks one contiguous part of
  // the sorted order (the keys at its range boundaries and the runs that
  // cross into the next range stay in that XCD's L2).  The blocks past the
  // last whole stripe keep their order.
  const int64_t nb = (int64_t)gridDim.x - a.long_blocks;
  const int64_t blk = (int64_t)blockIdx.x - a.long_blocks;
  const int64_t full = nb / kXcds * kXcds;
  walk_range<L, Q, OUT, EXACT, NT>(a, blk < full ? blk % kXcds * (nb / kXcds) + blk / kXcds
                                                 : blk);
}

// The apply's second launch: the long runs that cross chunks.  The run
// leaving chunk j (chunk_owner[j] = its slot + 1) is the sum, in chunk order,
// of chunk j's side-1 row and the side-0 rows of the chunks it enters, found
// from the first key of each later chunk.  Block b looks after chunks b,
// b + gridDim.x, ...: its threads read kWalkThreads of their owners at once
// and list the non-zero ones, which the block then finishes one by one.
// Walker g adds rows g, g + G, ... of a run and walker 0 adds the walkers'
// sums in walker order, so the order of the additions is fixed.
template <int L, int Q, int OUT, bool EXACT>
__global__ __launch_bounds__(kWalkThreads) void combine_kernel(const WalkArgs a) {
  constexpr int G = kWalkThreads / L;
  __shared__ double s_part[kWalkThreads / L][L * 4];
  __shared__ unsigned long long s_last;
  __shared__ uint32_t s_list[kWalkThreads];
  __shared__ uint32_t s_count;
  const int lane = threadIdx.x % L, g = threadIdx.x / L, tid = threadIdx.x;
  const int64_t stride = gridDim.x;
  for (int64_t j0 = blockIdx.x; j0 < a.num_chunks; j0 += stride * kWalkThreads) {
    // the owners, read beside the plan's stamp (one round trip)
    const int64_t jt = j0 + tid * stride;
    const uint32_t own = jt < a.num_chunks ? a.chunk_owner[jt] : 0u;
    if (j0 == blockIdx.x && !plan_ok<OUT>(a, false)) return;
    if (tid == 0) s_count = 0;
    __syncthreads();
    if (own != 0) s_list[atomicAdd(&s_count, 1u)] = (uint32_t)tid;
    __syncthreads();
    const uint32_t count = s_count;
#pragma unroll 1
    for (uint32_t i0 = 0; i0 < count; ++i0) {
      const int64_t j = j0 + (int64_t)s_list[i0] * stride;
      const uint32_t owner = a.chunk_owner[j];
      if (owner > (uint32_t)a.n || (j + 1) * kChunk >= a.n) {  // not from a plan of these ids
        if (tid == 0) add_mark(a.err, kNoPlanMark);
        continue;
      }
      const uint32_t key = a.keys[(j + 1) * kChunk - 1];
      uint2 tw[Q];   // SignSGD: the run's bf16 table row
      f32x4 tg[Q];   // dense: the run's fp32 gradient table row
      if (g == 0) {  // read while the chunks are found and summed
        if constexpr (OUT == kOutSignSGD)
          load_quads<L, Q, EXACT>(a.table, table_row(a, key), a.quads, lane, tw);
        if constexpr (OUT == kOutDense && Q == 1)
          load_grad_row<L, Q, EXACT>(a, table_row(a, key), lane, tg);
      }
      // the last chunk the run enters: the chunks after j whose first key is
      // the run's, kWalkThreads at a time
      if (tid == 0) s_last = (unsigned long long)(j + 1);
      __syncthreads();
      for (int64_t base = j + 1;; base += kWalkThreads) {
        const int64_t jj = base + tid;
        const bool in = jj < a.num_chunks && a.keys[jj * kChunk] == key;
        if (in) atomicMax(&s_last, (unsigned long long)jj);
        // the run is contiguous: it goes on past this batch only if the
        // batch's last chunk is in it
        if (!__syncthreads_or(in && tid == kWalkThreads - 1)) break;
      }
      const int64_t jl = (int64_t)s_last;
      double acc[Q][4];
      zero_acc<Q>(acc);
      // rows in order: chunk j side 1, then chunks j + 1 .. jl side 0;
      // walker g's rows g, g + G, ..., kRows of them in flight at a time
      constexpr int kRows = 4;
#pragma unroll 1
      for (int64_t i0 = g; i0 <= jl - j; i0 += (int64_t)G * kRows) {
        f64x2 lo[kRows][Q], hi[kRows][Q];
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
          const int64_t i = i0 + (int64_t)u * G;
          const f64x2 *row = partial_row(a, j + (i <= jl - j ? i : 0), i == 0 ? 1 : 0);
#pragma unroll
          for (int k = 0; k < Q; ++k) {
            const int64_t qd = lane + (int64_t)k * L;
            const bool ok = i <= jl - j && (EXACT || qd < a.quads);
            lo[u][k] = ok ? row[2 * qd] : f64x2{0.0, 0.0};
            hi[u][k] = ok ? row[2 * qd + 1] : f64x2{0.0, 0.0};
          }
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u)
#pragma unroll
          for (int k = 0; k < Q; ++k) {
            acc[k][0] += lo[u][k].x;
            acc[k][1] += lo[u][k].y;
            acc[k][2] += hi[u][k].x;
            acc[k][3] += hi[u][k].y;
          }
      }
      block_combine<L, Q>(acc, s_part);  // (its barriers also settle s_last's reads)
      if (g == 0) emit_row<L, Q, OUT>(key, owner - 1, a, lane, acc, tw, tg);
    }
    __syncthreads();  // s_list and s_count are rewritten next
  }
}

template <int L, int Q, int OUT>
void launch_walkers(WalkArgs a, hipStream_t s) {
  const int64_t walker_blocks = (a.num_ranges * L + kWalkThreads - 1) / kWalkThreads;
  // (the grid is apply_blocks(), which the entry points have checked)
  a.long_blocks = (uint32_t)long_blocks(a.num_chunks);
  a.long_group = (uint32_t)long_group(a.num_chunks);
  const unsigned blocks = (unsigned)(a.long_blocks + walker_blocks);
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
  // the long runs that cross chunks: usually none, or a handful
  const unsigned cblocks = (unsigned)(a.num_chunks < kCombineBlocks ? a.num_chunks : kCombineBlocks);
  if (exact)
    hipLaunchKernelGGL((combine_kernel<L, Q, OUT, true>), dim3(cblocks), dim3(kWalkThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((combine_kernel<L, Q, OUT, false>), dim3(cblocks), dim3(kWalkThreads), 0,
                       s, a);
}

// One quad (4 values) per lane: a walker is quads lanes wide, up to a whole
// wavefront (head_dim 256: one 64-lane walker per wavefront, each load
// instruction one 512-byte bf16 row, each store one 1 KB fp32 row); wider
// rows give each lane 2, 4 or 8 quads.
template <int OUT>
void dispatch_walkers(const WalkArgs &a, hipStream_t s) {
  const int64_t q = a.quads;
  switch (walker_lanes(q)) {
    case 2: launch_walkers<2, 1, OUT>(a, s); return;
    case 4: launch_walkers<4, 1, OUT>(a, s); return;
    case 8: launch_walkers<8, 1, OUT>(a, s); return;
    case 16: launch_walkers<16, 1, OUT>(a, s); return;
    case 32: launch_walkers<32, 1, OUT>(a, s); return;
    default:  // a whole wavefront: 1, 2, 4 or 8 quads a lane
      if (q <= 64) launch_walkers<64, 1, OUT>(a, s);
      else if (q <= 128) launch_walkers<64, 2, OUT>(a, s);
      else if (q <= 256) launch_walkers<64, 4, OUT>(a, s);
      else launch_walkers<64, 8, OUT>(a, s);
  }
}


}  // namespace
}  // namespace engram
