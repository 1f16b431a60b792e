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
// are summed whole by the leading blocks of the same launch, a block per
// run, its walkers taking interleaved ranges of the run and adding their
// sums in a fixed order.  No work item waits on another, and hot rows
// (hundreds of contributions) do not serialise a walker.
#pragma once

#include "engram_scatter_dev.h"

namespace engram {

constexpr int kWalkThreads = 256;
constexpr int64_t kLongBlocks = 1024;  // most blocks that sum long runs
constexpr int64_t kXcds = 8;           // XCDs of an MI355X (blocks go to them in turn)
// Gradient tensors larger than this are read with non-temporal loads: half
// the MI355X's 256 MB Infinity Cache, so a tensor that could still be cached
// when the apply runs is read normally.
constexpr int64_t kStreamGradBytes = int64_t(128) << 20;
constexpr int64_t kLongSpan = 64;      // fewest ranges per long-run block

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
  if constexpr (OUT == kOutSignSGD)
    load_quads<L, Q, EXACT>(a.table, table_row(a, key), a.quads, lane, tw);
  if constexpr (OUT == kOutDense && Q == 1) load_grad_row<L, Q, EXACT>(a, table_row(a, key), lane, tg);
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
  // Only a complete plan of these n and table_rows, none of whose waits
  // expired, is read; otherwise nothing is written (U = 0) and it is counted.
  const PlanScalars *pl = a.plan;
  const bool stalled = pl->stalled != 0;
  if (stalled || pl->n != (uint64_t)a.n || pl->table_rows != (uint64_t)a.sentinel) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (OUT == kOutSparse) *a.num_unique = 0;
      add_mark(a.err, stalled ? kStallMark : kNoPlanMark);
    }
    return;
  }
  if (OUT == kOutSparse && blockIdx.x == 0 && threadIdx.x == 0) *a.num_unique = (int64_t)pl->unique;
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


}  // namespace
}  // namespace engram
