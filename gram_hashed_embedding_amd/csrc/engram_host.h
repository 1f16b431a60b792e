// engram_host.h -- the host side of libengram.so in plain C++ (no HIP
// headers): the hash constants, the scatter workspace layout, the argument
// checks every entry point makes, and the launchers the entry points call.
//
// The extern "C" entry points (engram_host.cpp) check their arguments and
// then call one launcher per piece of work.  The launchers live in the HIP
// sources (engram_*.hip); they set up and enqueue kernels and return
// ENGRAM_OK or ENGRAM_EHIP (or ENGRAM_EINVAL for a grid too large to
// launch).  A CPU-only build of the same entry points links stand-ins for
// the launchers, so the checks can run under host sanitizers without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

// Widest row any entry point takes (2^30 values); keeps every byte count of
// a row far from overflow.
constexpr int64_t kMaxDim = int64_t(1) << 30;
// Widest row of the sorted scatter (its walkers hold a row in registers).
constexpr int64_t kMaxSortedDim = 2048;

// a * b <= limit for non-negative a, b, without overflow.
inline bool mul_fits(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work-items of one launch (blocks times threads per block): the dispatch
// packet holds that count in 32 bits, so a grid must stay at or below
// 2^32 - 1 of them.  Every launcher checks its grids with grid_fits before
// enqueuing anything (ENGRAM_EINVAL when one does not fit), or strides its
// blocks over the work so that no size needs more.
constexpr int64_t kMaxGridItems = int64_t(0xFFFFFFFF);
inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= kMaxGridItems / threads;
}

// Number of bits of x (0 for 0).
inline int bit_width_u64(uint64_t x) {
  int b = 0;
  while (x != 0) {
    ++b;
    x >>= 1;
  }
  return b;
}

// ------------------------------------------------------------------ hash ---
// Everything the hash needs, passed by value as kernel arguments (about 1.6 KB).
struct HashParams {
  const int64_t *tokens;  // [batch, stride]
  const int64_t *seg;     // [batch, stride] packed segment ids, or null
  int64_t stride;         // positions per row of tokens / seg
  int64_t start;          // first hashed position of every row
  int64_t local;          // hashed positions per row
  int64_t eos;
  int32_t n;  // ngram_size
  int32_t J;  // heads_per_ngram
  int32_t H;  // (n - 1) * J
  int32_t pad;
  uint64_t mult[ENGRAM_MAX_NGRAM];
  uint64_t prime[ENGRAM_MAX_HEADS];
  uint64_t magic[ENGRAM_MAX_HEADS];  // floor((2^64 - 1) / prime)
  int64_t offset[ENGRAM_MAX_HEADS];
};

// Checks the arguments every hashing entry point shares (positions
// [start, end) of rows of `stride` tokens) and fills *hp; *tokens_out
// receives batch * (end - start).
int make_hash_params(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                     int64_t stride, int64_t start, int64_t end, int32_t ngram_size,
                     int32_t heads_per_ngram, int64_t eos_id, const int64_t *h_multipliers,
                     const int64_t *h_primes, const int64_t *h_offsets, int64_t table_rows,
                     HashParams *hp, int64_t *tokens_out);

// ------------------------------------------------------- scatter layout ---
// Sizes of the sorted scatter, shared by the plan and the apply.
constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per full tile
constexpr int kMaxBins = 256;                         // digits of one sort pass
constexpr int kSlotThreads = 256;                     // ranges per tile of the slot scan
constexpr int kRange = 16;                            // sorted positions per walker
// counters: 4 pass tickets and the slot scan's ticket (8 words), then the
// digit totals, [copy][segment][pass][digit]: kHistCopies copies of one
// segment for a sort of the whole key array, or one copy per segment for a
// sort of per-head segments.
constexpr int kHistCopies = 8;
constexpr int kTicketWords = 8;
constexpr int kSlotTicketAt = 4;
constexpr int kHistSets = kHistCopies > ENGRAM_MAX_HEADS ? kHistCopies : ENGRAM_MAX_HEADS;
constexpr int kSortCounters = kTicketWords + kHistSets * 4 * kMaxBins;

// Long runs: a distinct row whose run of sorted positions starts in one
// 16-position range, covers the whole next range and reaches the one after
// (the runs a range walker leaves out).  The apply sums them chunk by chunk
// (kChunk sorted positions each, aligned), in parallel; a run that crosses
// chunks leaves one fp64 partial-sum row in each chunk it touches, which the
// apply's second launch adds up in chunk order.
constexpr int64_t kChunk = 512;

// The apply's launch: blocks of kWalkThreads threads, the first
// long_blocks(chunks) summing long runs, then the range walkers, one per
// kRange sorted positions, walker_lanes(head_dim / 4) lanes each (one 4-value
// quad of the row per lane, the quad count rounded up to a power of two, at
// most one wavefront).  Long blocks take groups of long_group(chunks)
// consecutive chunks (at most kLongGroup), the groups dealt out to them in
// turn: one chunk each while there are at most kLongBlocks chunks, and never
// more than kLongBlocks of them, so that at any size they share the GPU with
// the walkers from the start.
constexpr int kWalkThreads = 256;
constexpr int kLongGroup = 4;
constexpr int64_t kLongBlocks = 256;
inline int64_t long_blocks(int64_t num_chunks) {
  return num_chunks < kLongBlocks ? num_chunks : kLongBlocks;
}
inline int64_t long_group(int64_t num_chunks) {
  const int64_t nlong = long_blocks(num_chunks);
  const int64_t per = nlong > 0 ? (num_chunks + nlong - 1) / nlong : 1;
  return per < kLongGroup ? per : kLongGroup;
}
inline int64_t walker_lanes(int64_t quads) {
  int64_t l = 2;
  while (l < quads && l < 64) l *= 2;
  return l;
}

// Where the parts of the sorted path's workspace start (bytes, 256-aligned).
struct Plan {
  int64_t num_tiles, num_ranges, slot_tiles;
  int bits, passes, per_pass;
  int64_t status_words;  // look-back words the workspace holds
  int64_t num_chunks;    // kChunk-position chunks of the sorted order
  size_t keys_a, vals_a, keys_b, vals_b, status, counters, head_off, scalars, chunk_owner,
      partials, total;
};

// Blocks of the apply's first launch for a plan of rows head_dim wide.
inline int64_t apply_blocks(const Plan &p, int64_t head_dim) {
  const int64_t walkers = p.num_ranges * walker_lanes(head_dim / 4);
  return long_blocks(p.num_chunks) + (walkers + kWalkThreads - 1) / kWalkThreads;
}

// The plan's scalars at Plan::scalars (the start of the workspace): written
// by the plan, read by the apply.
struct PlanScalars {
  uint32_t unique;      // U, the number of distinct valid rows
  uint32_t stalled;     // non-zero when a wait of the plan expired
  uint64_t n;           // the plan's n and table_rows, written by its last
  uint64_t table_rows;  // kernel; 0 until the plan is complete
  uint64_t pad[5];
};
static_assert(sizeof(PlanScalars) == 64, "the scalars take one 64-byte slot");

// Checks shared by every sorted-scatter mode; fills the workspace layout.
bool make_plan(int64_t n, int64_t table_rows, int64_t dim, Plan *p);

// The sorted path needs 32-bit keys (table_rows itself is the drop key) and
// 32-bit flat indices.
inline bool sorted_limits_ok(int64_t n, int64_t table_rows) {
  return table_rows < (int64_t)UINT32_MAX && n < (int64_t)UINT32_MAX;
}

// What an apply writes for each distinct row r with sum S_r.
constexpr int kOutDense = 0;    // grad_table[r] += fp32(S_r)
constexpr int kOutSparse = 1;   // unique_ids[u] = r, unique_grads[u] = fp32(S_r)
constexpr int kOutSignSGD = 2;  // table[r] = bf16(fp32(table[r]) - lr * sign(fp32(S_r)))

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

// ------------------------------------------------------------ convolution --
constexpr int kConvMaxKernel = 16;

struct ConvCall {
  const void *x, *halo;  // bf16 [batch, seq, channels], [batch, halo_len, channels] or null
  int64_t halo_len;
  const int64_t *seg;    // [batch, halo_len + seq] or null
  const void *weight;    // bf16 [channels, K]
  const void *bias;      // bf16 [channels] or null
  void *out;             // bf16 [batch, seq, channels]
  int64_t batch, seq, channels;
  int32_t K, dilation;
};

// -------------------------------------------------------------- launchers --
// Each enqueues its kernels on `stream` (a hipStream_t) for arguments the
// entry point has checked.
int launch_hash(const HashParams &hp, int64_t tokens, int64_t *d_row_ids, void *stream);
int launch_gather(const int64_t *d_row_ids, int64_t n, const void *d_table, int64_t table_rows,
                  int64_t head_dim, void *d_out, int64_t *d_err_count, void *stream);
int launch_lookup(const HashParams &hp, int64_t n, const void *d_table, int64_t head_dim,
                  void *d_out, int64_t *d_row_ids, void *stream);
// The plan of n ids: given (d_row_ids), or hashed from the tokens (hp, when
// d_row_ids is null).
int launch_plan(const int64_t *d_row_ids, const HashParams *hp, int64_t n, int64_t table_rows,
                const Plan &p, void *d_workspace, int64_t *d_err_count, void *stream);
int launch_apply(const void *d_grads, int64_t n, int64_t head_dim, int64_t table_rows,
                 const Plan &p, void *d_workspace, const ApplyOut &o, int64_t *d_err_count,
                 void *stream);
int launch_scatter_atomic(const int64_t *d_row_ids, int64_t n, const void *d_grads,
                          int64_t head_dim, float *d_grad_table, int64_t table_rows,
                          int64_t *d_err_count, void *stream);
int launch_write_zero(int64_t *d_value, void *stream);
int launch_signsgd(const int64_t *d_unique_ids, const float *d_unique_grads,
                   const int64_t *d_num_unique, int64_t capacity, int64_t head_dim, void *d_table,
                   int64_t table_rows, float lr, int64_t *d_err_count, void *stream);
int launch_ple_conv(const ConvCall &c, void *stream);
// Device address of the current device's copy of the library's fixed
// scratch array (engram_scatter_add_rowsparse_noalloc), or null.
void *static_scratch();
// hipEventRecord(event, stream) and hipStreamWaitEvent(stream, event, 0)
// for engram_run_ops (event non-null).
int record_event(void *event, void *stream);
int wait_event(void *stream, void *event);

}  // namespace engram
