// engram_scatter_dev.h -- the sorted scatter's workspace as seen from the
// device code: the views the plan (engram_sort.hip) writes and the apply
// (engram_apply_*.hip) reads, and the marks both add to the error counter.
#pragma once

#include "engram_internal.h"

namespace engram {

// Added to *err when a bounded wait of the plan expires (its results are
// then not valid), and when an apply finds no complete plan of its n and
// table_rows in the workspace (it then writes nothing; U = 0).
constexpr int64_t kStallMark = int64_t(1) << 40;
constexpr int64_t kNoPlanMark = int64_t(1) << 41;
static_assert(kStallMark == ENGRAM_ERR_STALLED && kNoPlanMark == ENGRAM_ERR_NO_PLAN,
              "the marks the header documents");

// Workspace views shared by the plan and the apply.
struct Views {
  uint32_t *keys_a, *vals_a, *keys_b, *vals_b;
  uint64_t *status;
  uint32_t *counters, *head_off;
  PlanScalars *scalars;
  uint32_t *chunk_owner;  // the apply's: long runs that leave each chunk
  double *partials;       // the apply's: partial-sum rows of long runs
  const uint32_t *sorted_keys, *sorted_vals;  // where the last sort pass leaves them
};

inline Views views_of(const Plan &p, void *ws) {
  char *base = static_cast<char *>(ws);
  Views v;
  v.keys_a = reinterpret_cast<uint32_t *>(base + p.keys_a);
  v.vals_a = reinterpret_cast<uint32_t *>(base + p.vals_a);
  v.keys_b = reinterpret_cast<uint32_t *>(base + p.keys_b);
  v.vals_b = reinterpret_cast<uint32_t *>(base + p.vals_b);
  v.status = reinterpret_cast<uint64_t *>(base + p.status);
  v.counters = reinterpret_cast<uint32_t *>(base + p.counters);
  v.head_off = reinterpret_cast<uint32_t *>(base + p.head_off);
  v.scalars = reinterpret_cast<PlanScalars *>(base + p.scalars);
  v.chunk_owner = reinterpret_cast<uint32_t *>(base + p.chunk_owner);
  v.partials = reinterpret_cast<double *>(base + p.partials);
  // passes alternate a -> b -> a ...: an odd pass count ends in a
  v.sorted_keys = (p.passes % 2 == 1) ? v.keys_a : v.keys_b;
  v.sorted_vals = (p.passes % 2 == 1) ? v.vals_a : v.vals_b;
  return v;
}

// Add `mark` to *err once (when err is not null).
__device__ __forceinline__ void add_mark(int64_t *err, int64_t mark) {
  if (err != nullptr)
    atomicAdd(reinterpret_cast<unsigned long long *>(err), (unsigned long long)mark);
}

}  // namespace engram
