// engram_scatter.hip -- the sorted scatter-add's apply launch, the fp32
// atomic comparison variant, and the fixed scratch array of the
// allocation-free entry point.
//
// The plan (sort and slots) is engram_sort.hip; the apply's kernels are
// engram_apply_dev.h, built once per output form.  The atomic variant adds
// every gradient element to the dense fp32 table with one hardware float
// atomic in L2; the order of additions is not fixed, so it is the comparison
// for the deterministic sorted path, not a replacement.
#include <mutex>

#include "engram_apply_dev.h"

namespace engram {
namespace {

constexpr int kAtomicThreads = 256;
constexpr int kAtomicUnroll = 4;

__global__ void write_zero_kernel(int64_t *p) { *p = 0; }

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

}  // namespace

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

}  // namespace engram

// Apply: the per-row sums of one gradient tensor, given the plan of its ids.
int engram::launch_apply(const void *grads, int64_t n, int64_t dim, int64_t table_rows,
                         const Plan &p, void *ws, const ApplyOut &o, int64_t *err,
                         void *stream) {
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
  a.chunk_owner = v.chunk_owner;
  a.partials = v.partials;
  a.num_chunks = p.num_chunks;
  a.long_blocks = 0;  // set with the grid
  a.long_group = 1;
  a.plan = v.scalars;
  a.num_unique = o.num_unique;
  a.err = err;
  // (the entry points have checked this grid before enqueuing anything)
  if (!grid_fits(apply_blocks(p, dim), kWalkThreads)) return ENGRAM_EINVAL;
  hipStream_t s = as_stream(stream);
  if (o.mode == kOutSparse)
    walk_sparse(a, s);
  else if (o.mode == kOutDense)
    walk_dense(a, s);
  else
    walk_signsgd(a, s);
  return launch_status();
}

int engram::launch_write_zero(int64_t *d_value, void *stream) {
  hipLaunchKernelGGL(write_zero_kernel, dim3(1), dim3(1), 0, as_stream(stream), d_value);
  return launch_status();
}

int engram::launch_scatter_atomic(const int64_t *ids, int64_t n, const void *grads, int64_t dim,
                                  float *grad_table, int64_t table_rows, int64_t *err,
                                  void *stream) {
  hipStream_t s = as_stream(stream);
  const int64_t cpr = dim / 8;
  const int64_t total = n * cpr;
  const int64_t per_block = (int64_t)kAtomicThreads * kAtomicUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  if (!grid_fits(blocks, kAtomicThreads)) return ENGRAM_EINVAL;
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
