// engram_optim.hip -- row-sparse SignSGD step into the bf16 table, for gfx950.
//
// The prime-rl v0.9.1.dev179 release notes and pull request 3434 (both in
// their Validation sections) train the model with SignSGD (learning rate
// 1e-6) and the default FP32 optimizer math.  The pages give no formula;
// the reading taken here: each row r that the backward touched, with its
// fp32 gradient sum S_r, becomes bf16(fp32(w) - lr * sign(S_r)) element by
// element (subtraction in fp32, sign(0) = 0, one rounding to bf16, nearest
// with ties to even).  Rows not touched keep their values.
//
// Design.  The step reads the row-sparse gradient (ids, fp32 sums and the
// count U, which stays on the device) and updates rows in place: one lane
// per 8 values, i.e. 32 bytes of fp32 gradient and 16 bytes of bf16 table
// read and 16 bytes written, all loads of a lane issued before any is used.
// The grid covers the capacity; lanes past U exit.  The same update is also
// fused into the backward's apply (engram_scatter_apply_signsgd), which
// never writes the fp32 sums at all.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kOptThreads = 256;
constexpr int kOptUnroll = 2;

template <int LOG2_CPR>
__global__ __launch_bounds__(kOptThreads) void signsgd_rowsparse_kernel(
    const int64_t *__restrict__ ids, const f32x4 *__restrict__ grads,
    const int64_t *__restrict__ num_unique, int64_t capacity, int64_t cpr, u32x4 *table,
    int64_t table_rows, float lr, int64_t *err) {
  const int64_t count = min(*num_unique, capacity);
  const int64_t total = count * cpr;
  const int64_t base = (int64_t)blockIdx.x * (kOptThreads * kOptUnroll) + threadIdx.x;
  int64_t r[kOptUnroll], j[kOptUnroll], c[kOptUnroll];
  bool ok[kOptUnroll];
  int bad = 0;
#pragma unroll
  for (int k = 0; k < kOptUnroll; ++k) {
    c[k] = base + (int64_t)k * kOptThreads;
    int64_t u;
    if (LOG2_CPR >= 0) {
      u = c[k] >> LOG2_CPR;
      j[k] = c[k] & ((1 << (LOG2_CPR < 0 ? 0 : LOG2_CPR)) - 1);
    } else {
      u = c[k] / cpr;
      j[k] = c[k] - u * cpr;
    }
    r[k] = c[k] < total ? ids[u] : -1;
    ok[k] = r[k] >= 0 && r[k] < table_rows;
    bad += (c[k] < total && !ok[k] && j[k] == 0 && r[k] != -1) ? 1 : 0;
  }
  u32x4 w[kOptUnroll];
  f32x4 g0[kOptUnroll], g1[kOptUnroll];
#pragma unroll
  for (int k = 0; k < kOptUnroll; ++k) {
    w[k] = ok[k] ? table[r[k] * cpr + j[k]] : u32x4{0u, 0u, 0u, 0u};
    const int64_t gi = ok[k] ? c[k] : 0;
    g0[k] = grads[2 * gi];
    g1[k] = grads[2 * gi + 1];
  }
#pragma unroll
  for (int k = 0; k < kOptUnroll; ++k) {
    if (!ok[k]) continue;
    float f[8];
    unpack_bf16x8(w[k], f);
    const float g[8] = {g0[k].x, g0[k].y, g0[k].z, g0[k].w, g1[k].x, g1[k].y, g1[k].z, g1[k].w};
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = signsgd_bf16(f[e], g[e], lr);
    table[r[k] * cpr + j[k]] =
        u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
  }
  count_errors(bad, err);
}

}  // namespace
}  // namespace engram

int engram::launch_signsgd(const int64_t *d_unique_ids, const float *d_unique_grads,
                           const int64_t *d_num_unique, int64_t capacity, int64_t head_dim,
                           void *d_table, int64_t table_rows, float lr, int64_t *d_err_count,
                           void *stream) {
  const int64_t cpr = head_dim / 8;
  const int64_t per_block = (int64_t)kOptThreads * kOptUnroll;
  const int64_t blocks = (capacity * cpr + per_block - 1) / per_block;
  if (!grid_fits(blocks, kOptThreads)) return ENGRAM_EINVAL;
  const dim3 grid((unsigned)blocks), block(kOptThreads);
  hipStream_t s = as_stream(stream);
  const f32x4 *g = reinterpret_cast<const f32x4 *>(d_unique_grads);
  u32x4 *t = static_cast<u32x4 *>(d_table);
  switch (cpr) {
#define ENGRAM_SGD_CASE(L2)                                                                  \
  case (1 << L2):                                                                            \
    hipLaunchKernelGGL(signsgd_rowsparse_kernel<L2>, grid, block, 0, s, d_unique_ids, g,     \
                       d_num_unique, capacity, cpr, t, table_rows, lr, d_err_count);         \
    break;
    ENGRAM_SGD_CASE(0)
    ENGRAM_SGD_CASE(1)
    ENGRAM_SGD_CASE(2)
    ENGRAM_SGD_CASE(3)
    ENGRAM_SGD_CASE(4)
    ENGRAM_SGD_CASE(5)
    ENGRAM_SGD_CASE(6)
    ENGRAM_SGD_CASE(7)
    ENGRAM_SGD_CASE(8)
#undef ENGRAM_SGD_CASE
    default:
      hipLaunchKernelGGL(signsgd_rowsparse_kernel<-1>, grid, block, 0, s, d_unique_ids, g,
                         d_num_unique, capacity, cpr, t, table_rows, lr, d_err_count);
  }
  return launch_status();
}
