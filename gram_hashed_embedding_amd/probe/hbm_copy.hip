// hbm_copy.hip -- a measurement probe, not part of the C ABI: the
// streaming-copy rate of this GPU's HBM, the practical ceiling beside the
// 8 TB/s the hot path's roofline is quoted against.
//
// One lane moves one 16-byte chunk: a non-temporal load (the source is read
// once) and a non-temporal store (the destination is not read again), 256
// lanes per block and as many blocks as chunks / 256.  On MI355X this shape
// measured fastest among 1, 2, 4 and 8 chunks per lane, plain or
// non-temporal loads and stores, and grid-stride loops of 1024 to 8192 blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4 *__restrict__ src,
                                                          u32x4 *__restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

}  // namespace

// Copy n16 16-byte chunks from src to dst (device pointers, 16-byte aligned)
// on `stream`.  Returns 0, or -1 for arguments it cannot launch.
extern "C" int engram_probe_stream_copy(const void *src, void *dst, int64_t n16, void *stream) {
  if (n16 <= 0 || src == nullptr || dst == nullptr) return -1;
  const int64_t blocks = (n16 + 255) / 256;
  if (blocks > INT32_MAX) return -1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                     static_cast<u32x4 *>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
