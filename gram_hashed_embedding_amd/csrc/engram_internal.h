// engram_internal.h -- device helpers shared by the HIP translation units of
// libengram.so.  Not part of the public ABI (that is include/engram.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram_host.h"

namespace engram {

// 16-byte vector of four 32-bit words: eight bf16 values, or four fp32.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // four bf16 values

constexpr int kWave = 64;  // CDNA wavefront width

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Status of the launches just enqueued on this thread.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

// bf16 element e (0..7) of a 16-byte chunk, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack_bf16x8(const u32x4 &v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// fp32 -> bf16 bits, rounded to nearest with ties to even (a NaN stays a
// quiet NaN): add just under half of the dropped low half, plus one when the
// kept half is odd, and keep the high half.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One SignSGD element in fp32: w - lr * sign(g), sign(0) = 0, as bf16 bits.
__device__ __forceinline__ uint32_t signsgd_bf16(float w, float g, float lr) {
  const float s = g > 0.0f ? 1.0f : (g < 0.0f ? -1.0f : 0.0f);
  return bf16_bits_rne(w - lr * s);
}

// Add a lane's count of invalid ids to *err (when err is not null).  Invalid
// ids are rare, so one atomic per lane that saw any is cheap.
__device__ __forceinline__ void count_errors(int bad, int64_t *err) {
  if (err != nullptr && bad != 0)
    atomicAdd(reinterpret_cast<unsigned long long *>(err), (unsigned long long)bad);
}

}  // namespace engram
