// engram_conv.hip -- the PLE causal dilated depthwise convolution with
// per-segment zero history, for gfx950.
//
// What is computed follows the NeMo AutoModel v0.7 API page
// "qwen3_8_flash_next.engram", Qwen3_8_FlashNextPLELayer: _causal_short_conv
// (a causal depthwise convolution over [batch, sequence, channels], zeros as
// the history on the left; under context parallelism the preceding
// (K - 1) * dilation positions come from the previous rank), _segmented_conv
// (each packed segment is convolved as if it began a row, so no tap reads
// another segment), conv_kernel_size (4) and short_conv_dilation
// (= ngram_size).  Readings where the page is silent: the taps follow
// F.conv1d, out[t, c] = bias[c] + sum_k w[c, k] * x[t - (K-1-k) * d, c]; a
// tap before the row start (after the halo, if one is given) or across a
// change of segment id reads 0; bf16 data, the sum accumulated in fp32
// from the bias in tap order, rounded once to bf16 (nearest, ties to even).
//
// Design (K = 4, dilation 1..8).  Bound by HBM: every input is read once
// and every output written once.  A lane owns 4 channels (8 bytes of a
// row: a wavefront covers 256 channels, whole 128-byte lines) and kT = 24
// consecutive positions of one batch row; it loads the 24 + (K-1) * d rows
// of its window at once (clamped addresses, so no load waits behind a
// branch), then computes its 24 outputs from registers and writes them
// with non-temporal stores (the output is not read again here).  The window's
// segment ids are turned into "run start" positions by one wavefront (a
// ballot of the positions where the id changes, then the highest change at
// or before each position) and shared through LDS.  The history rows of a
// tile are the last rows of the tile before it; blocks are numbered so that
// the tiles one XCD runs are consecutive, so those rows are usually still
// in that XCD's L2.  Other kernel sizes and dilations take a plain kernel
// that reads its taps straight from memory.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvQuads = kConvThreads;  // channel quads per block (1024 channels)
constexpr int kT = 24;                    // positions per lane
constexpr int kXcds = 8;                  // XCDs of an MI355X (blocks go round-robin)

struct ConvArgs {
  const uint2 *x;     // [batch, seq, quads]
  const uint2 *halo;  // [batch, halo_len, quads] or null
  const int64_t *seg; // [batch, halo_len + seq] or null
  const uint2 *w;     // [channels, K] bf16, as raw 16-bit words
  const uint16_t *bias;
  uint2 *out;         // [batch, seq, quads]
  int64_t batch, seq, quads, halo_len;
  int32_t K, dil;
  int64_t tiles, groups;  // position tiles per row, channel-quad groups
};

// A position's row of this lane's 4 channels: the halo for p in
// [-halo_len, 0), x for p in [0, seq); anything else reads a valid address
// whose value is never used.
__device__ __forceinline__ const uint2 *row_ptr(const ConvArgs &a, int64_t b, int64_t p,
                                                int64_t qd) {
  if (p >= 0) return a.x + (b * a.seq + min(p, a.seq - 1)) * a.quads + qd;
  if (p >= -a.halo_len) return a.halo + (b * a.halo_len + a.halo_len + p) * a.quads + qd;
  return a.x + b * a.seq * a.quads + qd;
}

// Block -> (batch, group, tile), tiles fastest, numbered so that the blocks
// one XCD receives (every kXcds-th) run consecutive tiles.
__device__ __forceinline__ int64_t logical_block(int64_t n) {
  const int64_t lin = blockIdx.x, x = lin % kXcds, i = lin / kXcds;
  const int64_t q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + i;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <int D>
__global__ __launch_bounds__(kConvThreads) void ple_conv_k4_kernel(const ConvArgs a) {
  constexpr int K = 4;
  constexpr int H = (K - 1) * D;  // history rows
  constexpr int W = kT + H;       // window rows
  static_assert(W <= kWave, "one wavefront covers the window's segment ids");
  __shared__ int64_t s_start[W];  // run start of each window position
  const int64_t lb = logical_block(a.batch * a.groups * a.tiles);
  const int64_t tile = lb % a.tiles, rest = lb / a.tiles;
  const int64_t grp = rest % a.groups, b = rest / a.groups;
  const int64_t t0 = tile * kT;
  const int64_t qd = grp * kConvQuads + threadIdx.x;
  const bool lane_on = qd < a.quads;
  const int64_t qq = lane_on ? qd : 0;

  // the window's rows: positions t0 - H .. t0 + kT - 1
  uint2 v[W];
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = *row_ptr(a, b, t0 - H + i, qq);
  // weights (4 channels x K taps, bf16) and bias
  float wf[4][K], bias[4];
  {
    const uint16_t *wp = reinterpret_cast<const uint16_t *>(a.w) + qq * 4 * K;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int k = 0; k < K; ++k) wf[c][k] = bf16_bits_to_f32(wp[c * K + k]);
      bias[c] = a.bias != nullptr ? bf16_bits_to_f32(a.bias[qq * 4 + c]) : 0.0f;
    }
  }
  // run starts: a position starts a run at the row start or where the
  // segment id changes; positions before the row start get a start past
  // every tap so they read zero
  if (threadIdx.x < kWave) {
    const int i = threadIdx.x;
    const int64_t p = t0 - H + i;
    bool change = false;
    if (i < W && p >= -a.halo_len) {
      change = p == -a.halo_len;
      if (!change && a.seg != nullptr) {
        const int64_t *sr = a.seg + b * (a.halo_len + a.seq) + a.halo_len;
        change = p < a.seq && sr[p] != sr[p - 1];
      }
    }
    const unsigned long long m = __ballot(change) & ((2ull << i) - 1ull);
    int64_t start;
    if (p < -a.halo_len) start = INT64_MAX;                       // before the row
    else if (m != 0ull) start = t0 - H + (63 - __builtin_clzll(m));  // latest change
    else start = INT64_MIN;                                        // run began earlier
    if (i < W) s_start[i] = start;
  }
  __syncthreads();
  if (!lane_on) return;

#pragma unroll
  for (int tt = 0; tt < kT; ++tt) {
    const int64_t t = t0 + tt;
    if (t >= a.seq) break;
    const int64_t run = s_start[H + tt];
    float acc[4] = {bias[0], bias[1], bias[2], bias[3]};
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int wi = tt + k * D;  // window index of position t - (K-1-k) * D
      const bool ok = t0 - H + wi >= run && t0 - H + wi >= -a.halo_len;
      const uint2 r = v[wi];
      acc[0] += wf[0][k] * (ok ? bf16_lo(r.x) : 0.0f);
      acc[1] += wf[1][k] * (ok ? bf16_hi(r.x) : 0.0f);
      acc[2] += wf[2][k] * (ok ? bf16_lo(r.y) : 0.0f);
      acc[3] += wf[3][k] * (ok ? bf16_hi(r.y) : 0.0f);
    }
    const uint32_t o0 = bf16_bits_rne(acc[0]), o1 = bf16_bits_rne(acc[1]);
    const uint32_t o2 = bf16_bits_rne(acc[2]), o3 = bf16_bits_rne(acc[3]);
    __builtin_nontemporal_store(u32x2{o0 | (o1 << 16), o2 | (o3 << 16)},
                                reinterpret_cast<u32x2 *>(a.out + (b * a.seq + t) * a.quads + qd));
  }
}

// Any K <= kConvMaxKernel and dilation: one lane per (position, channel quad),
// each tap read from memory and checked against the segment ids directly.
__global__ __launch_bounds__(kConvThreads) void ple_conv_generic_kernel(const ConvArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (i >= a.batch * a.seq * a.quads) return;
  const int64_t qd = i % a.quads, bt = i / a.quads;
  const int64_t t = bt % a.seq, b = bt / a.seq;
  const uint16_t *wp = reinterpret_cast<const uint16_t *>(a.w) + qd * 4 * a.K;
  const int64_t *sr = a.seg != nullptr ? a.seg + b * (a.halo_len + a.seq) + a.halo_len : nullptr;
  float acc[4];
  for (int c = 0; c < 4; ++c)
    acc[c] = a.bias != nullptr ? bf16_bits_to_f32(a.bias[qd * 4 + c]) : 0.0f;
  for (int k = 0; k < a.K; ++k) {
    const int64_t p = t - (int64_t)(a.K - 1 - k) * a.dil;
    bool ok = p >= -a.halo_len;
    for (int64_t j = p; ok && sr != nullptr && j < t; ++j) ok = sr[j] == sr[j + 1];
    const uint2 r = ok ? *row_ptr(a, b, p, qd) : uint2{0u, 0u};
    acc[0] += bf16_bits_to_f32(wp[0 * a.K + k]) * (ok ? bf16_lo(r.x) : 0.0f);
    acc[1] += bf16_bits_to_f32(wp[1 * a.K + k]) * (ok ? bf16_hi(r.x) : 0.0f);
    acc[2] += bf16_bits_to_f32(wp[2 * a.K + k]) * (ok ? bf16_lo(r.y) : 0.0f);
    acc[3] += bf16_bits_to_f32(wp[3 * a.K + k]) * (ok ? bf16_hi(r.y) : 0.0f);
  }
  a.out[bt * a.quads + qd] = uint2{bf16_bits_rne(acc[0]) | (bf16_bits_rne(acc[1]) << 16),
                                   bf16_bits_rne(acc[2]) | (bf16_bits_rne(acc[3]) << 16)};
}

}  // namespace
}  // namespace engram

int engram::launch_ple_conv(const ConvCall &c, void *stream) {
  ConvArgs a = {};
  a.x = static_cast<const uint2 *>(c.x);
  a.halo = static_cast<const uint2 *>(c.halo);
  a.seg = c.seg;
  a.w = static_cast<const uint2 *>(c.weight);
  a.bias = static_cast<const uint16_t *>(c.bias);
  a.out = static_cast<uint2 *>(c.out);
  a.batch = c.batch;
  a.seq = c.seq;
  a.quads = c.channels / 4;
  a.halo_len = c.halo_len;
  a.K = c.K;
  a.dil = c.dilation;
  a.tiles = (c.seq + kT - 1) / kT;
  a.groups = (a.quads + kConvQuads - 1) / kConvQuads;
  hipStream_t s = as_stream(stream);
  const int64_t blocks = c.batch * a.groups * a.tiles;
  if (c.K == 4 && c.dilation <= 8) {
    if (!grid_fits(blocks, kConvThreads)) return ENGRAM_EINVAL;
    const dim3 grid((unsigned)blocks), block(kConvThreads);
    switch (c.dilation) {
#define ENGRAM_CONV_CASE(D) \
  case D: hipLaunchKernelGGL(ple_conv_k4_kernel<D>, grid, block, 0, s, a); break;
      ENGRAM_CONV_CASE(1)
      ENGRAM_CONV_CASE(2)
      ENGRAM_CONV_CASE(3)
      ENGRAM_CONV_CASE(4)
      ENGRAM_CONV_CASE(5)
      ENGRAM_CONV_CASE(6)
      ENGRAM_CONV_CASE(7)
      ENGRAM_CONV_CASE(8)
#undef ENGRAM_CONV_CASE
    }
  } else {
    const int64_t n = c.batch * c.seq * a.quads;
    const int64_t gb = (n + kConvThreads - 1) / kConvThreads;
    if (!grid_fits(gb, kConvThreads)) return ENGRAM_EINVAL;
    hipLaunchKernelGGL(ple_conv_generic_kernel, dim3((unsigned)gb), dim3(kConvThreads), 0, s, a);
  }
  return launch_status();
}
