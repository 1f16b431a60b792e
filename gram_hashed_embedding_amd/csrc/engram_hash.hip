// engram_hash.hip -- n-gram row hash for gfx950.
//
// Computes the global row of every (batch, position, head) as described on
// the NeMo AutoModel v0.7 API page "qwen3_8_flash_next.engram":
// Qwen3_8_FlashNextNGramEmbedding (class description: bigram heads first,
// then trigram, ...; the history is cleared after an EOS; signed int64
// arithmetic that wraps; non-negative remainders; head offsets from the
// checkpoint),
// _shift_right_after_eos (history never crosses an EOS or a packed-segment
// boundary) and _hash_input_ids (output [batch, sequence, ngram_heads]).
//
// The slice form follows _forward_global_slice on the same page: the
// complete (replicated) sequence is available, and only positions
// [seq_start, seq_end) of every row are hashed, so their history may reach
// back before seq_start (a context-parallel cut keeps the tokens before it
// and the EOS resets at it).
//
// Readings taken where the page is silent: the tokens of an order are
// combined by a wrapping sum of token * multiplier; multiplier k scales the
// token k positions back; a position with no valid history token reads 0.
//
// Design.  One block covers 64 consecutive tokens of the flattened
// [batch, slice] array.  Phase 1: one lane per token loads its last
// ngram_size positions at once (the whole history an n-gram can see, so no
// scan over the sequence is needed) and walks back through them, stopping
// at the row start, an EOS or a segment change; it keeps the running order
// mixes M_2..M_n (a prefix sum, so every order costs one multiply-add) in
// LDS.  Phase 2: the block's 64 * H outputs are one contiguous span of the
// row-id array, so lane i writes output i: the stores are fully coalesced.  Each output reduces its
// order's mix by its head's prime with a Barrett step on |mix| (one 64x64
// high multiply, one correction) and adds the head offset.  The arithmetic
// is integer-only and tiny next to the 8 bytes written per output; the
// kernel is bound by its HBM traffic and launch latency.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kHashThreads = 256;
constexpr int kHashTokens = 64;
constexpr int64_t kFill = 0;  // history token read where none is valid

struct HashArgs {
  const int64_t *tokens;  // [batch, stride]
  const int64_t *seg;     // [batch, stride], may be null
  int64_t *rows;          // [batch, local, H]
  int64_t total_tokens;   // batch * local
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

// Floor remainder of a signed 64-bit x by p in [1, 2^63): Barrett reduction
// of |x| with magic = floor((2^64-1)/p).  The estimate q = hi64(|x| * magic)
// is floor(|x|/p) or one less, so one conditional subtraction finishes it.
__device__ __forceinline__ uint64_t floor_mod(int64_t x, uint64_t p, uint64_t magic) {
  const bool neg = x < 0;
  const uint64_t u = neg ? (uint64_t)0 - (uint64_t)x : (uint64_t)x;
  const uint64_t q = __umul64hi(u, magic);
  uint64_t r = u - q * p;
  if (r >= p) r -= p;
  if (neg && r != 0) r = p - r;
  return r;
}

__global__ __launch_bounds__(kHashThreads) void hash_kernel(const HashArgs a) {
  __shared__ uint64_t s_mix[kHashTokens][ENGRAM_MAX_NGRAM - 1];
  __shared__ uint64_t s_prime[ENGRAM_MAX_HEADS];
  __shared__ uint64_t s_magic[ENGRAM_MAX_HEADS];
  __shared__ int64_t s_off[ENGRAM_MAX_HEADS];

  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * kHashTokens;
  for (int h = tid; h < a.H; h += kHashThreads) {
    s_prime[h] = a.prime[h];
    s_magic[h] = a.magic[h];
    s_off[h] = a.offset[h];
  }

  // Phase 1: the order mixes of one token per lane.  The lane's whole
  // history (and its segment ids) is loaded at once, positions before the
  // row start reading the lane's own token (never used), so the walk back
  // below costs one memory round trip.
  if (tid < kHashTokens && tok0 + tid < a.total_tokens) {
    const int64_t f = tok0 + tid;
    const int64_t b = f / a.local;
    const int64_t t = a.start + (f - b * a.local);  // position inside its row
    const int64_t *tp = a.tokens + b * a.stride + t;
    const int64_t *sp = a.seg != nullptr ? a.seg + b * a.stride + t : nullptr;
    int64_t hist[ENGRAM_MAX_NGRAM], segs[ENGRAM_MAX_NGRAM];
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_NGRAM; ++k) {
      const int64_t back = (k < a.n && t - k >= 0) ? k : 0;
      hist[k] = tp[-back];
      segs[k] = sp != nullptr ? sp[-back] : 0;
    }
    uint64_t mix = (uint64_t)hist[0] * a.mult[0];  // wraps modulo 2^64
    bool valid = true;
#pragma unroll
    for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k) {
      if (k >= a.n) break;
      // Step back from t-k+1 to t-k: stop at the row start, at an EOS
      // (which closes the segment before t-k+1) or at a segment change.
      valid = valid && t - k >= 0 && hist[k] != a.eos && segs[k] == segs[k - 1];
      const int64_t s_k = valid ? hist[k] : kFill;
      mix += (uint64_t)s_k * a.mult[k];
      s_mix[tid][k - 1] = mix;  // mix of order k + 1
    }
  }
  __syncthreads();

  // Phase 2: contiguous, coalesced row-id stores.
  const int64_t ntok = min((int64_t)kHashTokens, a.total_tokens - tok0);
  const int nout = (int)ntok * a.H;
  int64_t *out = a.rows + tok0 * a.H;
  for (int o = tid; o < nout; o += kHashThreads) {
    const int tl = o / a.H;
    const int h = o - tl * a.H;
    const int order = h / a.J;  // g - 2
    const int64_t x = (int64_t)s_mix[tl][order];
    out[o] = s_off[h] + (int64_t)floor_mod(x, s_prime[h], s_magic[h]);
  }
}

}  // namespace
}  // namespace engram

namespace engram {
namespace {

int hash_window(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch, int64_t stride,
                int64_t start, int64_t end, int32_t ngram_size, int32_t heads_per_ngram,
                int64_t eos_id, const int64_t *h_multipliers, const int64_t *h_primes,
                const int64_t *h_offsets, int64_t table_rows, int64_t *d_row_ids,
                void *stream) {
  if (batch < 0 || stride < 0 || table_rows < 0) return ENGRAM_EINVAL;
  if (start < 0 || end < start || end > stride) return ENGRAM_EINVAL;
  if (ngram_size < 2 || ngram_size > ENGRAM_MAX_NGRAM || heads_per_ngram < 1)
    return ENGRAM_EINVAL;
  const int64_t H = (int64_t)(ngram_size - 1) * heads_per_ngram;
  if (H > ENGRAM_MAX_HEADS) return ENGRAM_EINVAL;
  if (h_multipliers == nullptr || h_primes == nullptr || h_offsets == nullptr)
    return ENGRAM_EINVAL;
  if (!mul_fits(batch, stride, INT64_MAX)) return ENGRAM_EINVAL;
  const int64_t local = end - start;
  const int64_t total = batch * local;
  if (!mul_fits(total, H * 8, INT64_MAX)) return ENGRAM_EINVAL;
  if ((total + kHashTokens - 1) / kHashTokens > INT32_MAX) return ENGRAM_EINVAL;

  HashArgs a = {};
  for (int64_t h = 0; h < H; ++h) {
    const int64_t p = h_primes[h], off = h_offsets[h];
    if (p <= 0 || off < 0 || off > table_rows - p) return ENGRAM_EINVAL;
    a.prime[h] = (uint64_t)p;
    a.magic[h] = UINT64_MAX / (uint64_t)p;
    a.offset[h] = off;
  }
  for (int k = 0; k < ngram_size; ++k) a.mult[k] = (uint64_t)h_multipliers[k];
  if (total == 0) return ENGRAM_OK;
  if (d_tokens == nullptr || d_row_ids == nullptr) return ENGRAM_EINVAL;

  a.tokens = d_tokens;
  a.seg = d_seq_ids;
  a.rows = d_row_ids;
  a.total_tokens = total;
  a.stride = stride;
  a.start = start;
  a.local = local;
  a.eos = eos_id;
  a.n = ngram_size;
  a.J = heads_per_ngram;
  a.H = (int32_t)H;
  const unsigned blocks = (unsigned)((total + kHashTokens - 1) / kHashTokens);
  hipLaunchKernelGGL(hash_kernel, dim3(blocks), dim3(kHashThreads), 0, as_stream(stream), a);
  return launch_status();
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" int engram_hash(const int64_t *d_tokens, const int64_t *d_seq_ids, int64_t batch,
                           int64_t seq, int32_t ngram_size, int32_t heads_per_ngram,
                           int64_t eos_id, const int64_t *h_multipliers,
                           const int64_t *h_primes, const int64_t *h_offsets,
                           int64_t table_rows, int64_t *d_row_ids, void *stream) {
  if (seq < 0) return ENGRAM_EINVAL;
  return hash_window(d_tokens, d_seq_ids, batch, seq, 0, seq, ngram_size, heads_per_ngram,
                     eos_id, h_multipliers, h_primes, h_offsets, table_rows, d_row_ids, stream);
}

extern "C" int engram_hash_slice(const int64_t *d_tokens, const int64_t *d_seq_ids,
                                 int64_t batch, int64_t global_seq, int64_t seq_start,
                                 int64_t seq_end, int32_t ngram_size, int32_t heads_per_ngram,
                                 int64_t eos_id, const int64_t *h_multipliers,
                                 const int64_t *h_primes, const int64_t *h_offsets,
                                 int64_t table_rows, int64_t *d_row_ids, void *stream) {
  return hash_window(d_tokens, d_seq_ids, batch, global_seq, seq_start, seq_end, ngram_size,
                     heads_per_ngram, eos_id, h_multipliers, h_primes, h_offsets, table_rows,
                     d_row_ids, stream);
}
