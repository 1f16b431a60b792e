// engram_hash_dev.h -- the n-gram row hash as device code, shared by the
// hash kernel, the fused lookup (hash + gather in one kernel) and the plan
// that sorts row ids it computes from the tokens.
//
// What is computed follows the NeMo AutoModel v0.7 API page
// "qwen3_8_flash_next.engram", Qwen3_8_FlashNextNGramEmbedding: the class
// description (bigram heads first, then trigram, ...; the history is cleared
// after an EOS; signed int64 arithmetic that wraps; non-negative remainders;
// head offsets from the checkpoint), _shift_right_after_eos, _hash_input_ids
// and _forward_global_slice.  Readings where the page is silent: the tokens
// of an order combine by a wrapping sum of token * multiplier; multiplier k
// scales the token k positions back; a position with no valid history token
// reads 0.
#pragma once

#include "engram_internal.h"

namespace engram {

constexpr int64_t kHashFill = 0;  // history token read where none is valid

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

// The order mixes of hashed token f (f = b * local + position in the slice):
// mix[k - 1] is the mix of order k + 1, for k = 1 .. n - 1.  The token's
// whole history (and its segment ids) is loaded at once, positions before
// the row start reading the token itself (never used), so the walk back
// costs one memory round trip; it stops at the row start, at an EOS (which
// closes the segment before the next position) or at a segment change.
// N: the most positions loaded (ngram_size when known at compile time, so
// no register holds a position the order never reads).
template <int N = ENGRAM_MAX_NGRAM>
__device__ __forceinline__ void token_mixes(const HashParams &a, int64_t f,
                                            uint64_t (&mix)[ENGRAM_MAX_NGRAM - 1]) {
  const int64_t b = f / a.local;
  const int64_t t = a.start + (f - b * a.local);  // position inside its row
  const int64_t *tp = a.tokens + b * a.stride + t;
  const int64_t *sp = a.seg != nullptr ? a.seg + b * a.stride + t : nullptr;
  int64_t hist[N], segs[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int64_t back = (k < a.n && t - k >= 0) ? k : 0;
    hist[k] = tp[-back];
    segs[k] = sp != nullptr ? sp[-back] : 0;
  }
  uint64_t m = (uint64_t)hist[0] * a.mult[0];  // wraps modulo 2^64
  bool valid = true;
#pragma unroll
  for (int k = 0; k < ENGRAM_MAX_NGRAM - 1; ++k) mix[k] = 0;
#pragma unroll
  for (int k = 1; k < N; ++k) {
    valid = valid && k < a.n && t - k >= 0 && hist[k] != a.eos && segs[k] == segs[k - 1];
    const int64_t s_k = valid ? hist[k] : kHashFill;
    m += (uint64_t)s_k * a.mult[k];
    mix[k - 1] = m;
  }
}

// Row of one head of a token whose order mixes are known.
__device__ __forceinline__ int64_t head_row(const HashParams &a, const uint64_t mix, int h) {
  return a.offset[h] + (int64_t)floor_mod((int64_t)mix, a.prime[h], a.magic[h]);
}

// Row of flat lookup i = f * H + h of the slice (head h of hashed token f);
// N as for token_mixes.
template <int N = ENGRAM_MAX_NGRAM>
__device__ __forceinline__ int64_t lookup_row(const HashParams &a, int64_t i) {
  const int64_t f = i / a.H;
  const int h = (int)(i - f * a.H);
  uint64_t mix[ENGRAM_MAX_NGRAM - 1];
  token_mixes<N>(a, f, mix);
  const int order = h / a.J;  // g - 2
  uint64_t m = mix[0];
#pragma unroll
  for (int k = 1; k < N - 1; ++k) m = order == k ? mix[k] : m;
  return head_row(a, m, h);
}

}  // namespace engram
