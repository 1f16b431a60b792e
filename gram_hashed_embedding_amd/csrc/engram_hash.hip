// engram_hash.hip -- n-gram row hash for gfx950.
//
// Computes the global row of every (batch, position, head) as described on
// the NeMo AutoModel v0.7 API page "qwen3_8_flash_next.engram":
// Qwen3_8_FlashNextNGramEmbedding (class description: bigram heads first,
// then trigram, ...; the history is cleared after an EOS; signed int64
// arithmetic that wraps; non-negative remainders; head offsets from the
// checkpoint), _shift_right_after_eos (history never crosses an EOS or a
// packed-segment boundary) and _hash_input_ids (output
// [batch, sequence, ngram_heads]).
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
// Design.  A block covers 64 consecutive tokens of the flattened
// [batch, slice] array at a time (the blocks stride over the array when it
// holds more tokens than one grid's worth: a grid stays within 2^32 work-items).
// Phase 1: one lane per token computes the running
// order mixes M_2..M_n of its token (token_mixes in engram_hash_dev.h: the
// token's whole history loaded at once, then a walk back through it) and
// keeps them in LDS.  Phase 2: the block's 64 * H outputs are one contiguous
// span of the row-id array, so lane i writes output i: the stores are fully
// coalesced.  Each output reduces its order's mix by its head's prime with a
// Barrett step on |mix| (one 64x64 high multiply, one correction) and adds
// the head offset.  The arithmetic is integer-only and tiny next to the 8
// bytes written per output; the kernel is bound by its HBM traffic and
// launch latency.
#include "engram_hash_dev.h"

namespace engram {
namespace {

constexpr int kHashThreads = 256;
constexpr int kHashTokens = 64;

struct HashArgs {
  HashParams p;
  int64_t *rows;         // [batch, local, H]
  int64_t total_tokens;  // batch * local
};

__global__ __launch_bounds__(kHashThreads) void hash_kernel(const HashArgs a) {
  __shared__ uint64_t s_mix[kHashTokens][ENGRAM_MAX_NGRAM - 1];
  __shared__ uint64_t s_prime[ENGRAM_MAX_HEADS];
  __shared__ uint64_t s_magic[ENGRAM_MAX_HEADS];
  __shared__ int64_t s_off[ENGRAM_MAX_HEADS];

  const int tid = threadIdx.x;
  for (int h = tid; h < a.p.H; h += kHashThreads) {
    s_prime[h] = a.p.prime[h];
    s_magic[h] = a.p.magic[h];
    s_off[h] = a.p.offset[h];
  }
  for (int64_t tok0 = (int64_t)blockIdx.x * kHashTokens; tok0 < a.total_tokens;
       tok0 += (int64_t)gridDim.x * kHashTokens) {
    // Phase 1: the order mixes of one token per lane.
    if (tid < kHashTokens && tok0 + tid < a.total_tokens) {
      uint64_t mix[ENGRAM_MAX_NGRAM - 1];
      token_mixes(a.p, tok0 + tid, mix);
#pragma unroll
      for (int k = 0; k < ENGRAM_MAX_NGRAM - 1; ++k)
        if (k < a.p.n - 1) s_mix[tid][k] = mix[k];
    }
    __syncthreads();

    // Phase 2: contiguous, coalesced row-id stores.
    const int64_t ntok = min((int64_t)kHashTokens, a.total_tokens - tok0);
    const int nout = (int)ntok * a.p.H;
    int64_t *out = a.rows + tok0 * a.p.H;
    for (int o = tid; o < nout; o += kHashThreads) {
      const int tl = o / a.p.H;
      const int h = o - tl * a.p.H;
      const int order = h / a.p.J;  // g - 2
      const int64_t x = (int64_t)s_mix[tl][order];
      out[o] = s_off[h] + (int64_t)floor_mod(x, s_prime[h], s_magic[h]);
    }
    __syncthreads();  // s_mix is rewritten for the next tokens
  }
}

}  // namespace
}  // namespace engram

int engram::launch_hash(const HashParams &hp, int64_t tokens, int64_t *d_row_ids,
                        void *stream) {
  const int64_t need = (tokens + kHashTokens - 1) / kHashTokens;
  const int64_t most = kMaxGridItems / kHashThreads;
  const int64_t blocks = need < most ? need : most;
  const HashArgs a = {hp, d_row_ids, tokens};
  hipLaunchKernelGGL(hash_kernel, dim3((unsigned)blocks), dim3(kHashThreads), 0,
                     as_stream(stream), a);
  return launch_status();
}
