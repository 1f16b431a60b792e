"""Seeded synthetic workloads for the hashed n-gram embedding.

This module only draws inputs: token batches, packed-segment IDs, hash
constants (multipliers, primes, cumulative head offsets) and the recipes for
the bf16 table and upstream gradients.  It performs none of the method's
arithmetic (no hashing, lookup or accumulation), so both the HIP path and
the CPU oracle can take their inputs from here.

Token IDs follow the released vocabulary width of 151936 ids; id 0 is kept
for EOS in every workload, so Zipf-distributed ids are ranks 1..151935.

The five workloads:

=========  ==========  =====  =========================================  =====  ==========
name       tokens      n, J   primes (offsets cumulative) -> table rows  dim    notes
=========  ==========  =====  =========================================  =====  ==========
tiny       [2, 128]    3, 2   1009, 1013, 1019, 1021 -> 4062             32     uniform ids
medium     [4, 4096]   3, 8   first 16 primes above 2^20 -> 16,778,782   64     forward only
full       [1, 32768]  3, 16  largest 32 primes <= 6.25M -> 200M rows    256    packed docs
backward   [4, 4096]   3, 8   as medium                                  64     dense fp32 grads
e2e        [8, 8192]   4, 8   largest 24 primes <= 8,333,333 -> 200M     256    row-sparse
=========  ==========  =====  =========================================  =====  ==========
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

VOCAB = 151936
EOS_ID = 0
# the pad token of the pad-tail workload: the last id of the vocabulary (the
# rarest Zipf rank, so real tokens almost never equal it)
PAD_ID = VOCAB - 1

# Constants printed on the NeMo AutoModel API page
# "nemo_automodel.components.models.qwen3_8_flash_next.engram", section Data.
PAGE_LAYER_MULTIPLIERS = (23703573157769, 20109073645365, 8052911324071)
PAGE_HEAD_VOCAB_SIZES_PRINTED = (20000003, 20000023, 20000033, 20000047,
                                 20000059, 20000063, 20000069, 20000077)
PAGE_HEAD_OFFSETS_PRINTED = (0, 20000003, 40000026, 60000059, 80000106,
                             100000165, 120000228, 140000297)
PAGE_PADDED_ROWS = 320001536


# ---------------------------------------------------------------------------
# primes (configuration only)
# ---------------------------------------------------------------------------
def is_prime(n: int) -> bool:
    """Deterministic Miller-Rabin for n < 3.3e24 (fixed witness set)."""
    if n < 2:
        return False
    small = (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41)
    for p in small:
        if n % p == 0:
            return n == p
    d, s = n - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    for a in small:
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(s - 1):
            x = pow(x, 2, n)
            if x == n - 1:
                break
        else:
            return False
    return True


def primes_above(lo: int, count: int) -> list[int]:
    """The first `count` primes strictly greater than `lo`."""
    out, x = [], lo + 1
    while len(out) < count:
        if is_prime(x):
            out.append(x)
        x += 1
    return out


def primes_at_most(hi: int, count: int) -> list[int]:
    """The largest `count` primes <= `hi`, ascending."""
    out, x = [], hi
    while len(out) < count:
        if is_prime(x):
            out.append(x)
        x -= 1
    return sorted(out)


def cumulative_offsets(primes) -> list[int]:
    """Head offsets packed back to back: offset[h] = sum of primes[:h]."""
    out, acc = [], 0
    for p in primes:
        out.append(acc)
        acc += p
    return out


def seeded_multipliers(ngram_size: int, seed: int) -> np.ndarray:
    """Full-range int64 multipliers, forced odd, signs mixed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max,
                     size=ngram_size, dtype=np.int64, endpoint=True)
    return m | np.int64(1)


# ---------------------------------------------------------------------------
# tokens
# ---------------------------------------------------------------------------
def uniform_tokens(rng, shape, lo, hi):
    return rng.integers(lo, hi, size=shape, dtype=np.int64)


def zipf_tokens(rng, shape, s, vocab=VOCAB):
    """Ranks 1..vocab-1 with P(r) proportional to r^-s, by inverse CDF."""
    ranks = np.arange(1, vocab, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    u = rng.random(size=int(np.prod(shape)))
    idx = np.searchsorted(cdf, u, side="right")
    idx = np.minimum(idx, vocab - 2)
    return (idx + 1).astype(np.int64).reshape(shape)


def insert_eos(rng, tokens, prob, eos_id=EOS_ID):
    """Overwrite each position independently with EOS with probability prob."""
    mask = rng.random(size=tokens.shape) < prob
    out = tokens.copy()
    out[mask] = eos_id
    return out


def packed_documents(rng, batch, seq, zipf_s, mean_len=2048.0, sigma=1.0,
                     eos_id=EOS_ID):
    """Rows of packed documents: lengths round(LogNormal(ln(mean) - sigma^2/2,
    sigma)) (so the mean is `mean_len`), at least 1; each complete document
    ends with EOS; the last document of a row is cut at the row end.
    Returns (tokens [batch, seq], segment ids [batch, seq] = document index)."""
    tokens = zipf_tokens(rng, (batch, seq), zipf_s)
    seg = np.empty((batch, seq), dtype=np.int64)
    mu = math.log(mean_len) - 0.5 * sigma * sigma
    for b in range(batch):
        pos, doc = 0, 0
        while pos < seq:
            length = max(1, int(round(rng.lognormal(mu, sigma))))
            end = min(seq, pos + length)
            seg[b, pos:end] = doc
            if pos + length <= seq:
                tokens[b, end - 1] = eos_id
            pos, doc = end, doc + 1
    return tokens, seg


def packed_with_pad_tail(rng, batch, seq, zipf_s, mean_len=2048.0, sigma=1.0,
                         eos_id=EOS_ID, pad_id=PAD_ID):
    """Rows of packed documents as packed_documents draws them, except that a
    row holds only whole documents: the rest of the row after the last one
    that fits is padding, pad_id tokens in a segment of their own.  Returns
    (tokens, segment ids)."""
    tokens = zipf_tokens(rng, (batch, seq), zipf_s)
    seg = np.empty((batch, seq), dtype=np.int64)
    mu = math.log(mean_len) - 0.5 * sigma * sigma
    for b in range(batch):
        pos, doc = 0, 0
        while True:
            length = max(1, int(round(rng.lognormal(mu, sigma))))
            if pos + length > seq:
                break
            seg[b, pos:pos + length] = doc
            tokens[b, pos + length - 1] = eos_id
            pos, doc = pos + length, doc + 1
        tokens[b, pos:] = pad_id
        seg[b, pos:] = doc
    return tokens, seg


def random_segments(shape, mean_length, seed):
    """Packed segment ids: each position starts a new segment with
    probability 1/mean_length (ids are running counts along each row)."""
    rng = np.random.Generator(np.random.PCG64([seed, 99]))
    starts = rng.random(size=shape) < 1.0 / mean_length
    return np.cumsum(starts, axis=-1).astype(np.int64)


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    ngram_size: int
    heads_per_ngram: int
    primes: tuple
    table_rows: int
    dim: int
    seed: int
    token_kind: str            # "uniform" | "zipf" | "packed" | "packed_pad"
    token_lo: int = 0
    token_hi: int = VOCAB
    zipf_s: float = 1.1
    eos_prob: float = 0.0
    eos_id: int = EOS_ID
    table_std: float = 0.02
    grads: str = "none"        # "none" | "dense" | "rowsparse"

    @property
    def heads(self) -> int:
        return (self.ngram_size - 1) * self.heads_per_ngram

    @property
    def offsets(self) -> tuple:
        return tuple(cumulative_offsets(self.primes))

    @property
    def tokens_per_batch(self) -> int:
        return self.batch * self.seq

    @property
    def lookups(self) -> int:
        return self.batch * self.seq * self.heads

    def multipliers(self, variant: int = 0) -> np.ndarray:
        return seeded_multipliers(self.ngram_size, self.seed * 1000 + 7 + variant)

    def tokens(self, variant: int = 0, with_segments: bool = False):
        """Token batch number `variant` (0, 1, ...), and segment IDs when
        requested (packed workloads; None otherwise)."""
        rng = np.random.Generator(np.random.PCG64([self.seed, variant]))
        shape = (self.batch, self.seq)
        seg = None
        if self.token_kind == "uniform":
            tok = uniform_tokens(rng, shape, self.token_lo, self.token_hi)
        elif self.token_kind == "zipf":
            tok = zipf_tokens(rng, shape, self.zipf_s)
        elif self.token_kind == "packed":
            tok, seg = packed_documents(rng, self.batch, self.seq, self.zipf_s)
        elif self.token_kind == "packed_pad":
            tok, seg = packed_with_pad_tail(rng, self.batch, self.seq, self.zipf_s)
        else:
            raise ValueError(self.token_kind)
        if self.eos_prob > 0:
            tok = insert_eos(rng, tok, self.eos_prob, self.eos_id)
        return (tok, seg) if with_segments else tok

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "seq": self.seq,
                "ngram_size": self.ngram_size,
                "heads_per_ngram": self.heads_per_ngram, "heads": self.heads,
                "table_rows": self.table_rows, "head_dim": self.dim,
                "lookups": self.lookups, "seed": self.seed}


def _padded(total: int, to: int) -> int:
    return ((total + to - 1) // to) * to


def tiny() -> Workload:
    primes = (1009, 1013, 1019, 1021)
    return Workload("tiny", 2, 128, 3, 2, primes, sum(primes), 32, 1001,
                    "uniform", token_lo=1, token_hi=1000, eos_prob=1 / 64,
                    grads="dense")


def medium() -> Workload:
    primes = tuple(primes_above(1 << 20, 16))
    return Workload("medium", 4, 4096, 3, 8, primes, sum(primes), 64, 1002,
                    "uniform", token_lo=0, token_hi=VOCAB, eos_prob=1 / 2048)


def full() -> Workload:
    primes = tuple(primes_at_most(6_250_000, 32))
    return Workload("full", 1, 32768, 3, 16, primes, 200_000_000, 256, 1003,
                    "packed", zipf_s=1.1)


def backward() -> Workload:
    primes = tuple(primes_above(1 << 20, 16))
    return Workload("backward", 4, 4096, 3, 8, primes, sum(primes), 64, 1004,
                    "zipf", zipf_s=1.2, eos_prob=1 / 2048, grads="dense")


def e2e() -> Workload:
    primes = tuple(primes_at_most(8_333_333, 24))
    return Workload("e2e", 8, 8192, 4, 8, primes, 200_000_000, 256, 1005,
                    "zipf", zipf_s=1.1, eos_prob=1 / 4096, grads="rowsparse")


def e2e_padtail() -> Workload:
    """The e2e shape with packs that end in a pad-token tail of their own
    segment (the layer gives the tail padding its own sequence id): every
    head then hashes the tail's tokens into one row, runs of thousands of
    terms."""
    primes = tuple(primes_at_most(8_333_333, 24))
    return Workload("e2e_padtail", 8, 8192, 4, 8, primes, 200_000_000, 256, 1006,
                    "packed_pad", zipf_s=1.1, grads="rowsparse")


WORKLOADS = {"tiny": tiny, "medium": medium, "full": full,
             "backward": backward, "e2e": e2e, "e2e_padtail": e2e_padtail}


def get(name: str) -> Workload:
    return WORKLOADS[name]()


# ---------------------------------------------------------------------------
# device tensors (torch is imported lazily: the CPU-only paths need numpy)
# ---------------------------------------------------------------------------
def make_table(rows: int, dim: int, seed: int, device, std: float = 0.02,
               chunk_rows: int = 1 << 22):
    """bf16 table [rows, dim] ~ N(0, std), filled in row chunks from one
    seeded torch generator on `device`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    table = torch.empty((rows, dim), dtype=torch.bfloat16, device=device)
    for start in range(0, rows, chunk_rows):
        table[start:start + chunk_rows].normal_(0.0, std, generator=gen)
    return table


def make_grads(n: int, dim: int, seed: int, device, chunk_rows: int = 1 << 20):
    """Upstream gradients bf16 [n, dim] ~ N(0, 1)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    g = torch.empty((n, dim), dtype=torch.bfloat16, device=device)
    for start in range(0, n, chunk_rows):
        g[start:start + chunk_rows].normal_(0.0, 1.0, generator=gen)
    return g


def make_grad_table(rows: int, dim: int, seed: Optional[int], device,
                    chunk_rows: int = 1 << 22):
    """fp32 gradient table: zeros when seed is None, else N(0, 1)."""
    import torch
    if seed is None:
        return torch.zeros((rows, dim), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.empty((rows, dim), dtype=torch.float32, device=device)
    for start in range(0, rows, chunk_rows):
        t[start:start + chunk_rows].normal_(0.0, 1.0, generator=gen)
    return t


# ---------------------------------------------------------------------------
# the PLE convolution's workload
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    """Inputs of the causal depthwise PLE convolution.  The pages print no
    model widths: channels = hc_count * hidden_size is taken as 4 * 2048, a
    stand-in; kernel 4 and dilation = ngram_size follow the API page (the
    e2e workload's ngram_size is 4).  Rows are packed documents as in the
    full-scale workload (segment ids = document index)."""
    name: str
    batch: int
    seq: int
    channels: int
    kernel_size: int
    dilation: int
    seed: int

    @property
    def history(self) -> int:
        return (self.kernel_size - 1) * self.dilation

    def segments(self, variant: int = 0, halo: int = 0) -> np.ndarray:
        """Segment ids int64 [batch, halo + seq]."""
        rng = np.random.Generator(np.random.PCG64([self.seed, 77, variant]))
        _, seg = packed_documents(rng, self.batch, halo + self.seq, 1.1)
        return seg

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "seq": self.seq,
                "channels": self.channels, "kernel_size": self.kernel_size,
                "dilation": self.dilation, "seed": self.seed}


def ple_conv() -> ConvWorkload:
    return ConvWorkload("ple_conv", batch=8, seq=8192, channels=8192, kernel_size=4,
                        dilation=4, seed=1006)


def make_bf16(shape, seed: int, device, std: float = 1.0):
    """bf16 tensor of the given shape ~ N(0, std), from a seeded generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = t.view(-1)
    step = 1 << 26
    for start in range(0, flat.numel(), step):
        flat[start:start + step].normal_(0.0, std, generator=gen)
    return t
