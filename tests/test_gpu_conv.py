"""GPU parity of the PLE causal dilated depthwise convolution
(engram_ple_conv) against the oracle: bit-exact bf16 outputs."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")


def inputs(B, S, C, K, seed, halo_len=0, seg_mean=None):
    x = workloads.make_bf16((B, S, C), seed, "cuda")
    w = workloads.make_bf16((C, K), seed + 1, "cuda", std=0.5)
    bias = workloads.make_bf16((C,), seed + 2, "cuda", std=0.5)
    halo = workloads.make_bf16((B, halo_len, C), seed + 3, "cuda") if halo_len else None
    seg = None
    if seg_mean:
        seg = workloads.random_segments((B, halo_len + S), seg_mean, seed)
    return x, w, bias, halo, seg


def check(oracle, B, S, C, K, d, seed, halo_len=0, seg_mean=None, with_bias=True):
    x, w, bias, halo, seg = inputs(B, S, C, K, seed, halo_len, seg_mean)
    b = bias if with_bias else None
    got = E.engram_ple_conv(x, w, d, bias=b, seq_ids=None if seg is None else dev(seg),
                            halo=halo)
    torch.cuda.synchronize()
    want = oracle.ple_conv(bits(x), bits(w), d, None if b is None else bits(b), seg,
                           None if halo is None else bits(halo))
    assert np.array_equal(bits(got), want), (B, S, C, K, d, halo_len, seg_mean)


@pytest.mark.parametrize("d", range(1, 9))
@pytest.mark.parametrize("seg_mean", [None, 3, 40])
def test_kernel4_every_dilation(oracle, d, seg_mean):
    check(oracle, 2, 77, 48, 4, d, 10 * d, seg_mean=seg_mean)


@pytest.mark.parametrize("S", [1, 15, 16, 17, 100, 257])
@pytest.mark.parametrize("C", [8, 24, 1024, 1032, 2056])
def test_shapes(oracle, S, C):
    """Ragged sequence tiles and channel groups (1024 channels per block)."""
    check(oracle, 2, S, C, 4, 3, S * 7 + C, seg_mean=20)


@pytest.mark.parametrize("halo_len,seg_mean", [(9, None), (9, 5), (12, 4), (3, 7), (1, None)])
def test_halo(oracle, halo_len, seg_mean):
    """The context-parallel form: the preceding positions as a halo."""
    check(oracle, 2, 50, 40, 4, 3, 300 + halo_len, halo_len=halo_len, seg_mean=seg_mean)


def test_no_bias(oracle):
    check(oracle, 3, 40, 16, 4, 4, 5, seg_mean=6, with_bias=False)


@pytest.mark.parametrize("K,d", [(1, 1), (3, 2), (5, 3), (4, 9), (2, 12), (16, 1)])
def test_other_kernel_sizes(oracle, K, d):
    """Shapes the tiled kernel does not take (the plain kernel runs)."""
    check(oracle, 2, 60, 16, K, d, K * 31 + d, halo_len=5, seg_mean=9)


def test_workload_sampled(oracle):
    """The benchmark's shape ([8, 8192, 8192], dilation 4, packed
    documents): every output of 2 rows x 3 channel windows against the
    oracle (channels are independent, so a window's oracle needs only its
    own inputs and weights), and a zero-weight check over everything."""
    wl = workloads.ple_conv()
    B, S, C, K = wl.batch, wl.seq, wl.channels, wl.kernel_size
    x = workloads.make_bf16((B, S, C), wl.seed, "cuda")
    w = workloads.make_bf16((C, K), wl.seed + 1, "cuda", std=0.5)
    bias = workloads.make_bf16((C,), wl.seed + 2, "cuda", std=0.5)
    seg = wl.segments()
    out = E.engram_ple_conv(x, w, wl.dilation, bias=bias, seq_ids=dev(seg))
    torch.cuda.synchronize()
    for b in (0, B - 1):
        for c0 in (0, 4096 - 32, C - 64):
            sl = slice(c0, c0 + 64)
            want = oracle.ple_conv(bits(x[b:b + 1, :, sl]), bits(w[sl]), wl.dilation,
                                   bits(bias[sl]), seg[b:b + 1])
            assert np.array_equal(bits(out[b:b + 1, :, sl]), want), (b, c0)
    # zero weights and bias: every output is exactly zero
    zero = E.engram_ple_conv(x, torch.zeros_like(w), wl.dilation, bias=torch.zeros_like(bias),
                             seq_ids=dev(seg), out=out)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(zero.view(torch.int16) & 0x7fff).item()) == 0
    del x, out
    release()
