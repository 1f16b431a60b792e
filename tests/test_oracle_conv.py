"""CPU pins for the oracle's causal depthwise PLE convolution (no GPU, no
HIP code).

Source: NeMo AutoModel v0.7 API page (qwen3_8_flash_next.engram),
Qwen3_8_FlashNextPLELayer: _causal_short_conv (causal depthwise convolution
with zeros as the left history), _segmented_conv (each packed segment is
convolved on its own with zeros ahead of it), conv_kernel_size 4 and
short_conv_dilation = ngram_size (so 9 positions of history at ngram 3, the
nine-position CP boundary the page gives).

The pins: torch's conv1d (a library routine) on integer-valued data, where
every product and sum is exact, so the bf16 result must match exactly, with
zero padding on the left and, for packed rows, one conv1d per segment as the
page describes; the impulse response in closed form; the halo form against
the plain form on the joined row; hand-written rounding ties.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


def to_bits(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def to_float(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .float().numpy()


def torch_conv(x, w, bias, d):
    """F.conv1d over [batch, seq, channels] with (K-1)*d zeros on the left."""
    K = w.shape[1]
    xt = torch.tensor(x, dtype=torch.float64).permute(0, 2, 1)
    xt = F.pad(xt, ((K - 1) * d, 0))
    wt = torch.tensor(w, dtype=torch.float64)[:, None, :]
    bt = None if bias is None else torch.tensor(bias, dtype=torch.float64)
    y = F.conv1d(xt, wt, bt, dilation=d, groups=x.shape[2])
    return y.permute(0, 2, 1).numpy()


def int_data(rng, B, S, C, K):
    x = rng.integers(-4, 5, (B, S, C)).astype(np.float32)
    w = rng.integers(-3, 4, (C, K)).astype(np.float32)
    bias = rng.integers(-3, 4, C).astype(np.float32)
    return x, w, bias


@pytest.mark.parametrize("K,d", [(4, 3), (4, 4), (1, 1), (3, 2)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_matches_conv1d_on_exact_data(oracle, K, d, with_bias):
    rng = np.random.Generator(np.random.PCG64(K * 10 + d))
    x, w, bias = int_data(rng, 2, 40, 6, K)
    b = bias if with_bias else None
    got = oracle.ple_conv(to_bits(x), to_bits(w), d, None if b is None else to_bits(b))
    want = torch_conv(x, w, b, d)
    assert np.array_equal(to_float(got), want.astype(np.float32))


def test_segments_match_one_conv1d_per_segment(oracle):
    """The page's procedure: every segment is convolved alone by its own conv1d
    with zeros ahead of it."""
    rng = np.random.Generator(np.random.PCG64(5))
    K, d, S = 4, 3, 50
    x, w, bias = int_data(rng, 2, S, 5, K)
    seg = np.zeros((2, S), dtype=np.int64)
    seg[0, 7:] = 1
    seg[0, 8:] = 2      # a one-position segment
    seg[0, 30:] = 3
    seg[1, 20:] = 9
    got = to_float(oracle.ple_conv(to_bits(x), to_bits(w), d, to_bits(bias), seq_ids=seg))
    for b in range(2):
        starts = [0] + [t for t in range(1, S) if seg[b, t] != seg[b, t - 1]] + [S]
        for a, e in zip(starts, starts[1:]):
            want = torch_conv(x[b:b + 1, a:e], w, bias, d)[0]
            assert np.array_equal(got[b, a:e], want.astype(np.float32)), (b, a, e)


def test_impulse_response_spans_nine_positions(oracle):
    """A unit impulse at p reaches p, p+3, p+6, p+9 (K = 4, dilation 3:
    nine positions of history) with the taps in reverse order."""
    S, C, p = 30, 2, 11
    x = np.zeros((1, S, C), dtype=np.float32)
    x[0, p, :] = 1.0
    w = np.array([[5, 6, 7, 8], [-1, -2, -3, -4]], dtype=np.float32)
    got = to_float(oracle.ple_conv(to_bits(x), to_bits(w), 3))[0]
    want = np.zeros((S, C), dtype=np.float32)
    for k in range(4):
        want[p + (3 - k) * 3] = w[:, k]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("with_seg", [False, True])
def test_halo_equals_joined_row(oracle, with_seg):
    """Feeding the previous positions as a halo gives the outputs the
    convolution of the whole row gives at those positions."""
    rng = np.random.Generator(np.random.PCG64(8))
    K, d, H, S = 4, 3, 9, 33
    x, w, bias = int_data(rng, 2, H + S, 4, K)
    seg = None
    if with_seg:
        seg = np.zeros((2, H + S), dtype=np.int64)
        seg[0, 5:] = 1       # a change inside the halo
        seg[1, H + 2:] = 1   # a change just after it
    whole = oracle.ple_conv(to_bits(x), to_bits(w), d, to_bits(bias), seq_ids=seg)
    part = oracle.ple_conv(to_bits(x[:, H:]), to_bits(w), d, to_bits(bias), seq_ids=seg,
                           halo_bits=to_bits(x[:, :H]))
    assert np.array_equal(part, whole[:, H:])
    alone = oracle.ple_conv(to_bits(x[:, H:]), to_bits(w), d, to_bits(bias))
    assert not np.array_equal(alone, whole[:, H:])   # without the halo the start differs


def test_rounding_ties_to_even(oracle):
    """1 + 2^-8 is a tie between 1 and 1 + 2^-7: it goes to the even 1;
    1 + 3 * 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: it goes up."""
    x = np.ones((1, 1, 2), dtype=np.float32)
    w = np.array([[0, 0, 0, 1], [0, 0, 0, 1]], dtype=np.float32)
    bias = np.array([2 ** -8, 3 * 2 ** -8], dtype=np.float32)
    got = to_float(oracle.ple_conv(to_bits(x), to_bits(w), 3, to_bits(bias)))[0, 0]
    assert list(got) == [1.0, 1.0 + 2 ** -6]
