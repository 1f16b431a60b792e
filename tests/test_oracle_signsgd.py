"""CPU pins for the oracle's row-sparse SignSGD step (no GPU, no HIP code).

Source: prime-rl v0.9.1.dev179 release notes and pull request 3434,
Validation sections (the RL runs trained with SignSGD, learning rate 1e-6,
default FP32 optimizer math).  Reading: each listed row of the bf16 table
becomes bf16(fp32(w) - lr * sign(g)), subtraction in fp32, one rounding to
bf16 (nearest, ties to even), sign(0) = 0.

The pins: torch's own fp32 arithmetic and fp32 -> bf16 conversion (a library
routine, round to nearest even) on random data; exact binary cases with the
tie-breaking written out by hand; degenerate cases.
"""
import numpy as np
import pytest
import torch


def bf16_bits(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def as_float(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .float().numpy()


@pytest.mark.parametrize("lr", [1e-6, 2.0 ** -8, 0.03125, 0.3])
def test_matches_torch_rounding(oracle, lr):
    rng = np.random.Generator(np.random.PCG64(11))
    rows, dim = 200, 48
    table = bf16_bits(rng.normal(0, 0.02, (rows, dim)))
    ids = rng.choice(rows, 60, replace=False).astype(np.int64)
    grads = rng.normal(0, 1, (60, dim)).astype(np.float32)
    grads[rng.random((60, dim)) < 0.1] = 0.0
    got, bad = oracle.signsgd_rowsparse(ids, grads, table, lr)
    assert bad == 0
    want = torch.from_numpy(table.view(np.int16)).view(torch.bfloat16).clone()
    upd = want[torch.from_numpy(ids)].float() - torch.tensor(lr, dtype=torch.float32) * \
        torch.sign(torch.from_numpy(grads))
    want[torch.from_numpy(ids)] = upd.to(torch.bfloat16)
    assert np.array_equal(got, want.view(torch.int16).numpy().view(np.uint16))


def test_hand_cases_and_ties(oracle):
    """w = 1 and lr = 2^-8: 1 - 2^-8 is representable; 1 + 2^-8 is a tie
    between 1 and 1 + 2^-7 and goes to the even 1; 1 + 2^-7 + 2^-8 is a tie
    between 1 + 2^-7 (odd) and 1 + 2^-6 (even) and goes up; g = 0 leaves w."""
    table = bf16_bits([[1.0, 1.0, 1.0 + 2 ** -7, 0.5, 0.0]])
    grads = np.array([[1.0, -1.0, -3.0, 0.0, -2.0]], dtype=np.float32)
    got, bad = oracle.signsgd_rowsparse(np.array([0]), grads, table, 2.0 ** -8)
    assert bad == 0
    assert list(as_float(got)[0]) == [1.0 - 2 ** -8, 1.0, 1.0 + 2 ** -6, 0.5, 2 ** -8]


def test_small_lr_vanishes_in_bf16(oracle):
    """lr = 1e-6 is far below half a bf16 step of a 0.02-sized weight."""
    table = bf16_bits([[0.02, -0.02, 0.015625]])
    got, _ = oracle.signsgd_rowsparse(np.array([0]), np.array([[1.0, -1.0, 5.0]],
                                                             dtype=np.float32), table, 1e-6)
    assert np.array_equal(got, table)


def test_unlisted_rows_and_invalid_ids(oracle):
    table = bf16_bits(np.arange(12, dtype=np.float32).reshape(4, 3))
    grads = np.ones((3, 3), dtype=np.float32)
    got, bad = oracle.signsgd_rowsparse(np.array([2, -1, 9]), grads, table, 0.5)
    assert bad == 1                       # 9 is out of range; -1 is padding
    f = as_float(got)
    assert list(f[2]) == [5.5, 6.5, 7.5]
    for r in (0, 1, 3):
        assert np.array_equal(got[r], table[r])
