"""The GPU parity comparison (tests/parity.py) on the CPU: it passes rounding-level
differences and fails local corruptions that a single global relative L2 lets
through."""
import numpy as np
import pytest

from parity import HEADS_SEQ, HEADS_STATE, check


def _noisy(ref, rel, seed):
    rng = np.random.default_rng(seed)
    return ref * (1 + rel * rng.standard_normal(ref.shape))


def test_rounding_level_differences_pass():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((2, 300, 3, 64))
    s = rng.standard_normal((2, 3, 64, 64))
    check(_noisy(o, 1e-6, 2), o, 2e-3, "o", HEADS_SEQ)
    check(_noisy(s, 1e-7, 3), s, 1e-5, "state", HEADS_STATE)


def test_a_wrong_column_fragment_of_one_state_fails():
    # 16 elements of one head's state halved, in a 2.9B-shaped decode batch: the global
    # relative L2 is 0.5 sqrt(16 / 5.24M) = 8.7e-4, under 2e-3; that head's own is 0.03
    rng = np.random.default_rng(4)
    s = rng.standard_normal((32, 40, 64, 64))
    bad = s.copy()
    bad[7, 13, 16:32, 9] *= 0.5
    with pytest.raises(AssertionError, match="head"):
        check(bad, s, 2e-3, "state", HEADS_STATE)


def test_one_wrong_element_in_a_long_head_fails():
    # one output of a head of 8192 tokens off by half its head's RMS: that head's
    # relative L2 is 0.5 / sqrt(8192 * 64) = 6.9e-4, below 2e-3; the element bound is 2e-2
    rng = np.random.default_rng(5)
    o = rng.standard_normal((1, 8192, 2, 64))
    bad = o.copy()
    bad[0, 4000, 1, 17] += 0.5
    with pytest.raises(AssertionError, match="element"):
        check(bad, o, 2e-3, "o", HEADS_SEQ)


def test_a_zero_head_must_stay_zero():
    o = np.zeros((1, 4, 2, 64))
    o[:, :, 0] = 1.0
    bad = o.copy()
    bad[0, 2, 1, 3] = 1e-30
    check(o, o, 1e-5, "o", HEADS_SEQ)
    with pytest.raises(AssertionError):
        check(bad, o, 1e-5, "o", HEADS_SEQ)


def test_bf16_outputs_get_half_an_ulp_of_their_own():
    import torch
    rng = np.random.default_rng(6)
    o = rng.standard_normal((2, 50, 3, 64)) * np.exp(rng.standard_normal((2, 50, 3, 64)))
    r = torch.from_numpy(o).float().to(torch.bfloat16).double().numpy()
    check(r, o, 4e-3, "bf16 o", HEADS_SEQ, elem_rel=2.0 ** -8)
