"""Pins of the two error measures every GPU parity test is decided by.

`oracle.rel_l2` is the whole-tensor relative L2 error (the tolerance of the
method's statement: <= 1e-4 for fp32 inputs, <= 2e-2 for bf16), and
`oracle.row_err` bounds the worst (token, head) row against the reference's
typical row.  Both are checked here against hand-computed values, and each
check is shown to reject plausible mistakes in the measure itself (a wrong
divisor, a missing square root, a mean where a maximum belongs), so that a
broken checker cannot turn the parity suite green by itself.
"""
import math

import numpy as np
import pytest

import oracle

# ---------------------------------------------------------------- hand values
# a = (3, 4), b = (0, 5): a - b = (3, -1), ||a - b|| = sqrt(10), ||b|| = 5.
RL2_CASES = [
    ([3.0, 4.0], [0.0, 5.0], math.sqrt(10.0) / 5.0),
    # the reference is the second argument: ||a - b|| = 1 over ||b|| = 2
    ([1.0, 0.0], [2.0, 0.0], 0.5),
    ([2.0, 0.0], [1.0, 0.0], 1.0),
    # a zero reference gives the absolute L2 norm of the difference: ||(1, 2, 2)|| = 3
    ([1.0, 2.0, 2.0], [0.0, 0.0, 0.0], 3.0),
    # identical arrays
    ([0.25, -7.0, 1e-3], [0.25, -7.0, 1e-3], 0.0),
    # shapes are flattened: the same numbers as the first case in a 2 x 1 layout
    ([[3.0], [4.0]], [[0.0], [5.0]], math.sqrt(10.0) / 5.0),
]

# b rows (3, 4) and (0, 0): row norms 5 and 0, RMS row norm sqrt(25 / 2);
# a differs from b by (1, 0) in the second row only: worst row error 1.
ROW_CASES = [
    ([[3.0, 4.0], [1.0, 0.0]], [[3.0, 4.0], [0.0, 0.0]], 1.0 / math.sqrt(12.5)),
    # an all-zero reference: the absolute norm of the worst row, ||(2, 2, 1)|| = 3
    ([[0.0, 0.0, 0.0], [2.0, 2.0, 1.0]], [[0.0, 0.0, 0.0], [0.0, 0.0, 0.0]], 3.0),
    # three axes: rows along the last one; one row of four off by (0, 0, 0, 2)
    (np.concatenate([np.ones((2, 3, 4)).ravel()[:-1], [3.0]]).reshape(2, 3, 4),
     np.ones((2, 3, 4)), 2.0 / 2.0),
]


def _check_rel_l2(fn):
    for a, b, want in RL2_CASES:
        got = fn(np.array(a), np.array(b))
        if not math.isclose(got, want, rel_tol=1e-14, abs_tol=1e-15):
            return False
    return True


def _check_row_err(fn):
    for a, b, want in ROW_CASES:
        got = fn(np.array(a), np.array(b))
        if not (np.isfinite(got) and math.isclose(got, want, rel_tol=1e-14, abs_tol=1e-15)):
            return False
    return True


def test_rel_l2_hand_values():
    for a, b, want in RL2_CASES:
        assert oracle.rel_l2(np.array(a), np.array(b)) == pytest.approx(want, rel=1e-14, abs=1e-15)


def test_rel_l2_is_computed_in_fp64():
    """float32 inputs are widened before the difference: a difference below
    float32 resolution at 1.0 is still seen."""
    a = np.array([1.0 + 2.0 ** -30], dtype=np.float64)
    b = np.array([1.0], dtype=np.float32)
    assert oracle.rel_l2(a, b) == pytest.approx(2.0 ** -30, rel=1e-12)


def test_row_err_hand_values():
    for a, b, want in ROW_CASES:
        assert oracle.row_err(np.array(a), np.array(b)) == pytest.approx(want, rel=1e-14, abs=1e-15)
    assert oracle.row_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    with pytest.raises(ValueError):
        oracle.row_err(np.zeros((2, 4)), np.zeros((4, 2)))


def test_row_err_sees_what_rel_l2_averages_away():
    """A 15 % error on one token of a 64-token chunk passes the bf16 rel-L2
    tolerance of 2e-2 but not a per-row bound."""
    rng = np.random.default_rng(0)
    b = rng.standard_normal((64, 128))
    b /= np.linalg.norm(b, axis=1, keepdims=True)   # unit rows
    a = b.copy()
    a[17] *= 1.15
    assert oracle.rel_l2(a, b) == pytest.approx(0.15 / 8.0, rel=1e-12)
    assert oracle.rel_l2(a, b) <= 2e-2
    assert oracle.row_err(a, b) == pytest.approx(0.15, rel=1e-12)


# ---------------------------------------------------------------- planted mistakes
def _rl2_wrong_divisor(a, b):        # divides by the tested array's norm
    a, b = np.asarray(a, float).ravel(), np.asarray(b, float).ravel()
    na = np.linalg.norm(a)
    return float(np.linalg.norm(a - b) / na) if na > 0 else float(np.linalg.norm(a - b))


def _rl2_no_root(a, b):              # squared norms, no square root
    a, b = np.asarray(a, float).ravel(), np.asarray(b, float).ravel()
    nb = float((b ** 2).sum())
    d = float(((a - b) ** 2).sum())
    return d / nb if nb > 0 else d


def _rl2_max_abs(a, b):              # max-abs ratio in place of L2
    a, b = np.asarray(a, float).ravel(), np.asarray(b, float).ravel()
    nb = np.abs(b).max()
    return float(np.abs(a - b).max() / nb) if nb > 0 else float(np.abs(a - b).max())


def _rl2_sum_divisor(a, b):          # divides by ||a|| + ||b||
    a, b = np.asarray(a, float).ravel(), np.asarray(b, float).ravel()
    return float(np.linalg.norm(a - b) / (np.linalg.norm(a) + np.linalg.norm(b)))


def _rl2_zero_ref_zero(a, b):        # reports 0 when the reference vanishes
    a, b = np.asarray(a, float).ravel(), np.asarray(b, float).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else 0.0


def _rl2_float32(a, b):              # computed in float32
    a, b = np.asarray(a, np.float32).ravel(), np.asarray(b, np.float32).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


@pytest.mark.parametrize("mutant", [_rl2_wrong_divisor, _rl2_no_root, _rl2_max_abs,
                                    _rl2_sum_divisor, _rl2_zero_ref_zero])
def test_rel_l2_pins_reject_mutants(mutant):
    assert _check_rel_l2(oracle.rel_l2)
    assert not _check_rel_l2(mutant), f"{mutant.__name__} passes the rel_l2 pins"


def test_rel_l2_fp64_pin_rejects_float32_mutant():
    a = np.array([1.0 + 2.0 ** -30])
    b = np.array([1.0])
    assert _rl2_float32(a, b) == 0.0
    assert oracle.rel_l2(a, b) > 0.0


def _row_mean(a, b):                 # mean row error in place of the worst
    a, b = np.asarray(a, float), np.asarray(b, float)
    n = b.shape[-1]
    a, b = a.reshape(-1, n), b.reshape(-1, n)
    d = np.sqrt(((a - b) ** 2).sum(axis=1)).mean()
    t = np.sqrt((b ** 2).sum(axis=1).mean())
    return float(d / t) if t > 0 else float(d)


def _row_own_norm(a, b):             # each row against its own reference norm
    a, b = np.asarray(a, float), np.asarray(b, float)
    n = b.shape[-1]
    a, b = a.reshape(-1, n), b.reshape(-1, n)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.sqrt(((a - b) ** 2).sum(axis=1)) / np.sqrt((b ** 2).sum(axis=1))
    return float(np.nanmax(r)) if np.isfinite(r).any() else float("nan")


def _row_frobenius(a, b):            # worst row over the whole tensor's norm
    a, b = np.asarray(a, float), np.asarray(b, float)
    n = b.shape[-1]
    a, b = a.reshape(-1, n), b.reshape(-1, n)
    d = np.sqrt(((a - b) ** 2).sum(axis=1)).max()
    t = np.linalg.norm(b)
    return float(d / t) if t > 0 else float(d)


def _row_first_axis(a, b):           # rows along the first axis instead of the last
    a, b = np.asarray(a, float), np.asarray(b, float)
    n = b.shape[0]
    a, b = a.reshape(n, -1).T, b.reshape(n, -1).T
    d = np.sqrt(((a - b) ** 2).sum(axis=1)).max()
    t = np.sqrt((b ** 2).sum(axis=1).mean())
    return float(d / t) if t > 0 else float(d)


@pytest.mark.parametrize("mutant", [_row_mean, _row_own_norm, _row_frobenius, _row_first_axis])
def test_row_err_pins_reject_mutants(mutant):
    assert _check_row_err(oracle.row_err)
    assert not _check_row_err(mutant), f"{mutant.__name__} passes the row_err pins"
