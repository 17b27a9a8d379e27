"""Pins for the oracle's comparison metric, oracle.rel_l2 = ||x - y||_2 / ||y||_2 over
the whole tensor (y the reference; ||x|| when ||y|| = 0).  The librediffusion PR #21
page (section "Validation") reports its kernel against an fp32 reference by this
relative L2 error; every parity assertion in this suite goes through it, so it is
pinned by hand-computed values that each plausible mistake in it breaks."""
import math

import numpy as np
import pytest

import oracle


def pin_identical_is_zero(f):
    y = np.array([[1.5, -2.0], [0.25, 3.0]])
    assert f(y.copy(), y) == 0.0


def pin_double_is_one(f):
    y = np.array([1.0, -2.0, 2.0])
    assert abs(f(2.0 * y, y) - 1.0) < 1e-15


def pin_zero_candidate_is_one(f):
    y = np.array([3.0, 4.0])
    assert abs(f(np.zeros(2), y) - 1.0) < 1e-15


def pin_hand_value(f):
    # x = (3, 4), y = (0, 5): ||x - y|| = ||(3, -1)|| = sqrt(10), ||y|| = 5
    got = f(np.array([3.0, 4.0]), np.array([0.0, 5.0]))
    assert abs(got - math.sqrt(10.0) / 5.0) < 1e-15, got


def pin_zero_reference_gives_norm(f):
    # ||y|| = 0: the result is ||x||, so only exact zeros pass a bar of 0
    assert abs(f(np.array([3.0, 4.0]), np.zeros(2)) - 5.0) < 1e-15
    assert f(np.zeros(3), np.zeros(3)) == 0.0


def pin_whole_tensor(f):
    # one norm over every element, not a mean of per-row ratios: rows (1, 0) and
    # (0, 1) of y with x off by (1, 0) in row 0 only give 1 / sqrt(2)
    y = np.array([[1.0, 0.0], [0.0, 1.0]])
    x = np.array([[2.0, 0.0], [0.0, 1.0]])
    assert abs(f(x, y) - 1.0 / math.sqrt(2.0)) < 1e-15


def pin_reference_is_second(f):
    # asymmetric: normalised by the second argument
    x, y = np.array([2.0, 0.0]), np.array([1.0, 0.0])
    assert abs(f(x, y) - 1.0) < 1e-15 and abs(f(y, x) - 0.5) < 1e-15


def pin_bf16_tensor(f):
    # torch bf16 inputs are widened exactly: 1.0078125 = 1 + 2^-7 is a bf16
    import torch
    x = torch.tensor([1.0078125, 0.0], dtype=torch.bfloat16)
    assert abs(f(x, np.array([1.0, 0.0])) - 2.0 ** -7) < 1e-15


PINS = [pin_identical_is_zero, pin_double_is_one, pin_zero_candidate_is_one, pin_hand_value,
        pin_zero_reference_gives_norm, pin_whole_tensor, pin_reference_is_second, pin_bf16_tensor]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_rel_l2_pin(pin):
    pin(oracle.rel_l2)


def _flat(x, y):
    return oracle._as(x, np.float64).ravel(), oracle._as(y, np.float64).ravel()


def diff_of_norms(x, y):
    x, y = _flat(x, y)
    ny = np.linalg.norm(y)
    d = abs(np.linalg.norm(x) - ny)
    return d / ny if ny > 0 else d


def normalised_by_x(x, y):
    x, y = _flat(x, y)
    nx = np.linalg.norm(x)
    d = np.linalg.norm(x - y)
    return d / nx if nx > 0 else d


def squared(x, y):
    x, y = _flat(x, y)
    ny = np.linalg.norm(y)
    d = np.sum((x - y) ** 2)
    return d / ny ** 2 if ny > 0 else d


def max_abs(x, y):
    x, y = _flat(x, y)
    ny = np.max(np.abs(y))
    d = np.max(np.abs(x - y))
    return d / ny if ny > 0 else d


def mean_row_ratio(x, y):
    x, y = oracle._as(x, np.float64), oracle._as(y, np.float64)
    x, y = x.reshape(-1, x.shape[-1]), y.reshape(-1, y.shape[-1])
    r = [np.linalg.norm(a - b) / np.linalg.norm(b) if np.linalg.norm(b) > 0 else np.linalg.norm(a)
         for a, b in zip(x, y)]
    return float(np.mean(r))


def zero_ref_is_zero(x, y):
    x, y = _flat(x, y)
    ny = np.linalg.norm(y)
    return np.linalg.norm(x - y) / ny if ny > 0 else 0.0


MUTANTS = [diff_of_norms, normalised_by_x, squared, max_abs, mean_row_ratio, zero_ref_is_zero]


@pytest.mark.parametrize("bad", MUTANTS, ids=lambda f: f.__name__)
def test_rel_l2_pins_catch_planted_mistake(bad):
    failed = []
    for pin in PINS:
        try:
            pin(bad)
        except (AssertionError, ZeroDivisionError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no rel_l2 pin caught {bad.__name__}"
