"""The parity metrics of the GPU tests (gpu_util.Parity), checked on the CPU
against hand-computed values: per-row infinity norm, element-wise error with
the row's rms (or 1e-3 of it) as floor, whole-tensor infinity norm."""
import math

import numpy as np
import pytest

from gpu_util import Parity


def test_identical_is_zero():
    ref = np.random.default_rng(0).standard_normal((3, 50))
    p = Parity("same").add(ref.copy(), ref, axis=1)
    assert p.row_inf == p.elem_rms == p.elem_rms3 == p.whole_inf == 0.0
    p.check(1e-12, 1e-12, 1e-12)


def test_hand_computed_values():
    # two rows over the last axis; row 0 = [3, -4, 0, 0] (max 4, rms 2.5), row 1 = [1, 1, 1, 1]
    ref = np.array([[3.0, -4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0]])
    y = ref.copy()
    y[0, 2] = 0.01      # error 0.01 where ref is 0: floor rms 2.5, floor 1e-3 rms 2.5e-3
    y[1, 3] = 1.002     # error 0.002 on a row of max 1 and rms 1
    p = Parity("hand").add(y, ref, axis=1)
    assert math.isclose(p.row_inf, max(0.01 / 4.0, 0.002 / 1.0))
    assert math.isclose(p.elem_rms, max(0.01 / 2.5, 0.002 / 1.0))
    assert math.isclose(p.elem_rms3, 0.01 / 2.5e-3)
    assert math.isclose(p.whole_inf, 0.01 / 4.0)


def test_blocks_combine_as_one():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((6, 40))
    y = ref + 1e-6 * rng.standard_normal(ref.shape)
    whole = Parity("whole").add(y, ref, axis=1)
    parts = Parity("parts")
    for i in range(0, 6, 2):
        parts.add(y[i:i + 2], ref[i:i + 2], axis=1)
    for attr in ("row_inf", "elem_rms", "elem_rms3", "whole_inf"):
        assert math.isclose(getattr(whole, attr), getattr(parts, attr)), attr
    assert parts.count == ref.size


def test_nan_fails_every_bar():
    ref = np.ones((2, 8))
    y = ref.copy()
    y[1, 5] = np.nan
    p = Parity("nan").add(y, ref, axis=1)
    with pytest.raises(AssertionError):
        p.check(1.0)


def test_gate_and_tight_bar_trip():
    ref = np.ones((1, 10))
    y = ref.copy()
    y[0, 0] = 1.0 + 1e-4
    p = Parity("bar").add(y, ref, axis=1)
    p.check(2e-3)                       # within the gate
    with pytest.raises(AssertionError):
        p.check(2e-3, tight=5e-5)       # but not the tight bar
    with pytest.raises(AssertionError):
        p.check(5e-5)
