"""The canonical router-weight-gradient dot, pinned to exact arithmetic and
hand-derived results."""
import numpy as np
import pytest

from oracle import moe_oracle as O

import pins


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H_chunks", [1, 5, 64, 65, 200, 896])
def test_integer_rows_are_exact(dtype, H_chunks):
    V = 4 if dtype == "f32" else 8
    pins.check_dot_integer(O.canonical_dot, dtype, H=V * H_chunks)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H", [128, 2048, 2816, 7168])
def test_error_bound_against_exact_sum(dtype, H):
    pins.check_dot_bound(O.canonical_dot, dtype, H=H)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_derived_order(dtype):
    pins.check_dot_order(O.canonical_dot, dtype)


def test_commutes_in_operands():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((4, 2816)).astype(np.float32)
    b = rng.standard_normal((4, 2816)).astype(np.float32)
    assert np.array_equal(O.canonical_dot(a, b, "f32"), O.canonical_dot(b, a, "f32"))


def test_rejects_partial_chunk():
    with pytest.raises(ValueError):
        O.canonical_dot(np.zeros((1, 6), np.float32), np.zeros((1, 6), np.float32), "f32")
