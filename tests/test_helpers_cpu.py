"""The per-head error norm of the parity tests: a local error in a low-magnitude
head is seen, a head that is zero up to rounding is not divided by its noise."""
import numpy as np

from helpers import rel_err, rel_err_heads


def test_per_head_error_sees_a_small_head():
    ref = np.ones((1, 3, 4, 5))
    ref[0, 2] *= 1e-2                      # a quiet head
    x = ref.copy()
    x[0, 2, 1, 1] += 5e-4                  # 5 % of that head, 0.05 % of the tensor
    assert rel_err(x, ref) < 1e-3
    assert abs(rel_err_heads(x, ref) - 5e-2) < 1e-9


def test_per_head_error_floors_silent_heads():
    ref = np.ones((2, 2, 8))
    ref[1, 1] = 0.0
    x = ref.copy()
    x[1, 1, 0] = 1e-9                      # rounding noise in an all-zero head
    assert rel_err_heads(x, ref) == 1e-9 / 1e-2
