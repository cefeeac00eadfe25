"""CPU checks of the rounding-flip allowance used by the GPU parity tests."""
import numpy as np

from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dw_flip_allowance, flip_ulps, rel_errors, storage_ulp


def test_storage_ulp():
    assert storage_ulp(1.0, "bf16") == 2.0 ** -7
    assert storage_ulp(-3.0, "bf16") == 2.0 ** -6
    assert storage_ulp(1.0, "f32") == 2.0 ** -23
    assert storage_ulp(0.0, "bf16") == 0.0


def test_flip_only_at_a_rounding_midpoint():
    u = np.array([1.0 + 2.0 ** -8,            # the midpoint of 1 and 1 + 2^-7: either rounding is possible
                  1.0 + 2.0 ** -8 - 2.0 ** -22,  # within 2^-16 relative of it
                  1.0 + 2.0 ** -9,            # a quarter ulp from 1: rounds to 1 under any fp32 error
                  5.0])                       # exact
    s = O.round_bf16(u)
    f = flip_ulps(u, s, "bf16")
    assert list(f) == [2.0 ** -7, 2.0 ** -7, 0.0, 0.0]


def test_allowance_sums_flips_times_rows():
    ids = np.array([[0, 1], [1, 0]])
    flips = np.zeros((2, 2, 3))
    flips[0, 1, 2] = 0.5       # token 0, slot 1 (expert 1), row 2
    flips[1, 0, 0] = 0.25      # token 1, slot 0 (expert 1), row 0
    rows = np.array([[1.0, -2.0], [3.0, 4.0]])
    a = dw_flip_allowance(flips, ids, rows, 2)
    assert np.all(a[0] == 0)
    assert np.allclose(a[1][2], [0.5, 1.0]) and np.allclose(a[1][0], [0.75, 1.0]) and np.all(a[1][1] == 0)
    at = dw_flip_allowance(flips, ids, rows, 2, transpose=True)
    assert np.allclose(at[1], a[1].T)


def test_allowance_applies_to_the_max_check_only():
    r = np.ones(1000)
    g = r.copy()
    g[0] += 0.05                      # one element off by 5%
    allow = np.zeros(1000)
    allow[0] = 0.05
    mx, mn = rel_errors(g, r)
    assert mx > 0.02
    assert_close("x", g, r, allow=allow)   # granted: max within tolerance after the allowance
    g2 = g.copy()
    g2[1:] += 0.003                   # a systematic 0.3% error is not covered by any allowance
    try:
        assert_close("x", g2, r, allow=allow)
    except AssertionError:
        pass
    else:
        raise AssertionError("the mean check must not take the allowance")
