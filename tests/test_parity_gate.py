"""The attention parity gate (tests/gpu_util.py) on the CPU: the flat bar
for N(0,1) inputs, and the bf16 bound used for scaled queries, which admits
the rounding of P and of O but not a wrong output."""

import numpy as np
import pytest

from gpu_util import BF16_U, MAX_ABS, assert_close


def bits_of(x):
    """fp64 -> bf16 bits, round to nearest even (through fp32, exact here:
    the test values are fp32 values)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def peaked_case(rng, n=4096):
    ref = rng.standard_normal(n) * 0.3
    ref[::97] = 4.1779      # |O| near max|V|: bf16 values there are 2^-5 apart
    return ref


def test_flat_bar_rejects_an_output_near_four_off_by_rounding_plus_p_error():
    ref = peaked_case(np.random.default_rng(0))
    pre = ref.copy()
    pre[::97] -= 0.007                  # pre-rounding error 0.007 on the large outputs
    got = bits_of(pre)                  # then bf16 rounding: 4.1709 -> 4.15625
    with pytest.raises(AssertionError):
        assert_close(got, ref)
    assert_close(got, ref, vmax=4.6)    # within u * (|O| + max|V|)


def test_bf16_bound_rejects_wrong_outputs():
    rng = np.random.default_rng(1)
    ref = peaked_case(rng)
    for bad in (0.05, -0.05):           # one element at |O| ~ 0.3 off by 0.05
        r = ref.copy()
        got = bits_of(r)
        g = (np.asarray(got, np.uint32) << 16).view(np.float32).astype(np.float64)
        g[5] += bad
        with pytest.raises(AssertionError):
            assert_close(bits_of(g), ref, vmax=4.6)
    with pytest.raises(AssertionError):  # the big element off by a bf16 step and a half
        g = ref.copy()
        g[0] += 1.5 * 2 ** -5
        assert_close(bits_of(g), ref, vmax=4.6)
    with pytest.raises(AssertionError):  # small errors everywhere: the mean gate
        assert_close(bits_of(ref + 0.004), ref, vmax=4.6)


def test_bound_is_the_flat_bar_for_small_outputs():
    ref = np.full(64, 0.2)
    assert BF16_U * (0.2 + 4.6) + 1e-3 < MAX_ABS
    got = bits_of(ref + 0.021)
    with pytest.raises(AssertionError):
        assert_close(got, ref, vmax=4.6)
