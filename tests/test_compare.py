"""The parity tests' comparison helpers (tests/_compare.py), on values whose
answer is known by construction."""
import numpy as np

from _compare import (assert_gated_close, bf16_mismatch, bf16_near_tie, f32_mismatch)


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_near_tie_flags_midpoints_only():
    one_ulp = 2.0 ** -7  # BF16 spacing in [1, 2)
    o = np.array([1.0 + 0.5 * one_ulp,            # exactly a midpoint
                  1.0 + 0.5 * one_ulp + 5e-6,     # inside the band (1e-6 + 1e-5 |o|)
                  1.0 + 0.5 * one_ulp + 3e-5,     # outside it
                  1.0,                            # a BF16 value: half an ulp away
                  -(3.0 + 0.5 * 2.0 ** -6),       # a negative midpoint in [2, 4)
                  4e-7, 0.0])                     # tiny values: within the absolute band
    assert list(bf16_near_tie(o)) == [True, True, False, False, True, True, True]


def test_bf16_and_f32_tolerances():
    a = _bits([1.0, 1.0, 1.0, 1e-7])
    b = _bits([1.0 + 2.0 ** -7, 1.0 + 2.0 ** -6, 1.0 - 2.0 ** -7, -1e-7])
    assert list(bf16_mismatch(a, b)) == [False, True, True, False]  # 1, 2, 2 ulps; abs floor
    assert list(f32_mismatch([1.0001, 1.0002, 0.0], [1.0, 1.0, 9e-6])) == [False, True, False]


def test_gated_close_allows_second_ulp_only_near_ties():
    ref = _bits([1.0, 1.0])
    gpu = _bits([1.0 + 2.0 ** -6, 1.0 + 2.0 ** -6])  # two ulps off
    o_near = np.array([1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8])  # midpoints
    assert_gated_close("near", gpu, ref, o_near)
    o_far = np.array([1.0, 1.0])
    try:
        assert_gated_close("far", gpu, ref, o_far)
    except AssertionError:
        pass
    else:
        raise AssertionError("two ulps away from a non-tie o must fail")
