"""The parity rules themselves (tests/parity.py), on hand-made cases: an
exact tie of a value encoded as given must take the round-half-even code, a
value inside the 1e-6 band may take either code, and any other difference
fails."""
import numpy as np
import pytest

import parity as P


def _grid():
    # one group of 128 channels: scale 0.5, zero -1 (both exact in fp16)
    s = np.array([[0.5]])
    z = np.array([[-1.0]])
    return s, z


def test_exact_ties_round_half_to_even():
    s, z = _grid()
    x = np.zeros((1, 128))
    # boundaries z + (j + 1/2) s = -0.75, -0.25, 0.25
    x[0, :3] = [-0.75, -0.25, 0.25]
    x[0, 3:] = 0.5                       # code 3 exactly
    even = np.full((1, 128), 3, np.uint8)
    even[0, :3] = [0, 2, 2]              # 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    r = P.code_parity(even, x, s, z, 128, given=True)
    assert r["ties"] == 3 and r["tie_bad"] == 0 and r["exempt"] == 0
    up = even.copy()
    up[0, :3] = [1, 2, 3]                # round half up: two ties wrong
    with pytest.raises(AssertionError, match="exact ties"):
        P.code_parity(up, x, s, z, 128, given=True)
    # rotated values: the same elements are exempt, either code passes
    r = P.code_parity(up, x, s, z, 128, given=False)
    assert r["exempt"] == 3


def test_near_band_and_outside():
    s, z = _grid()
    x = np.full((1, 128), 0.5)
    x[0, 0] = -0.25 * (1 + 5e-7)         # inside the 1e-6 band, not a tie
    x[0, 1] = -0.25 * (1 + 5e-6)         # outside the band
    codes = np.full((1, 128), 3, np.uint8)
    codes[0, 0] = 2                      # the other side of the boundary: allowed
    codes[0, 1] = 1                      # correct for x = -0.2500013 (t = 1.4999975)
    r = P.code_parity(codes, x, s, z, 128, given=True)
    assert r["exempt"] == 1 and r["ties"] == 0
    codes[0, 1] = 2
    with pytest.raises(AssertionError, match="outside the exempt band"):
        P.code_parity(codes, x, s, z, 128, given=True)


def test_raw_agreement_and_rate_gate():
    s, z = _grid()
    x = np.full((1, 128), 0.5)
    codes = np.full((1, 128), 3, np.uint8)
    other = codes.copy()
    other[0, :5] = 2
    r = P.code_parity(codes, x, s, z, 128, oracle_codes=other)
    assert r["raw_bad"] == 5
    P.gate_exempt(5, 500_000)            # small sample: reported only
    with pytest.raises(AssertionError):
        P.gate_exempt(11, 1_000_000)     # above 1e-5 on a million elements
