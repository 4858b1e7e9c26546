"""Pins for the oracle's E4M3FN decoder (OCP 8-bit floating point, E4M3)."""
import math

import numpy as np
import torch

from oracle import fp8


def test_anchor_codes(golden):
    for code, value in golden("e4m3_anchors.txt"):
        got = fp8.decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        want = float(value)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_sign_symmetry_and_monotone():
    pos = fp8.decode(np.arange(0, 0x7F, dtype=np.uint8))
    neg = fp8.decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(-pos, neg)
    assert np.all(np.diff(pos) > 0)
    assert pos.max() == fp8.MAX_FINITE


def test_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = fp8.decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.isnan(got).sum() == 2


def test_round_trip_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = torch.from_numpy(fp8.decode(codes).astype(np.float32))
    back = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +0 and -0 both round-trip to their own code
    assert np.array_equal(back, codes)
