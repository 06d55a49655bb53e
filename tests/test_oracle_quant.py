"""Pins of the oracle's K4V4 quantiser and packer (CPU only).

The quantiser is checked against (1) hand-derived worked examples, (2) a
brute-force nearest-code search in exact rational arithmetic, and (3) the
invariants of an asymmetric round-to-nearest quantiser.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import hq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _val(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def _groups():
    with open(os.path.join(GOLD, "quant_groups.json")) as f:
        return json.load(f)["groups"]


@pytest.mark.parametrize("g", _groups(), ids=lambda g: g["name"])
def test_worked_examples(g):
    x = np.array([_val(v) for v in g["values"]], dtype=np.float64)
    assert np.all(x.astype(np.float16).astype(np.float64) == x), "fixture not fp16-exact"
    X = np.tile(x.astype(np.float16), 4)[None, :]          # 4 identical groups
    codes, s, m = O.quantize_groups(X)
    assert np.all(s.astype(np.float64) == _val(g["scale"]))
    assert np.all(m.astype(np.float64) == _val(g["min"]))
    assert codes[0, :32].tolist() == g["codes"]
    assert codes[0].tolist() == g["codes"] * 4


def _fp16_rne_fraction_check(exact: Fraction, got: np.float16) -> bool:
    """got is the nearest fp16 to ``exact`` (ties to even mantissa)."""
    g = Fraction(float(got))
    up = Fraction(float(np.nextafter(got, np.float16(np.inf))))
    dn = Fraction(float(np.nextafter(got, np.float16(-np.inf))))
    eg = abs(exact - g)
    if abs(exact - up) < eg or abs(exact - dn) < eg:
        return False
    for nb in (up, dn):
        if abs(exact - nb) == eg:     # tie: got must have an even mantissa
            return (np.float16(got).view(np.uint16) & 1) == 0
    return True


def _brute_codes(x, s, m):
    """argmin_c |x - (c*s + m)| over c in 0..15, ties to the even c."""
    out = []
    for xe in x:
        best = None
        for c in range(16):
            err = abs(xe - (c * s + m))
            if best is None or err < best[0] or (err == best[0] and c % 2 == 0):
                best = (err, c)
        out.append(best[1])
    return out


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_rational(seed):
    rng = np.random.default_rng(seed)
    # groups at very different scales, including subnormal-range groups
    scales = [1.0, 1e-3, 40.0, 3e-6, 2.0 ** -20, 1000.0]
    rows = []
    for sc in scales:
        rows.append((rng.standard_normal(128) * sc).astype(np.float16))
    # tie-rich rows: offsets that are exact half-multiples of a power-of-two scale
    base = rng.integers(-20, 20)
    rows.append(np.array([base + 0.5 * k for k in rng.integers(0, 31, 128)], np.float16))
    X = np.stack(rows)
    codes, s16, m16 = O.quantize_groups(X)
    n_ties = 0
    for r in range(X.shape[0]):
        for g in range(4):
            xs = [Fraction(float(v)) for v in X[r, 32 * g:32 * g + 32]]
            m, M = min(xs), max(xs)
            assert Fraction(float(m16[r, g])) == m
            assert _fp16_rne_fraction_check((M - m) / 15, s16[r, g])
            s = Fraction(float(s16[r, g]))
            got = codes[r, 32 * g:32 * g + 32].tolist()
            if s == 0:
                assert got == [0] * 32
                continue
            assert got == _brute_codes(xs, s, m)
            n_ties += sum(1 for xe in xs if ((xe - m) / s).denominator == 2)
    assert n_ties > 0          # the tie-rich row exercised half-even


def test_invariants_random():
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((256, 128)) * rng.uniform(0.01, 10, (256, 1))).astype(np.float16)
    codes, s16, m16 = O.quantize_groups(X)
    x = X.astype(np.float64).reshape(256, 4, 32)
    c = codes.reshape(256, 4, 32).astype(np.float64)
    s = s16.astype(np.float64)[:, :, None]
    m = m16.astype(np.float64)[:, :, None]
    assert codes.max() <= 15
    # the min maps to code 0, the max to 15 (normal scales)
    assert np.all(np.take_along_axis(c, x.argmin(axis=2)[:, :, None], 2) == 0)
    assert np.all(np.take_along_axis(c, x.argmax(axis=2)[:, :, None], 2) == 15)
    # reconstruction error at most half a step
    assert np.all(np.abs(x - (c * s + m)) <= s / 2 + 1e-300)


def test_signed_zero_is_stored_as_plus_zero():
    """A group of -0 values (or one whose minimum is -0): zero range, so the
    scale is 0 and every code 0; the stored scale and min are +0 (bits 0)."""
    X = np.zeros((2, 128), np.float16)
    X[0] = np.float16(-0.0)
    X[1, :32] = np.float16(-0.0)
    X[1, 32:] = np.abs(np.random.default_rng(1).standard_normal(96)).astype(np.float16)
    X[1, 32] = np.float16(-0.0)
    codes, s, m = O.quantize_groups(X)
    assert np.all(codes[0] == 0) and np.all(codes[1, :32] == 0)
    assert s.view(np.uint16)[0].tolist() == [0, 0, 0, 0]
    assert m.view(np.uint16)[0].tolist() == [0, 0, 0, 0]
    assert s.view(np.uint16)[1, 0] == 0 and m.view(np.uint16)[1, 0] == 0
    assert m.view(np.uint16)[1, 1] == 0 and s.view(np.uint16)[1, 1] != 0


def test_min_of_both_zeros_is_plus_zero_in_either_order():
    """-0 and +0 compare equal, so which one a min reduction returns depends
    on the order of the comparisons; the stored minimum of a group holding
    both is +0 (bits 0x0000) whichever comes first, and the codes and the
    scale do not depend on the order either."""
    rng = np.random.default_rng(7)
    tail = np.abs(rng.standard_normal(30)).astype(np.float16) + np.float16(0.5)
    a = np.concatenate([[np.float16(-0.0), np.float16(0.0)], tail]).astype(np.float16)
    b = np.concatenate([[np.float16(0.0), np.float16(-0.0)], tail]).astype(np.float16)
    c = np.concatenate([tail[:15], [np.float16(-0.0)], tail[15:], [np.float16(0.0)]]).astype(np.float16)
    X = np.zeros((3, 128), np.float16)
    X[0, :32], X[1, :32], X[2, :32] = a, b, c
    X[:, 32:] = np.float16(1.0)
    codes, s, m = O.quantize_groups(X)
    assert m.view(np.uint16)[:, 0].tolist() == [0, 0, 0]
    assert s[0, 0] == s[1, 0] == s[2, 0] and s[0, 0] > 0
    # the zeros take code 0 in every order; the shared tail the same codes
    assert codes[0, 0] == codes[0, 1] == codes[1, 0] == codes[1, 1] == 0
    assert np.array_equal(codes[0, 2:32], codes[1, 2:32])
    assert codes[2, 15] == codes[2, 31] == 0


def test_nibble_order_golden():
    with open(os.path.join(GOLD, "nibble_order.json")) as f:
        g = json.load(f)
    codes = np.array([g["codes"]], np.uint8)
    assert O.pack_nibbles(codes)[0].tolist() == g["bytes"]
    assert O.unpack_nibbles(np.array([g["bytes"]], np.uint8))[0].tolist() == g["codes"]


def test_pack_roundtrip_and_dequantize():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((64, 128)).astype(np.float16)
    packed, meta = O.quantize_pack_tokens(X)
    assert packed.shape == (64, 64) and meta.shape == (64, 4, 2)
    codes, s, m = O.quantize_groups(X)
    assert np.array_equal(O.unpack_nibbles(packed), codes)
    xh = O.dequantize(packed, meta)
    assert np.all(np.abs(xh - X.astype(np.float64)) <= np.repeat(s.astype(np.float64), 32, axis=1) / 2)
