"""Pins of the oracle's other strict low-bit widths (2-bit and 8-bit codes,
K and V chosen independently), CPU only.

* Quantiser: brute-force nearest-code search in exact rational arithmetic
  over 2^b - 1 steps (ties to the even code), the scale as the
  nearest fp16 of range / (2^b - 1), the min mapping to 0 and the max to
  2^b - 1, and a reconstruction error of at most half a step.
* Packing: hand-written byte layouts (tests/golden/code_order_2_8.json) and
  unpack(pack(c)) = c.
* The hybrid cache and decode at mixed widths: streaming merges equal a
  fresh pack (K2V4, K8V8, K4V2), fused decode equals the materialised one,
  and the 8-bit cache lies within its quantisation error of full precision.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import hq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _nearest_fp16(exact: Fraction, got: np.float16) -> bool:
    g = Fraction(float(got))
    up = Fraction(float(np.nextafter(got, np.float16(np.inf))))
    dn = Fraction(float(np.nextafter(got, np.float16(-np.inf))))
    eg = abs(exact - g)
    if abs(exact - up) < eg or abs(exact - dn) < eg:
        return False
    for nb in (up, dn):
        if abs(exact - nb) == eg:
            return (np.float16(got).view(np.uint16) & 1) == 0
    return True


def _brute(xs, s, m, qmax):
    out = []
    for xe in xs:
        best = None
        for c in range(qmax + 1):
            err = abs(xe - (c * s + m))
            if best is None or err < best[0] or (err == best[0] and c % 2 == 0):
                best = (err, c)
        out.append(best[1])
    return out


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("seed", range(3))
def test_bruteforce_rational(bits, seed):
    rng = np.random.default_rng(100 + seed)
    qmax = (1 << bits) - 1
    rows = [(rng.standard_normal(128) * sc).astype(np.float16) for sc in (1.0, 1e-3, 50.0, 2.0 ** -20)]
    base = int(rng.integers(-8, 8))
    rows.append(np.array([base + 0.5 * k for k in rng.integers(0, 2 * qmax, 128)], np.float16))
    X = np.stack(rows)
    codes, s16, m16 = O.quantize_groups(X, bits)
    n_ties = 0
    for r in range(X.shape[0]):
        for g in range(4):
            xs = [Fraction(float(v)) for v in X[r, 32 * g:32 * g + 32]]
            m, M = min(xs), max(xs)
            assert Fraction(float(m16[r, g])) == m
            assert _nearest_fp16((M - m) / qmax, s16[r, g])
            s = Fraction(float(s16[r, g]))
            got = codes[r, 32 * g:32 * g + 32].tolist()
            if s == 0:
                assert got == [0] * 32
                continue
            assert got == _brute(xs, s, m, qmax)
            n_ties += sum(1 for xe in xs if ((xe - m) / s).denominator == 2)
    if bits == 2:
        assert n_ties > 0


@pytest.mark.parametrize("bits", [2, 8])
def test_invariants(bits):
    rng = np.random.default_rng(9)
    qmax = (1 << bits) - 1
    X = (rng.standard_normal((128, 128)) * rng.uniform(0.01, 10, (128, 1))).astype(np.float16)
    codes, s16, m16 = O.quantize_groups(X, bits)
    x = X.astype(np.float64).reshape(128, 4, 32)
    c = codes.reshape(128, 4, 32).astype(np.float64)
    s = s16.astype(np.float64)[:, :, None]
    m = m16.astype(np.float64)[:, :, None]
    assert codes.max() <= qmax
    assert np.all(np.take_along_axis(c, x.argmin(axis=2)[:, :, None], 2) == 0)
    assert np.all(np.take_along_axis(c, x.argmax(axis=2)[:, :, None], 2) == qmax)
    assert np.all(np.abs(x - (c * s + m)) <= s / 2 + 1e-300)


def test_code_order_golden():
    with open(os.path.join(GOLD, "code_order_2_8.json")) as f:
        g = json.load(f)
    for key, bits in (("bits2", 2), ("bits8", 8), ("bits4_for_comparison", 4)):
        codes = np.array([g[key]["codes"]], np.uint8)
        assert O.pack_codes(codes, bits)[0].tolist() == g[key]["bytes"], key
        assert O.unpack_codes(np.array([g[key]["bytes"]], np.uint8), bits)[0].tolist() == g[key]["codes"]
    # the 4-bit packer agrees with the nibble packer
    c = np.random.default_rng(2).integers(0, 16, (3, 128)).astype(np.uint8)
    assert np.array_equal(O.pack_codes(c, 4), O.pack_nibbles(c))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(4)
    X = rng.standard_normal((16, 128)).astype(np.float16)
    packed, meta = O.quantize_pack_tokens(X, bits)
    assert packed.shape == (16, 128 * bits // 8) and meta.shape == (16, 4, 2)
    codes, s, _ = O.quantize_groups(X, bits)
    assert np.array_equal(O.unpack_codes(packed, bits), codes)
    xh = O.dequantize(packed, meta, bits)
    assert np.all(np.abs(xh - X.astype(np.float64)) <= np.repeat(s.astype(np.float64), 32, axis=1) / 2)


@pytest.mark.parametrize("kb,vb", [(2, 4), (8, 8), (4, 2)])
def test_streaming_equals_repack(kb, vb):
    L, W, T, d = 300, 32, 20, 128
    rng = np.random.default_rng(kb * 10 + vb)
    K = rng.standard_normal((L + T, d)).astype(np.float16)
    V = rng.standard_normal((L + T, d)).astype(np.float16)
    flag = np.zeros(L + T, np.uint8)
    flag[rng.choice(L - W, 10, replace=False)] = 1
    c = O.quant_pack_unit(K[:L], V[:L], L, W, flag[:L], kb, vb)
    for t in range(L, L + T):
        O.append_merge_unit(c, t, K[t], V[t])
    ref = O.quant_pack_unit(K[:L + T - 1], V[:L + T - 1], L + T - 1, W, flag[:L + T - 1], kb, vb)
    for key in ("kq", "vq", "kq_meta", "vq_meta", "q_pos", "kvl", "vvl", "vl_pos"):
        assert np.array_equal(c[key].view(np.uint8), ref[key].view(np.uint8)), key
    assert c["kq"].shape[1] == d * kb // 8 and c["vq"].shape[1] == d * vb // 8


@pytest.mark.parametrize("kb,vb", [(2, 4), (8, 8), (4, 2)])
def test_fused_equals_unfused(kb, vb):
    L, W, G, d = 400, 64, 4, 128
    rng = np.random.default_rng(kb + 3 * vb)
    K = rng.standard_normal((L + 1, d)).astype(np.float16)
    V = rng.standard_normal((L + 1, d)).astype(np.float16)
    c = O.quant_pack_unit(K[:L], V[:L], L, W, np.zeros(L, np.uint8), kb, vb)
    O.append_merge_unit(c, L, K[L], V[L])
    q = rng.standard_normal((G, d)).astype(np.float16)
    o1, l1 = O.decode_unfused(c, q, L)
    o2, l2 = O.decode_fused(c, q, L)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_k8v8_close_to_full_precision():
    """With 8-bit codes every key and value is within half a step (range /
    510) of its fp16 value, so decode is close to plain attention on the fp16
    keys (torch SDPA in float64): the bound here is loose, the 4-bit cache
    misses it by far more than the 8-bit one."""
    L, W, G, d = 500, 0, 4, 128
    rng = np.random.default_rng(12)
    K = rng.standard_normal((L + 1, d)).astype(np.float16)
    V = rng.standard_normal((L + 1, d)).astype(np.float16)
    q = rng.standard_normal((G, d)).astype(np.float16)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, :, None, :],
        torch.from_numpy(K.astype(np.float64))[None, None].expand(1, G, L + 1, d),
        torch.from_numpy(V.astype(np.float64))[None, None].expand(1, G, L + 1, d))[0, :, 0].numpy()
    errs = {}
    for bits in (8, 4):
        c = O.quant_pack_unit(K[:L], V[:L], L, W, np.zeros(L, np.uint8), bits, bits)
        O.append_merge_unit(c, L, K[L], V[L])
        o, _ = O.decode_fused(c, q, L)
        errs[bits] = np.abs(o - sdpa).max()
    assert errs[8] < 2e-3
    assert errs[8] * 8 < errs[4]
