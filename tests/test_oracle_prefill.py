"""Pins of the oracle's prefill hybrid-precision attention (INT8 QK for the
bulk of the keys, FP16 for vertical lines and the query's own window, one
softmax): hand-derived quantiser codes, exact-rational brute force, closed
forms that reduce to torch's float64 causal attention, and pure-Python
brute force of the mixed-precision logits on tiny inputs."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import hq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_rows.json")


def _rne(fr: Fraction) -> int:
    f = math.floor(fr)
    r = fr - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def test_int8_golden():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float16)[None]
        codes, scale = O.int8_quantize_rows(x)
        assert codes[0].tolist() == c["codes"], c["why"]
        assert np.float32(scale[0]) == np.float32(c["scale"]), c["why"]


def test_int8_exact_rational():
    rng = np.random.default_rng(5)
    rows = np.clip(rng.standard_normal((300, 16)) * rng.choice([1e-3, 1.0, 50.0, 1e4], size=(300, 1)), -6e4, 6e4)
    rows = rows.astype(np.float16)
    # rows with exact half-integer quotients: amax 127 * 2^k and x = (n + 1/2) 2^k
    for k, r in enumerate(rows[:40]):
        e = float(2.0 ** (k % 9 - 4))
        r[:] = (np.arange(16) - 8 + 0.5) * e
        r[0] = 127 * e
    codes, scales = O.int8_quantize_rows(rows)
    for x, c, s in zip(rows, codes, scales):
        xs = [Fraction(float(v)) for v in x]
        amax = max(abs(v) for v in xs)
        if amax == 0:
            assert not c.any() and s == 0
            continue
        want = [_rne(127 * v / amax) for v in xs]
        assert c.tolist() == want
        assert s == np.float32(float(amax) / 127.0)


def test_int8_invariants():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((200, 128)) * 3).astype(np.float16)
    c, s = O.int8_quantize_rows(x)
    assert np.abs(c.astype(int)).max() <= 127
    # the largest-magnitude element maps to +-127, and the rule is odd
    j = np.abs(x.astype(np.float64)).argmax(axis=1)
    assert np.all(np.abs(c[np.arange(200), j].astype(int)) == 127)
    c2, s2 = O.int8_quantize_rows(-x)
    assert np.array_equal(c2.astype(int), -c.astype(int)) and np.array_equal(s, s2)
    # dequantisation error within half a step, plus what rounding the
    # step to fp32 moves the largest code (127 |s - amax/127| <= 127 ulp/2)
    err = np.abs(c * s[:, None].astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -24))


def _sdpa(Q, K, V):
    """torch float64 causal attention of one unit: Q [G][L][d], K, V [L][d]."""
    q = torch.from_numpy(np.asarray(Q, np.float64))
    k = torch.from_numpy(np.asarray(K, np.float64))[None].expand(q.shape[0], -1, -1).contiguous()
    v = torch.from_numpy(np.asarray(V, np.float64))[None].expand(q.shape[0], -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()


def _unit(G=4, L=96, d=128, seed=0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((G, L, d)).astype(np.float16)
    K = rng.standard_normal((L, d)).astype(np.float16)
    V = rng.standard_normal((L, d)).astype(np.float16)
    return Q, K, V


def test_window_covering_everything_is_full_precision():
    Q, K, V = _unit()
    o, _ = O.prefill_hybrid_unit(Q, K, V, None, W=96)
    assert np.abs(o - _sdpa(Q, K, V)).max() < 1e-12


def test_all_vertical_lines_is_full_precision():
    Q, K, V = _unit(seed=1)
    o, _ = O.prefill_hybrid_unit(Q, K, V, np.ones(96, np.uint8), W=0)
    assert np.abs(o - _sdpa(Q, K, V)).max() < 1e-12


def test_no_window_no_lines_is_dequantised_attention():
    Q, K, V = _unit(seed=2)
    o, _ = O.prefill_hybrid_unit(Q, K, V, None, W=0)
    q8, sq = O.int8_quantize_rows(Q)
    k8, sk = O.int8_quantize_rows(K)
    Qh = q8.astype(np.float64) * sq[..., None].astype(np.float64)
    Kh = k8.astype(np.float64) * sk[:, None].astype(np.float64)
    assert np.abs(o - _sdpa(Qh, Kh, V)).max() < 1e-12
    # and it is not the full-precision result
    assert np.abs(o - _sdpa(Q, K, V)).max() > 1e-4


def test_brute_force_mixed():
    G, L, d, W = 2, 23, 16, 5
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((G, L, d)).astype(np.float16)
    K = (rng.standard_normal((L, d)) * 2).astype(np.float16)
    V = rng.standard_normal((L, d)).astype(np.float16)
    flag = (rng.random(L) < 0.3).astype(np.uint8)
    o, lse = O.prefill_hybrid_unit(Q, K, V, flag, W)
    # the row form on a scattered subset of positions gives the same rows
    sub = np.array([22, 3, 0, 17, 9])
    o_s, l_s = O.prefill_rows_unit(Q[:, sub], sub, K, V, flag, W)
    assert np.abs(o_s - o[:, sub]).max() < 1e-12 and np.abs(l_s - lse[:, sub]).max() < 1e-12
    tau = 1.0 / math.sqrt(d)

    def q8row(r):
        amax = max(abs(float(v)) for v in r)
        if amax == 0:
            return [0] * len(r), 0.0
        return [_rne(127 * Fraction(float(v)) / Fraction(amax)) for v in r], float(np.float32(amax / 127.0))

    kq = [q8row(K[i]) for i in range(L)]
    for h in range(G):
        for p in range(L):
            qc, qs = q8row(Q[h, p])
            z = []
            for i in range(p + 1):
                if flag[i] or p - i < W:
                    z.append(tau * math.fsum(float(a) * float(b) for a, b in zip(Q[h, p], K[i])))
                else:
                    kc, ks = kq[i]
                    z.append(tau * sum(a * b for a, b in zip(qc, kc)) * qs * ks)
            m = max(z)
            w = [math.exp(v - m) for v in z]
            sw = math.fsum(w)
            for e in range(d):
                ref = math.fsum(w[i] * float(V[i, e]) for i in range(p + 1)) / sw
                assert abs(o[h, p, e] - ref) < 1e-12
            assert abs(lse[h, p] - (m + math.log(sw))) < 1e-12


def test_first_row_and_lse():
    Q, K, V = _unit(seed=4)
    o, lse = O.prefill_hybrid_unit(Q, K, V, None, W=8)
    assert np.array_equal(o[:, 0], np.broadcast_to(V[0].astype(np.float64), o[:, 0].shape))
    # lse of row 0 is its single logit (key 0 is in the window)
    z0 = (Q[:, 0].astype(np.float64) @ K[0].astype(np.float64)) / math.sqrt(128)
    assert np.abs(lse[:, 0] - z0).max() < 1e-12


def test_flag_changes_only_queries_past_the_window():
    Q, K, V = _unit(seed=7, L=80)
    W, i = 8, 30
    f = np.zeros(80, np.uint8)
    o0, _ = O.prefill_hybrid_unit(Q, K, V, f, W)
    f[i] = 1
    o1, _ = O.prefill_hybrid_unit(Q, K, V, f, W)
    diff = np.abs(o1 - o0).max(axis=(0, 2))
    assert np.all(diff[:i + W] == 0)           # before the key, or key already in the window
    assert np.all(diff[i + W:] > 0)


def test_batch_driver_gqa_mapping():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, L, d = 2, 4, 2, 40, 128
    Q = rng.standard_normal((B, Hq, L, d)).astype(np.float16)
    K = rng.standard_normal((B, Hkv, L, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, L, d)).astype(np.float16)
    flag = (rng.random((B, Hkv, L)) < 0.2).astype(np.uint8)
    o, lse = O.prefill_hybrid(Q, K, V, flag, 6)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ou, lu = O.prefill_hybrid_unit(Q[b, h:h + 1], K[b, g], V[b, g], flag[b, g], 6)
            assert np.array_equal(o[b, h], ou[0]) and np.array_equal(lse[b, h], lu[0])
