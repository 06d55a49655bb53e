"""Pins of the oracle's hybrid decode attention (CPU only).

Special cases the pages' mode table names (HyQuant README, 'Mode reference'):
full precision ('dense') is the hybrid path with every prefix token kept in
FP16 (rho = 1, or a window covering the prefix); the strict low-bit cache
('d_k4v4') is the hybrid path with rho = 0 and no window, i.e. dequantise
every prefix token, then run standard attention (the KIVI-style baseline of
the agihunt digest, decode paragraph).  Both are checked against torch's
scaled_dot_product_attention in float64.
"""
import math

import numpy as np
import pytest
import torch

from oracle import hq_oracle as O
from hq_inputs import workload, batch


def _sdpa(q, K, V):
    """torch SDPA, float64, one query row per head: q [G][d], K/V [n][d]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, None, None, :]      # G,1,1,d
    Kt = torch.from_numpy(np.asarray(K, np.float64))[None, None].expand(q.shape[0], 1, -1, -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64))[None, None].expand(q.shape[0], 1, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous())
    return o[:, 0, 0, :].numpy()


def _setup(L, W, rho, seed=0, G=4, d=128):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, d)).astype(np.float16)
    V = rng.standard_normal((L, d)).astype(np.float16)
    qb = rng.standard_normal((G, min(64, L), d)).astype(np.float16)
    kn = rng.standard_normal(d).astype(np.float16)
    vn = rng.standard_normal(d).astype(np.float16)
    q = rng.standard_normal((G, d)).astype(np.float16)
    if L:
        _, _, flag = O.select_vertical_unit(K, qb, L, W, rho)
    else:
        flag = np.zeros(0, np.uint8)
    c = O.quant_pack_unit(K, V, L, W, flag)
    O.append_merge_unit(c, L, kn, vn)
    return K, V, kn, vn, q, c


@pytest.mark.parametrize("L,W,rho", [(300, 32, 1.0), (300, 300, 0.05), (300, 512, 0.0), (64, 64, 0.3)])
def test_full_precision_special_case(L, W, rho):
    K, V, kn, vn, q, c = _setup(L, W, rho)
    assert c["kq"].shape[0] == 0                    # nothing quantised
    Kall = np.concatenate([K, kn[None]])
    Vall = np.concatenate([V, vn[None]])
    want = _sdpa(q, Kall, Vall)
    for fused in (True, False):
        o, lse = (O.decode_fused if fused else O.decode_unfused)(c, q, L)
        assert np.max(np.abs(o - want)) < 1e-12


def test_strict_lowbit_special_case():
    L = 500
    K, V, kn, vn, q, c = _setup(L, 0, 0.0, seed=1)
    assert c["kq"].shape[0] == L and c["kvl"].shape[0] == 0
    # dequantise-then-attend: every prefix token through the quantiser
    pk, mk = O.quantize_pack_tokens(K)
    pv, mv = O.quantize_pack_tokens(V)
    Kall = np.concatenate([O.dequantize(pk, mk), kn[None].astype(np.float64)])
    Vall = np.concatenate([O.dequantize(pv, mv), vn[None].astype(np.float64)])
    want = _sdpa(q, Kall, Vall)
    o, _ = O.decode_fused(c, q, L)
    assert np.max(np.abs(o - want)) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_fused_equals_unfused(seed):
    wl = workload("tiny", L=700 + 37 * seed)
    x = batch(wl, steps=2)
    _, _, flag = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    caches = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flag)
    O.append_merge(caches, wl.L, x["k_dec"][0], x["v_dec"][0])
    o1, l1 = O.decode(caches, x["q_dec"][0], wl.L, fused=True)
    o2, l2 = O.decode(caches, x["q_dec"][0], wl.L, fused=False)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_softmax_weights_sum_to_one():
    """The output with every V set to ones is exactly one (weights sum to 1)."""
    K, V, kn, vn, q, c = _setup(400, 16, 0.05, seed=2)
    for key in ("vvl", "vwin", "vstg"):
        c[key] = np.ones_like(c[key])
    n = c["vq"].shape[0]
    c["vq"] = np.zeros_like(c["vq"])
    c["vq_meta"] = np.zeros_like(c["vq_meta"])
    c["vq_meta"][:, :, 1] = 1.0                      # min 1, scale 0 -> x_hat = 1
    o, _ = O.decode_fused(c, q, 400)
    assert np.max(np.abs(o - 1.0)) < 1e-13


def test_closed_forms():
    d, G = 128, 2
    rng = np.random.default_rng(9)
    # only the staged token (empty prefix): o = v_L and lse = tau q.k_L
    K, V, kn, vn, q, c = _setup(0, 8, 0.05, seed=4, G=G)
    o, lse = O.decode_fused(c, q, 0)
    assert np.max(np.abs(o - vn.astype(np.float64))) == 0
    want_lse = (q.astype(np.float64) @ kn.astype(np.float64)) / math.sqrt(d)
    assert np.max(np.abs(lse - want_lse)) < 1e-12
    # one dominant key -> o tends to its value
    L = 300
    K = rng.standard_normal((L, d)).astype(np.float16)
    V = rng.standard_normal((L, d)).astype(np.float16)
    qd = rng.standard_normal((1, d)).astype(np.float16)
    K[7] = (qd[0].astype(np.float32) * 8).astype(np.float16)
    flag = np.zeros(L, np.uint8)
    flag[7] = 1
    c = O.quant_pack_unit(K, V, L, 32, flag)
    O.append_merge_unit(c, L, K[8], V[8])
    o, _ = O.decode_fused(c, qd, L)
    assert np.max(np.abs(o[0] - V[7].astype(np.float64))) < 1e-6


def test_uniform_weights_mean_value():
    """All hybrid keys identical in value -> o is the plain mean of the values."""
    d, L = 128, 150
    rng = np.random.default_rng(12)
    kv = np.zeros(d, np.float16)                      # zero keys quantise exactly
    K = np.tile(kv, (L, 1))
    V = rng.standard_normal((L, d)).astype(np.float16)
    flag = np.zeros(L, np.uint8)
    flag[[1, 9]] = 1
    c = O.quant_pack_unit(K, V, L, 20, flag)
    O.append_merge_unit(c, L, kv, V[0])
    q = rng.standard_normal((3, d)).astype(np.float16)
    o, lse = O.decode_fused(c, q, L)
    Vt = np.concatenate([r[3] for r in O.hybrid_regions(c, L)])
    assert Vt.shape[0] == L + 1
    assert np.max(np.abs(o - Vt.mean(0)[None])) < 1e-13
    assert np.max(np.abs(lse - math.log(L + 1))) < 1e-13
