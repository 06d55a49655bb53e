"""Pins of the oracle's staging merge and byte accounting (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import hq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _unit(L0, T, d=128, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L0 + T + 1, d)).astype(np.float16)
    V = rng.standard_normal((L0 + T + 1, d)).astype(np.float16)
    return K, V


@pytest.mark.parametrize("L0,W,T", [(300, 32, 40), (300, 0, 20), (10, 32, 50), (0, 8, 20), (64, 64, 65)])
def test_streaming_equals_repack(L0, W, T):
    """After T merges (tokens L0..L0+T-1 merged, token L0+T staged) the cache
    equals a fresh pack of the dense prefix [0, L0+T) with the same vertical
    lines: K4 slots stay in ascending position."""
    K, V = _unit(L0, T)
    rng = np.random.default_rng(1)
    flag = np.zeros(L0 + T, np.uint8)
    n_nw0 = max(0, L0 - W)
    if n_nw0:
        flag[rng.choice(n_nw0, size=max(1, n_nw0 // 10), replace=False)] = 1
    c = O.quant_pack_unit(K[:L0], V[:L0], L0, W, flag[:L0])
    for t in range(L0, L0 + T + 1):
        O.append_merge_unit(c, t, K[t], V[t])
    L = L0 + T
    r = O.quant_pack_unit(K[:L], V[:L], L, W, flag[:L])
    for key in ("kq", "vq", "kq_meta", "vq_meta", "q_pos", "kvl", "vvl", "vl_pos"):
        assert np.array_equal(c[key].view(np.uint8), r[key].view(np.uint8)), key
    n_win = min(W, L)
    slots = np.arange(L - n_win, L) % max(W, 1)
    if W:
        assert np.array_equal(c["kwin"][slots], r["kwin"][slots])
        assert np.array_equal(c["vwin"][slots], r["vwin"][slots])
    assert c["stg_pos"].tolist() == [L]
    assert np.array_equal(c["kstg"][0], K[L])


def test_evicted_vertical_line_goes_to_fp16():
    K, V = _unit(100, 3)
    c = O.quant_pack_unit(K[:100], V[:100], 100, 16, np.zeros(100, np.uint8))
    n_q0 = c["kq"].shape[0]
    O.append_merge_unit(c, 100, K[100], V[100])           # only stages
    assert c["kq"].shape[0] == n_q0
    O.append_merge_unit(c, 101, K[101], V[101], evict_is_vl=True)
    assert c["vl_pos"].tolist() == [100 - 16]
    assert np.array_equal(c["kvl"][-1], K[84])
    assert c["kq"].shape[0] == n_q0
    O.append_merge_unit(c, 102, K[102], V[102])
    assert c["q_pos"][-1] == 85 and c["kq"].shape[0] == n_q0 + 1


def test_byte_accounting_closed_forms():
    with open(os.path.join(GOLD, "pages_constants.json")) as f:
        g = json.load(f)
    assert O.NB_MAX == g["query_buffer"]["nb_max"]
    for ex in g["query_buffer"]["examples"]:
        assert O.query_buffer_bytes(ex["Hq"], ex["d"]) == ex["bytes"]
    kg = g["kv_growth"]
    assert abs(O.kv_growth_vs_strict(kg["rho"]) - kg["growth_vs_strict_4bit"]) < 1e-12
    # with the fp16 {scale, min} per 32 elements (1 extra bit per element)
    assert abs(O.kv_growth_vs_strict(0.05, code_bits=5.0) - 0.11) < 1e-12
    # bytes per token per KV head at d = 128: K4V4 64+16+64+16, FP16 256+256
    assert O.k4v4_bytes_per_token(128) == 160 and O.fp16_bytes_per_token(128) == 512
    # a quantised unit's arrays really are that size
    K, V = _unit(200, 0)
    c = O.quant_pack_unit(K[:200], V[:200], 200, 0, np.zeros(200, np.uint8))
    per = (c["kq"].nbytes + c["vq"].nbytes + c["kq_meta"].nbytes + c["vq_meta"].nbytes) / 200
    assert per == 160
    # one decode step of the Llama-3.1-8B-shaped layer (B=1, 32/8 heads,
    # L = 32768, W = 128, rho = 5 %): 8 units of 31008 K4V4 + 1632 VL + 128
    # window + 1 staged tokens, plus q in and out
    n_vl = O.n_vertical(0.05, 32768 - 128)
    assert n_vl == 1632
    b = O.decode_step_bytes(1, 32, 8, 128, 32640 - n_vl, n_vl, 128, 1)
    assert b == 8 * (160 * 31008 + 512 * 1761) + 32 * 128 * 4 == 46919680
