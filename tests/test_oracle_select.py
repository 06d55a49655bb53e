"""Pins of the oracle's column-mass score and top-rho selection (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import hq_oracle as O
from hq_inputs import workload, batch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_unit(rng, L, G, nb, d=16):
    K = rng.standard_normal((L, d)).astype(np.float16)
    q = (rng.standard_normal((G, nb, d)) * 1.5).astype(np.float16)
    return K, q


def _brute_mass(K, q, L, W):
    """Pure-Python loops: softmax of every buffered query's causal row, then
    per-column sums over heads and queries, non-window columns only."""
    G, nb, d = q.shape
    tau = 1.0 / math.sqrt(d)
    n_nw = max(0, L - W)
    c = [0.0] * n_nw
    for h in range(G):
        for j in range(nb):
            p = L - nb + j
            z = [tau * sum(float(q[h, j, e]) * float(K[i, e]) for e in range(d)) for i in range(p + 1)]
            zm = max(z)
            ex = [math.exp(v - zm) for v in z]
            tot = sum(ex)
            for i in range(min(n_nw, p + 1)):
                c[i] += ex[i] / tot
    return c


@pytest.mark.parametrize("seed", range(12))
def test_topk_equals_bruteforce_sort(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(8, 64))
    W = int(rng.integers(0, 12))
    G = int(rng.integers(1, 4))
    nb = min(int(rng.integers(1, 9)), L)
    rho = float(rng.choice([0.0, 0.05, 0.1, 0.25, 0.5, 1.0]))
    K, q = _rand_unit(rng, L, G, nb)
    c_bf = _brute_mass(K, q, L, W)
    n_nw = max(0, L - W)
    n_vl = int(math.floor(rho * n_nw + 1e-6))
    order = sorted(range(n_nw), key=lambda i: (-c_bf[i], i))
    want = sorted(order[:n_vl])
    score, vl, flag = O.select_vertical_unit(K, q, L, W, rho)
    assert np.allclose(score[:n_nw], c_bf, rtol=1e-12, atol=1e-15)
    assert np.all(score[n_nw:] == 0)
    # no near-tie at the cut-off in these seeds, so the sets must agree exactly
    if 0 < n_vl < n_nw:
        srt = sorted(c_bf, reverse=True)
        assert srt[n_vl - 1] - srt[n_vl] > 1e-9
    assert vl.tolist() == want
    assert flag.sum() == n_vl and all(flag[i] == 1 for i in want)


def test_ties_go_to_lower_position():
    c = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.5])
    assert O.top_rho(c, 1).tolist() == [1]
    assert O.top_rho(c, 2).tolist() == [1, 3]
    assert O.top_rho(c, 3).tolist() == [1, 2, 3]
    assert O.top_rho(c, 4).tolist() == [1, 2, 3, 4]
    assert O.top_rho(c, 0).tolist() == []


@pytest.mark.parametrize("W", [0, 5, 40])
def test_mass_conservation(W):
    """Each causal softmax row sums to 1, so the non-window column mass of
    nb*G rows is at most nb*G, and exactly nb*G when W = 0."""
    rng = np.random.default_rng(W)
    L, G, nb = 96, 3, 16
    K, q = _rand_unit(rng, L, G, nb, d=32)
    dc = O.column_mass_unit(K, q, L, W)
    if W == 0:
        assert abs(dc.sum() - nb * G) < 1e-12
    else:
        assert dc.sum() <= nb * G + 1e-12
    a, lse = O.attention_rows(K, q[0], O.buffered_positions(L, nb), 32)
    assert np.allclose(a.sum(axis=1), 1.0, atol=1e-14)


def test_mass_matches_torch_softmax():
    """Column sums of torch's causal softmax (float64) over the same rows."""
    rng = np.random.default_rng(11)
    L, G, nb, W, d = 200, 4, 64, 32, 64
    K, q = _rand_unit(rng, L, G, nb, d=d)
    Kt = torch.from_numpy(K.astype(np.float64))
    qt = torch.from_numpy(q.astype(np.float64))
    logits = torch.einsum("hjd,id->hji", qt, Kt) / math.sqrt(d)
    pos = torch.arange(L - nb, L)[:, None]
    mask = torch.arange(L)[None, :] <= pos
    a = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1)
    want = a.sum(dim=(0, 1))[: L - W].numpy()
    got = O.column_mass_unit(K, q, L, W)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)
    lse_t = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()
    assert np.allclose(O.row_lse_unit(K, q, L), lse_t, rtol=1e-13, atol=1e-13)


def test_running_score_accumulates():
    rng = np.random.default_rng(5)
    L, G, nb, W = 80, 2, 8, 10
    K, q = _rand_unit(rng, L, G, nb)
    s1, _, _ = O.select_vertical_unit(K, q, L, W, 0.1)
    s2, _, _ = O.select_vertical_unit(K, q, L, W, 0.1, score_in=s1)
    assert np.allclose(s2, 2 * s1, rtol=1e-15)


def test_tiny_workload_counts_golden():
    with open(os.path.join(GOLD, "pages_constants.json")) as f:
        g = json.load(f)["tiny_workload"]
    n_nw, win = O.partition(g["L"], g["W"])
    assert n_nw == g["n_nonwindow"] and win.size == g["W"]
    assert O.n_vertical(g["rho"], n_nw) == g["n_vl"]
    # binary rho: 0.29 * 100 = 28.999999999999996 must still give 29
    assert O.n_vertical(0.29, 100) == 29
    assert O.n_vertical(1.0, 32640) == 32640
    assert O.n_vertical(0.0, 32640) == 0


def test_planted_lines_dominate_when_strong():
    """Structural check of the generator + oracle: strongly planted lines
    (a = 40) are all selected at the tiny shape."""
    wl = workload("tiny", strength=(40.0, 40.0))
    x = batch(wl, steps=1)
    _, idx, _ = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    for g in range(wl.Hkv):
        assert set(x["plant"][0].tolist()) <= set(idx[0][g].tolist())


def test_column_mass_given_lse():
    """With the rows' own LSE it is column_mass_unit; against a pure-Python
    brute force with an arbitrary LSE."""
    import math
    rng = np.random.default_rng(21)
    G, nb, d, L, W = 2, 5, 16, 30, 4
    K = rng.standard_normal((L, d)).astype(np.float16)
    qg = rng.standard_normal((G, nb, d)).astype(np.float16)
    own = O.row_lse_unit(K, qg, L)
    assert np.abs(O.column_mass_given_lse_unit(K, qg, own, L, W) - O.column_mass_unit(K, qg, L, W)).max() < 1e-12
    lse = rng.uniform(1.0, 3.0, (G, nb))
    got = O.column_mass_given_lse_unit(K, qg, lse, L, W)
    tau = 1.0 / math.sqrt(d)
    for i in range(L - W):
        want = 0.0
        for h in range(G):
            for jq in range(nb):
                p = L - nb + jq
                if i <= p:
                    z = tau * math.fsum(float(a) * float(b) for a, b in zip(qg[h, jq], K[i]))
                    want += math.exp(z - lse[h, jq])
        assert abs(got[i] - want) <= 1e-12 * max(1.0, want)
