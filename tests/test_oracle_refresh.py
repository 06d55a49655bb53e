"""Pins of the oracle's decode-time running refresh and scored merge (CPU).

* With every non-window token in FP16 (rho = 1) the refresh's increment is
  the plain causal column mass of dense keys (the pinned attention rows).
* With each row's normaliser computed from the same keys, every buffered row
  adds exactly 1 over the cached positions (mass conservation), whatever the
  quantised part holds.
* The refresh of a cache with K4V4 slots, pack-time and promoted vertical
  lines, a window and a staged token equals the dense column mass (pinned
  by brute force in the selection tests) of the key matrix indexed by
  position, each position's key rebuilt here from its own slot: a K4V4
  slot's nibbles (low first) times its scale plus its min, exactly.  A
  key paired with the wrong position changes that position's score.
* The cut-off is the n_vl-th largest running score of the non-window prefix
  (brute-force sort), +inf when n_vl = 0; the set is the exact top-n_vl.
* The scored merge promotes exactly when score >= cut, and is otherwise the
  plain merge.
"""
import math

import numpy as np
import pytest

from oracle import hq_oracle as O


def _prefix(L, d=128, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L + 8, d)).astype(np.float16)
    V = rng.standard_normal((L + 8, d)).astype(np.float16)
    return K, V, rng


def _exact_lse(keys, pos, qrows, rows_pos, d):
    """Natural-log LSE of each row over the keys at positions <= its own."""
    tau = 1.0 / math.sqrt(d)
    out = np.zeros(len(qrows))
    for r, (q, p) in enumerate(zip(qrows, rows_pos)):
        z = tau * (keys[pos <= p] @ q.astype(np.float64))
        m = z.max()
        out[r] = m + math.log(np.exp(z - m).sum())
    return out


def test_refresh_all_fp16_equals_dense_column_mass():
    L, W, G, nb, d = 200, 16, 2, 12, 128
    K, V, rng = _prefix(L)
    flag = np.ones(L, np.uint8)                     # rho = 1: no K4V4 token
    c = O.quant_pack_unit(K[:L], V[:L], L, W, flag)
    t = L
    O.append_merge_unit(c, t, K[t], V[t])           # the cache holds 0..t
    q = rng.standard_normal((G, nb, d)).astype(np.float16)
    rows_pos = t - nb + 1 + np.arange(nb)
    lse = np.zeros((G, nb))
    for h in range(G):
        _, lse[h] = O.attention_rows(K[:t + 1], q[h], rows_pos, d)
    score = np.zeros(t + 8)
    O.refresh_hybrid_unit(c, t, q, lse, 1.0, score)
    want = np.zeros(t + 8)
    for h in range(G):
        a, _ = O.attention_rows(K[:t + 1], q[h], rows_pos, d)
        want[:t + 1] += a.sum(axis=0)
    assert np.allclose(score, want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("W,rho", [(16, 0.05), (0, 0.1), (64, 0.0)])
def test_refresh_mass_conservation(W, rho):
    L, G, nb, d = 300, 4, 16, 128
    K, V, rng = _prefix(L, seed=3)
    n_nw = max(0, L - W)
    flag = np.zeros(L, np.uint8)
    flag[rng.choice(n_nw, size=n_nw // 20, replace=False)] = 1
    c = O.quant_pack_unit(K[:L], V[:L], L, W, flag)
    for t in range(L, L + 3):
        O.append_merge_unit(c, t, K[t], V[t])
    t = L + 2
    q = rng.standard_normal((G, nb, d)).astype(np.float16)
    pos, keys = O.hybrid_keys(c, t)
    assert sorted(pos.tolist()) == list(range(t + 1))
    rows_pos = t - nb + 1 + np.arange(nb)
    lse = np.stack([_exact_lse(keys, pos, q[h], rows_pos, d) for h in range(G)])
    score = np.zeros(t + 1)
    O.refresh_hybrid_unit(c, t, q, lse, rho, score)
    assert abs(score.sum() - G * nb) < 1e-9
    # running: a second identical refresh doubles every entry
    s2 = score.copy()
    O.refresh_hybrid_unit(c, t, q, lse, rho, s2)
    assert np.allclose(s2, 2 * score, rtol=1e-14)


def _keys_by_position(c, t, d=128):
    """Dense key matrix [t + 1][d] of the cache at decode position t, every
    position's key taken from its own slot (written out here, independently
    of the oracle's region lists): K4V4 slots dequantised from their bytes,
    vertical lines, window ring slots p mod W, the staged token."""
    K = np.full((t + 1, d), np.nan)
    seen = np.zeros(t + 1, np.int64)
    for s_ in range(c["kq"].shape[0]):
        row, p = c["kq"][s_], int(c["q_pos"][s_])
        for g in range(d // 32):
            scale, mn = (float(x) for x in c["kq_meta"][s_, g])
            for e in range(32):
                byte = int(row[(32 * g + e) // 2])
                code = byte & 0xF if e % 2 == 0 else byte >> 4
                K[p, 32 * g + e] = code * scale + mn
        seen[p] += 1
    for i in range(c["kvl"].shape[0]):
        p = int(c["vl_pos"][i])
        K[p] = c["kvl"][i].astype(np.float64)
        seen[p] += 1
    W = c["W"]
    for p in range(max(0, t - W), t):
        K[p] = c["kwin"][p % W].astype(np.float64)
        seen[p] += 1
    K[t] = c["kstg"][0].astype(np.float64)
    seen[t] += 1
    assert np.all(seen == 1)
    return K


@pytest.mark.parametrize("W", [16, 0])
def test_refresh_equals_dense_column_mass_of_the_cache_keys(W):
    L, G, nb, d, rho = 160, 2, 10, 128, 0.1
    K, V, rng = _prefix(L, seed=13)
    K = np.concatenate([K, rng.standard_normal((24, d)).astype(np.float16)])
    V = np.concatenate([V, rng.standard_normal((24, d)).astype(np.float16)])
    n_nw = L - W
    flag = np.zeros(L, np.uint8)
    flag[rng.choice(n_nw, size=n_nw // 10, replace=False)] = 1
    c = O.quant_pack_unit(K[:L], V[:L], L, W, flag)
    # stream tokens, promoting some of the ones that leave the window
    for t in range(L, L + 20):
        O.append_merge_unit(c, t, K[t], V[t], evict_is_vl=(t % 3 == 0))
    t = L + 19
    assert c["kvl"].shape[0] > n_nw // 10            # promoted lines joined the pack-time ones
    q = rng.standard_normal((G, nb, d)).astype(np.float16)
    lse = rng.uniform(2.0, 6.0, (G, nb))              # any normalisers: nothing cancels
    score = np.zeros(t + 1)
    O.refresh_hybrid_unit(c, t, q, lse, rho, score)
    want = O.column_mass_given_lse_unit(_keys_by_position(c, t, d), q, lse, t + 1, 0)
    assert np.allclose(score, want, rtol=1e-12, atol=0.0)
    # the pairing matters: a key moved to another position changes the result
    Kx = _keys_by_position(c, t, d)
    p0, p1 = int(c["q_pos"][3]), int(c["q_pos"][40])
    Kx[[p0, p1]] = Kx[[p1, p0]]
    bad = O.column_mass_given_lse_unit(Kx, q, lse, t + 1, 0)
    assert not np.allclose(score, bad, rtol=1e-9, atol=0.0)


def test_cut_off_and_set():
    L, W, G, nb, d, rho = 400, 32, 2, 8, 128, 0.05
    K, V, rng = _prefix(L, seed=7)
    c = O.quant_pack_unit(K[:L], V[:L], L, W, np.zeros(L, np.uint8))
    O.append_merge_unit(c, L, K[L], V[L])
    q = rng.standard_normal((G, nb, d)).astype(np.float16)
    lse = np.full((G, nb), 3.0)
    score = rng.uniform(0, 1, L + 1)
    score[10] = score[11] = score[12] = 5.0       # a tie at the top
    cut, sel = O.refresh_hybrid_unit(c, L, q, lse, rho, score)
    n_nw = L - W
    n_vl = O.n_vertical(rho, n_nw)
    srt = sorted(((-score[i], i) for i in range(n_nw)))
    assert cut == -srt[n_vl - 1][0]
    assert sel.tolist() == sorted(i for _, i in srt[:n_vl])
    cut0, sel0 = O.refresh_hybrid_unit(c, L, q, lse, 0.0, score.copy())
    assert cut0 == math.inf and sel0.size == 0


def test_scored_merge_promotes_exactly_at_the_cut():
    L, W, d = 120, 16, 128
    K, V, _ = _prefix(L, seed=9)
    for promote_score, want in [(0.75, True), (0.5, True), (0.49, False)]:
        c = O.quant_pack_unit(K[:L], V[:L], L, W, np.zeros(L, np.uint8))
        ref = O.quant_pack_unit(K[:L], V[:L], L, W, np.zeros(L, np.uint8))
        score = np.zeros(L + 8)
        assert O.append_merge_scored_unit(c, L, K[L], V[L], score, 0.5) is False   # only stages
        O.append_merge_unit(ref, L, K[L], V[L])
        score[L - W] = promote_score                 # the token leaving next
        got = O.append_merge_scored_unit(c, L + 1, K[L + 1], V[L + 1], score, 0.5)
        O.append_merge_unit(ref, L + 1, K[L + 1], V[L + 1], evict_is_vl=want)
        assert got is want
        for key in ("kq", "vq", "kq_meta", "vq_meta", "q_pos", "kvl", "vvl", "vl_pos"):
            assert np.array_equal(c[key].view(np.uint8), ref[key].view(np.uint8)), key


def test_refresh_causal_rows_skip_later_keys():
    """A buffered row never sees keys after its own position: with the staged
    token's key made huge, only the last row (the staged token itself) puts
    mass on it."""
    L, W, G, nb, d = 100, 8, 1, 4, 128
    K, V, rng = _prefix(L, seed=11)
    K[L] = np.float16(8.0)
    c = O.quant_pack_unit(K[:L], V[:L], L, W, np.zeros(L, np.uint8))
    O.append_merge_unit(c, L, K[L], V[L])
    q = np.ones((G, nb, d), np.float16)
    lse = np.zeros((G, nb))
    score = np.zeros(L + 1)
    O.refresh_hybrid_unit(c, L, q, lse, 0.05, score)
    tau = 1 / math.sqrt(d)
    assert score[L] == pytest.approx(math.exp(tau * 8.0 * d), rel=1e-12)
