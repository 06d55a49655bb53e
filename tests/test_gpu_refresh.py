"""GPU parity of the decode-time running refresh (hq_refresh_hybrid) and the
scored merge (hq_append_merge_scored) against the fp64 oracle.

The oracle builds its own hybrid cache from the same seeded inputs; the GPU
cache is first checked bit-exact against it, and the oracle's refresh then
runs on the oracle's cache, with row normalisers the oracle computes.

The oracle scores the keys the cache holds: a K4V4 key as its exact
dequantisation code * scale + min.  The kernel feeds the matrix cores that
key rounded to fp16 (one rounding per element, |error| <= u |x| + 2^-25 with
u = 2^-11), so a row's logit tau q.k moves by at most
beta = tau sum_e |q_e| (u |x_e| + 2^-25), and the row's contribution
exp(tau q.k - lse) at that key by a factor within exp(+-beta).  The bounds
below are computed from each case's own keys and queries (score_bounds):

* Running score at every cached position: |gpu - oracle| <= the sum over
  rows of p (exp(beta) - 1) (0 for the FP16 keys), plus 2e-5 relative (fp32
  MFMA scores of fp16 operands and exp2 against fp64, the bound the dense-key
  column mass meets); entries past position t are untouched; with exact
  normalisers every unit gains G * nb up to the summed bound (mass
  conservation).
* Integer work is exact: flags and indices are the top-n_vl of the GPU's own
  fp32 scores (ties to the lower position), and the cut-off is exactly the
  n_vl-th largest of them (+inf when n_vl = 0).
* The selected set differs from the oracle's only at positions whose oracle
  score lies within their own bound plus the largest bound of the prefix
  of the oracle's cut-off (the n_vl-th largest value moves by at most that
  largest bound), and the cut-offs differ by at most that largest bound.
* The scored merge is bit-exact with the oracle's on seeded scores, with
  scores placed exactly at the cut-off and one ulp below it.
* A whole decode loop (merge, decode, refresh every 16 tokens, promotion of
  leaving tokens at the cut-off) ends with the oracle's cache, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, workload
from oracle import hq_oracle as O

from gpu_util import SCORE_RTOL, assert_unit_equal, dev, gpu_pack, score_bounds, unit_from_gpu

pytestmark = pytest.mark.gpu



def _plant_flags(wl, x):
    """Vertical-line flags of the prefix: the first n_vl planted positions."""
    n_nw = max(0, wl.L - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    f = np.zeros((wl.B, wl.Hkv, wl.L), np.uint8)
    for b in range(wl.B):
        f[b, :, x["plant"][b][:n_vl]] = 1
    return f


def _exact_lse(c, t, q):
    """Natural-log LSE of rows q [G][nb][d] (positions t - nb + 1 + j) over
    the oracle cache's keys at positions up to each row's own."""
    G, nb, d = q.shape
    pos, keys = O.hybrid_keys(c, t)
    rows = t - nb + 1 + np.arange(nb)
    out = np.zeros((G, nb))
    for h in range(G):
        z = (q[h].astype(np.float64) @ keys.T) / math.sqrt(d)
        z = np.where(pos[None, :] <= rows[:, None], z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        out[h] = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def _build(wl, x, T, promote_every=3):
    """Prefix pack + T merges on the GPU and in the oracle.  Returns
    (gpu cache, oracle caches, t) with the token at t = L + T - 1 staged."""
    flags = _plant_flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T, extra_vl=T)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags)
    for s in range(T):
        t = wl.L + s
        ev = np.full((wl.B, wl.Hkv), 1 if s % promote_every == 1 else 0, np.uint8)
        H.hq_append_merge(cache.dims, cache, t, dev(x["k_dec"][s]), dev(x["v_dec"][s]),
                          evict_is_vl=dev(ev))
        O.append_merge(ref, t, x["k_dec"][s], x["v_dec"][s], ev)
    torch.cuda.synchronize()
    t = wl.L + T - 1
    for b in range(wl.B):
        for g in range(wl.Hkv):
            assert_unit_equal(unit_from_gpu(cache, b, g), ref[b][g], t, wl.W, tag=f"b{b} g{g}")
    return cache, ref, t


def _own_topk(s, n_vl):
    order = np.lexsort((np.arange(s.size), -s.astype(np.float64)))
    return np.sort(order[:n_vl])


def _refresh_and_check(wl, x, cache, ref, t, nb, seed=0, pad=5):
    B, Hkv, G = wl.B, wl.Hkv, wl.G
    ld = t + 1 + pad
    qb = np.ascontiguousarray(x["qbuf"][:, :, -nb:]) if nb <= x["qbuf"].shape[2] else None
    if qb is None:
        rng = np.random.default_rng(seed + 1)
        qb = rng.standard_normal((B, wl.Hq, nb, 128)).astype(np.float16)
    lse = np.zeros((B, wl.Hq, nb))
    for b in range(B):
        for g in range(Hkv):
            lse[b, g * G:(g + 1) * G] = _exact_lse(ref[b][g], t, qb[b, g * G:(g + 1) * G])
    rng = np.random.default_rng(seed)
    score_in = rng.uniform(0.0, 0.5, (B, Hkv, ld)).astype(np.float32)
    n_nw = max(0, t - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    score = dev(score_in)
    idx = torch.full((B, Hkv, max(1, n_vl)), -1, dtype=torch.int32, device="cuda")
    flag = torch.full((B, Hkv, ld), 7, dtype=torch.uint8, device="cuda")
    cut = torch.full((B, Hkv), -1.0, dtype=torch.float32, device="cuda")
    H.hq_refresh_hybrid(cache.dims, cache, t, dev(qb), dev(lse.astype(np.float32)), score, idx,
                        flag, cut)
    torch.cuda.synchronize()
    sg, ig, fg, cg = (score.cpu().numpy(), idx[:, :, :n_vl].cpu().numpy(), flag.cpu().numpy(),
                      cut.cpu().numpy())
    lse32 = lse.astype(np.float32).astype(np.float64)
    for b in range(B):
        for g in range(Hkv):
            tag = f"b{b} g{g}"
            so = score_in[b, g].astype(np.float64)
            cut_o, sel_o = O.refresh_hybrid_unit(ref[b][g], t, qb[b, g * G:(g + 1) * G],
                                                 lse32[b, g * G:(g + 1) * G], wl.rho, so)
            s = sg[b, g]
            bpos, bnd = score_bounds(ref[b][g], t, qb[b, g * G:(g + 1) * G], lse32[b, g * G:(g + 1) * G])
            tol = np.zeros(t + 1)
            tol[bpos] = bnd
            tol += SCORE_RTOL * so[:t + 1]
            err = np.abs(s[:t + 1] - so[:t + 1])
            worst = int(np.argmax(err / tol))
            assert np.all(err <= tol), (f"{tag} score err {err[worst]:.3e} > bound {tol[worst]:.3e} "
                                        f"at {worst} (score {so[worst]:.4e})")
            assert np.array_equal(s[t + 1:].view(np.uint32), score_in[b, g, t + 1:].view(np.uint32))
            gain = float(s[:t + 1].astype(np.float64).sum() - score_in[b, g, :t + 1].sum())
            assert abs(gain - G * nb) <= bnd.sum() + 1e-4 * G * nb, f"{tag} mass {gain} vs {G * nb}"
            # integer work: exact on the GPU's own scores
            mine = _own_topk(s[:n_nw], n_vl)
            assert np.array_equal(np.nonzero(fg[b, g])[0], mine), f"{tag} flags"
            assert np.array_equal(ig[b, g], mine), f"{tag} indices"
            if n_vl:
                want_cut = np.sort(s[:n_nw])[::-1][n_vl - 1]
                assert cg[b, g] == want_cut, f"{tag} cut {cg[b, g]} vs {want_cut}"
                diff = np.setxor1d(mine, sel_o)
                tmax = tol[:n_nw].max()
                bad = [p for p in diff if abs(so[p] - cut_o) > tol[p] + tmax]
                assert not bad, f"{tag}: {len(bad)} set differences outside the tie band"
                assert abs(cg[b, g] - cut_o) <= tmax
            else:
                assert cg[b, g] == np.inf and cut_o == math.inf
    return sg, cg


CASES = [
    # name, overrides, merged tokens T, buffered rows nb
    ("tiny", {}, 5, 64),
    ("tiny", {"W": 16}, 3, 64),                 # nb > W + 1: every chunk masked
    ("tiny", {"W": 0, "L": 300}, 4, 20),        # no window: staged token only
    ("tiny", {"L": 60}, 10, 32),                # t < W: nothing to select
    ("tiny", {"L": 5}, 1, 6),                   # nb = t + 1: a row at position 0
    ("tiny", {"rho": 1.0, "L": 700}, 2, 64),    # mostly vertical lines
    ("llama31_8b", {"L": 4096}, 3, 64),
    ("glm4_9b", {"B": 2, "L": 2048, "rho": 0.10}, 2, 64),   # G = 16: four row groups
    ("qwen3_32b", {"B": 2, "L": 1500}, 2, 64),             # G = 8: two row groups
]


@pytest.mark.parametrize("name,over,T,nb", CASES, ids=[f"{n}-{o}-T{T}-nb{nb}" for n, o, T, nb in CASES])
def test_refresh_parity(name, over, T, nb):
    wl = workload(name, **over)
    print(f"case {name} {over} T={T} nb={nb}", flush=True)
    x = batch(wl, steps=T)
    cache, ref, t = _build(wl, x, T)
    _refresh_and_check(wl, x, cache, ref, t, nb)


def test_refresh_full_size_llama_layer():
    """Llama-3.1-8B-shaped layer at full size (prefix 32768, two merged
    tokens): every unit, every position."""
    wl = workload("llama31_8b")
    print("case llama31_8b full size", flush=True)
    x = batch(wl, steps=2)
    cache, ref, t = _build(wl, x, 2)
    _refresh_and_check(wl, x, cache, ref, t, 64)


def test_refresh_deterministic():
    wl = workload("tiny", L=2000)
    x = batch(wl, steps=2)
    cache, ref, t = _build(wl, x, 2)
    qb = dev(x["qbuf"])
    lse = torch.full((wl.B, wl.Hq, 64), 6.0, dtype=torch.float32, device="cuda")
    n_vl = O.n_vertical(wl.rho, t - wl.W)
    outs = []
    for _ in range(2):
        score = torch.zeros((wl.B, wl.Hkv, t + 1), dtype=torch.float32, device="cuda")
        idx = torch.zeros((wl.B, wl.Hkv, n_vl), dtype=torch.int32, device="cuda")
        flag = torch.zeros((wl.B, wl.Hkv, t + 1), dtype=torch.uint8, device="cuda")
        cut = torch.zeros((wl.B, wl.Hkv), dtype=torch.float32, device="cuda")
        H.hq_refresh_hybrid(cache.dims, cache, t, qb, lse, score, idx, flag, cut)
        torch.cuda.synchronize()
        outs.append([a.cpu().numpy() for a in (score, idx, flag, cut)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("name,over", [("tiny", {"W": 16, "L": 200}), ("tiny", {"W": 0, "L": 150}),
                                       ("qwen3_32b", {"B": 2, "L": 400})])
def test_scored_merge_bit_exact(name, over):
    """Seeded scores with the leaving token's score put exactly at the cut-off
    (promoted), one ulp below it (kept K4V4) or at random."""
    wl = workload(name, **over)
    print(f"case {name} {over}", flush=True)
    T = 12
    x = batch(wl, steps=T)
    flags = _plant_flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T, extra_vl=T)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags)
    rng = np.random.default_rng(7)
    ld = wl.L + T
    cutv = np.full((wl.B, wl.Hkv), 0.5, np.float32)
    for s in range(T):
        t = wl.L + s
        score = rng.uniform(0.0, 1.0, (wl.B, wl.Hkv, ld)).astype(np.float32)
        ev = t - 1 - wl.W if wl.W > 0 else t - 1
        if ev >= 0 and s % 3 == 0:
            score[:, :, ev] = cutv
        elif ev >= 0 and s % 3 == 1:
            score[:, :, ev] = np.nextafter(cutv, np.float32(0))
        H.hq_append_merge_scored(cache.dims, cache, t, dev(x["k_dec"][s]), dev(x["v_dec"][s]),
                                 dev(score), dev(cutv))
        for b in range(wl.B):
            for g in range(wl.Hkv):
                O.append_merge_scored_unit(ref[b][g], t, x["k_dec"][s, b, g], x["v_dec"][s, b, g],
                                           score[b, g].astype(np.float64), float(cutv[b, g]))
        torch.cuda.synchronize()
        for b in range(wl.B):
            for g in range(wl.Hkv):
                assert_unit_equal(unit_from_gpu(cache, b, g), ref[b][g], t, wl.W, tag=f"s{s} b{b} g{g}")


def test_running_refresh_decode_loop():
    """The decode loop of the method on one small layer: every token is merged
    with the scored promotion rule, decoded (its LSE kept), and every 16
    tokens the last 16 queries refresh the running score and the cut-off.
    Every fifth decoded key repeats the attention-sink key, so those tokens
    gather mass and are promoted when they leave the window.  Both sides run
    the loop on their own (the oracle in fp64); the caches agree bit for bit
    at the end and the GPU's refreshes match the oracle's."""
    wl = workload("tiny", L=400, W=32, B=1)
    T, nb, every = 64, 16, 16
    x = batch(wl, steps=T)
    k_dec = x["k_dec"].copy()
    for s in range(0, T, 5):
        k_dec[s] = x["K"][:, :, 0]
    G, Hkv = wl.G, wl.Hkv
    flags = _plant_flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T, extra_vl=T)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags)
    ld = wl.L + T
    score_g = torch.zeros((1, Hkv, ld), dtype=torch.float32, device="cuda")
    cut_g = torch.full((1, Hkv), np.inf, dtype=torch.float32, device="cuda")
    score_o = np.zeros((Hkv, ld))
    bsum = np.zeros((Hkv, ld))                                   # summed refresh bounds
    cut_o = np.full(Hkv, np.inf)
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, ld)
    out = torch.empty((1, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse_g = torch.empty((1, wl.Hq), dtype=torch.float32, device="cuda")
    qhist, lhist_g, lhist_o = [], [], []
    promoted = 0
    for s in range(T):
        t = wl.L + s
        n_vl_before = cache.t["n_vl"].clone()
        H.hq_append_merge_scored(cache.dims, cache, t, dev(k_dec[s]), dev(x["v_dec"][s]),
                                 score_g, cut_g)
        dec_o = []
        for g in range(Hkv):
            dec_o.append(O.append_merge_scored_unit(ref[0][g], t, k_dec[s, 0, g], x["v_dec"][s, 0, g],
                                                    score_o[g], cut_o[g]))
        dec_g = (cache.t["n_vl"] - n_vl_before).cpu().numpy()[0].astype(bool)
        assert dec_g.tolist() == dec_o, f"step {s}: promotions {dec_g.tolist()} vs {dec_o}"
        promoted += int(dec_g.sum())
        q = x["q_dec"][s]
        H.hq_decode_attn(cache.dims, cache, t, dev(q), out, ws, lse=lse_g)
        lo = np.zeros(wl.Hq)
        for g in range(Hkv):
            _, lo[g * G:(g + 1) * G] = O.decode_fused(ref[0][g], q[0, g * G:(g + 1) * G], t)
        qhist.append(q[0])
        lhist_g.append(lse_g.cpu().numpy()[0].copy())
        lhist_o.append(lo)
        if (s + 1) % every == 0:
            qb = np.stack(qhist[-nb:], axis=1)[None]                # [1][Hq][nb][d]
            lg = np.stack(lhist_g[-nb:], axis=1)[None].astype(np.float32)
            lo_b = np.stack(lhist_o[-nb:], axis=1)
            assert np.abs(lg[0] - lo_b).max() <= 1e-3
            n_vl = O.n_vertical(wl.rho, t - wl.W)
            idx = torch.zeros((1, Hkv, max(1, n_vl)), dtype=torch.int32, device="cuda")
            flag = torch.zeros((1, Hkv, ld), dtype=torch.uint8, device="cuda")
            H.hq_refresh_hybrid(cache.dims, cache, t, dev(qb), dev(lg), score_g, idx, flag, cut_g)
            for g in range(Hkv):
                cut_o[g], _ = O.refresh_hybrid_unit(ref[0][g], t, qb[0, g * G:(g + 1) * G],
                                                    lo_b[g * G:(g + 1) * G], wl.rho, score_o[g])
            torch.cuda.synchronize()
            sg = score_g.cpu().numpy()[0]
            for g in range(Hkv):
                # the GPU's normalisers are its decode LSEs, within 1e-3 of the
                # oracle's; each refresh adds its bound, the running scores the sum
                _, bnd = score_bounds(ref[0][g], t, qb[0, g * G:(g + 1) * G], lo_b[g * G:(g + 1) * G],
                                      lse_tol=1e-3)
                bsum[g, O.hybrid_keys(ref[0][g], t)[0]] += bnd
                tol = bsum[g, :t + 1] + SCORE_RTOL * score_o[g, :t + 1]
                err = np.abs(sg[g, :t + 1] - score_o[g, :t + 1])
                assert np.all(err <= tol), f"step {s} g{g} score err {np.max(err - tol):.2e} over the bound"
    assert promoted > 0
    t = wl.L + T - 1
    for g in range(Hkv):
        assert_unit_equal(unit_from_gpu(cache, 0, g), ref[0][g], t, wl.W, tag=f"g{g}")


def test_refresh_cut_with_split_ties():
    """Running scores so large that the refresh's mass vanishes in their fp32
    rounding: most positions share one value, the cut-off falls inside that
    block and only its lowest positions are taken.  The refresh's top-k (the
    instance that also returns the cut-off) must pick exactly the top n_vl of
    its own scores, ties to the lower position, and return that value."""
    wl = workload("tiny", L=700)
    x = batch(wl, steps=2)
    cache, ref, t = _build(wl, x, 2)
    B, Hkv, G, nb = wl.B, wl.Hkv, wl.G, 64
    ld = t + 1
    qb = np.ascontiguousarray(x["qbuf"][:, :, -nb:])
    lse = np.zeros((B, wl.Hq, nb))
    for b in range(B):
        for g in range(Hkv):
            lse[b, g * G:(g + 1) * G] = _exact_lse(ref[b][g], t, qb[b, g * G:(g + 1) * G])
    n_nw = t - wl.W
    n_vl = O.n_vertical(wl.rho, n_nw)
    score_in = np.full((B, Hkv, ld), 1.0e9, np.float32)
    score_in[:, :, 5:5 + n_vl // 3] = 4.0e9                  # a third of the set clearly above
    score = dev(score_in)
    idx = torch.full((B, Hkv, n_vl), -1, dtype=torch.int32, device="cuda")
    flag = torch.full((B, Hkv, ld), 7, dtype=torch.uint8, device="cuda")
    cut = torch.full((B, Hkv), -1.0, dtype=torch.float32, device="cuda")
    H.hq_refresh_hybrid(cache.dims, cache, t, dev(qb), dev(lse.astype(np.float32)), score, idx, flag, cut)
    torch.cuda.synchronize()
    sg, ig, fg, cg = score.cpu().numpy(), idx.cpu().numpy(), flag.cpu().numpy(), cut.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            s = sg[b, g, :n_nw]
            want_cut = np.sort(s)[::-1][n_vl - 1]
            assert (s == want_cut).sum() > n_vl - (s > want_cut).sum(), "the cut must split a tie"
            mine = _own_topk(s, n_vl)
            assert np.array_equal(np.nonzero(fg[b, g])[0], mine), f"b{b} g{g} flags"
            assert np.array_equal(ig[b, g], mine), f"b{b} g{g} indices"
            assert cg[b, g] == want_cut, f"b{b} g{g} cut"
