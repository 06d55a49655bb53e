"""GPU parity of hq_select_vertical against the fp64 oracle.

* The column-mass score agrees with the oracle to a relative 2e-5.
* The selected set has exactly n_vl members and differs from the oracle's
  only at positions whose oracle score lies within 1e-5 (relative) of the
  oracle's cut-off value.
* Integer work is exact: the GPU's flags and indices are exactly the top-n_vl
  (ties to the lower position) of the GPU's own fp32 scores, ascending.
* Reruns are bit-identical; a second refresh adds the same delta again.
"""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import workload, batch
from oracle import hq_oracle as O

from gpu_util import dev

pytestmark = pytest.mark.gpu

SCORE_RTOL = 2e-5
TIE_BAND = 1e-5


def gpu_select(x, wl, score_in=None, lse=None):
    B, Hkv, Hq, L = wl.B, wl.Hkv, wl.Hq, wl.L
    dims = H.make_dims(B, Hq, Hkv, wl.W, wl.rho)
    n_nw = max(0, L - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    score = (torch.zeros((B, Hkv, L), dtype=torch.float32, device="cuda") if score_in is None
             else score_in.clone())
    idx = torch.full((B, Hkv, max(1, n_vl)), -1, dtype=torch.int32, device="cuda")
    flag = torch.full((B, Hkv, L), 7, dtype=torch.uint8, device="cuda")
    ws = H.workspace(dims, H.HQ_OP_SELECT, L)
    H.hq_select_vertical(dims, dev(x["qbuf"]), dev(x["K"]), L, score, idx, flag, ws,
                         lse=None if lse is None else dev(lse.astype(np.float32)))
    torch.cuda.synchronize()
    return score, idx[:, :, :n_vl].cpu().numpy(), flag.cpu().numpy(), n_vl


def exact_topk(c, n_vl):
    order = np.lexsort((np.arange(c.size), -c.astype(np.float64)))
    return np.sort(order[:n_vl])


def check(wl, x, score_g, idx_g, flag_g, n_vl, score_o):
    n_nw = max(0, wl.L - wl.W)
    sg = score_g.cpu().numpy()
    for b in range(wl.B):
        for g in range(wl.Hkv):
            so = score_o[b, g]
            # score accuracy
            if n_nw:
                err = np.abs(sg[b, g, :n_nw] - so[:n_nw]) / np.maximum(so[:n_nw], 1e-30)
                assert err.max() <= SCORE_RTOL, f"b{b} g{g} score rel err {err.max():.2e}"
            assert np.all(flag_g[b, g, n_nw:] == 0)
            # exact top-k of the GPU's own scores
            mine = exact_topk(sg[b, g, :n_nw], n_vl)
            got = np.nonzero(flag_g[b, g])[0]
            assert np.array_equal(got, mine), f"b{b} g{g} flags != top-k of own scores"
            assert np.array_equal(idx_g[b, g], mine)
            # set parity with the oracle up to the tie band
            want = O.top_rho(so[:n_nw], n_vl)
            if n_vl:
                cut = np.sort(so[:n_nw])[::-1][n_vl - 1]
                diff = np.setxor1d(got, want)
                bad = [p for p in diff if abs(so[p] - cut) > TIE_BAND * cut]
                assert not bad, f"b{b} g{g}: {len(bad)} set differences outside the tie band"


CASES = [
    ("tiny", {}),
    ("llama31_8b", {"L": 4096}),
    ("qwen3_8b", {"B": 2, "L": 3000}),
    ("glm4_9b", {"B": 2, "L": 2048, "rho": 0.10}),    # 16 query heads per KV head
    ("qwen3_32b", {"B": 2, "L": 1500}),
    ("tiny", {"W": 0, "L": 500}),                     # causal mask inside the non-window part
    ("tiny", {"L": 100}),                             # no non-window positions
    ("tiny", {"L": 40}),                              # nb = 40 < 64
    ("tiny", {"rho": 1.0, "L": 700}),
    ("tiny", {"rho": 0.0}),
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{o}" for n, o in CASES])
def test_select_parity(name, over):
    wl = workload(name, **over)
    print(f"case {name} {over}", flush=True)
    x = batch(wl, steps=1)
    score_o, _, _ = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl)
    check(wl, x, score_g, idx_g, flag_g, n_vl, score_o)


def test_select_full_size_llama_layer():
    wl = workload("llama31_8b")
    x = batch(wl, steps=1)
    score_o, _, _ = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl)
    assert n_vl == 1632
    check(wl, x, score_g, idx_g, flag_g, n_vl, score_o)


def test_select_full_size_gqa16_layer():
    """The GQA-16 grid's selection as timed: GLM-4-9B-shaped layer (32 query
    heads on 2 KV heads), B=8, L=32768, rho=5 %: 1024 rows per unit in four
    row groups, whose column-mass parts top-k folds in."""
    wl = workload("glm4_9b", rho=0.05)
    assert (wl.B, wl.L, wl.G) == (8, 32768, 16)
    x = batch(wl, steps=1)
    score_o, _, _ = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl)
    assert n_vl == 1632
    check(wl, x, score_g, idx_g, flag_g, n_vl, score_o)


def test_select_with_supplied_lse_and_running_score():
    wl = workload("qwen3_8b", B=2, L=2500)
    x = batch(wl, steps=1)
    G = wl.G
    lse = np.zeros((wl.B, wl.Hq, wl.nb))
    for b in range(wl.B):
        for g in range(wl.Hkv):
            lse[b, g * G:(g + 1) * G] = O.row_lse_unit(x["K"][b, g], x["qbuf"][b, g * G:(g + 1) * G], wl.L)
    s1, i1, f1, n_vl = gpu_select(x, wl)
    s2, i2, f2, _ = gpu_select(x, wl, lse=lse)
    a, c = s1.cpu().numpy(), s2.cpu().numpy()
    assert np.max(np.abs(a - c) / np.maximum(np.abs(a), 1e-30)) < 1e-5
    # second refresh with the same queries adds the identical delta
    s3, i3, f3, _ = gpu_select(x, wl, score_in=s1)
    assert np.array_equal(s3.cpu().numpy(), 2 * a)
    score_o, _, _ = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    check(wl, x, s2, i2, f2, n_vl, score_o)


def test_select_deterministic():
    wl = workload("glm4_9b", B=2, L=3000)
    x = batch(wl, steps=1)
    a = gpu_select(x, wl)
    b = gpu_select(x, wl)
    assert np.array_equal(a[0].cpu().numpy().view(np.uint32), b[0].cpu().numpy().view(np.uint32))
    assert np.array_equal(a[2], b[2])


def _own_topk_exact(wl, score_g, idx_g, flag_g, n_vl):
    """Flags and indices are exactly the top-n_vl of the GPU's own scores."""
    n_nw = max(0, wl.L - wl.W)
    sg = score_g.cpu().numpy()
    for b in range(wl.B):
        for g in range(wl.Hkv):
            mine = exact_topk(sg[b, g, :n_nw], n_vl)
            assert np.array_equal(np.nonzero(flag_g[b, g])[0], mine), f"b{b} g{g} flags"
            assert np.array_equal(idx_g[b, g], mine), f"b{b} g{g} indices"


def test_select_unrepresentative_sample():
    # running scores that are 0 exactly at the positions the top-k samples
    # (t + 1024 k, k = 0 mod 8) and large elsewhere: the sample's bracket
    # misses the cut-off and the full-range radix select must take over
    wl = workload("llama31_8b")
    x = batch(wl, steps=1)
    rng = np.random.default_rng(5)
    base = rng.uniform(1.0, 2.0, size=(wl.B, wl.Hkv, wl.L)).astype(np.float32)
    pos = np.arange(wl.L)
    sampled = ((pos // 1024) % 8) == 0
    base[:, :, sampled] = 0.0
    s_in = torch.from_numpy(base).to("cuda")
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl, score_in=s_in)
    _own_topk_exact(wl, score_g, idx_g, flag_g, n_vl)


def test_select_all_tied_scores():
    # a running score so large that every column mass rounds away: all
    # scores are equal, so the lowest n_vl positions are the set
    wl = workload("llama31_8b")
    x = batch(wl, steps=1)
    s_in = torch.full((wl.B, wl.Hkv, wl.L), 1.0e9, dtype=torch.float32, device="cuda")
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl, score_in=s_in)
    assert torch.all(score_g[:, :, :wl.L - wl.W] == 1.0e9)
    _own_topk_exact(wl, score_g, idx_g, flag_g, n_vl)
    assert np.array_equal(idx_g[0, 0], np.arange(n_vl))


def test_select_workspace_reuse():
    # one workspace across calls (a rho = 0 call in between): the score
    # histogram the kernels pass along must be left zeroed by every call
    wl = workload("llama31_8b", L=12000)
    x = batch(wl, steps=1)
    B, Hkv, Hq, L = wl.B, wl.Hkv, wl.Hq, wl.L
    n_vl = O.n_vertical(wl.rho, L - wl.W)
    ws = H.workspace(H.make_dims(B, Hq, Hkv, wl.W, wl.rho), H.HQ_OP_SELECT, L)
    q, k = dev(x["qbuf"]), dev(x["K"])

    def run(rho):
        dims = H.make_dims(B, Hq, Hkv, wl.W, rho)
        score = torch.zeros((B, Hkv, L), dtype=torch.float32, device="cuda")
        idx = torch.full((B, Hkv, max(1, n_vl)), -1, dtype=torch.int32, device="cuda")
        flag = torch.zeros((B, Hkv, L), dtype=torch.uint8, device="cuda")
        H.hq_select_vertical(dims, q, k, L, score, idx, flag, ws)
        torch.cuda.synchronize()
        return score.cpu().numpy(), idx.cpu().numpy(), flag.cpu().numpy()

    s1, i1, f1 = run(wl.rho)
    _, _, f0 = run(0.0)
    assert not f0.any()
    s2, i2, f2 = run(wl.rho)
    s3, i3, f3 = run(wl.rho)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(f1, f2) and np.array_equal(f1, f3)
    assert np.array_equal(i1[:, :, :n_vl], i2[:, :, :n_vl]) and np.array_equal(i1, i3)
    for b in range(B):
        for g in range(Hkv):
            assert np.array_equal(i1[b, g, :n_vl], exact_topk(s1[b, g, :L - wl.W], n_vl))


def test_select_two_segments():
    """A prefix longer than one top-k segment (32768 positions): keys past the
    first segment are re-read by the histogram passes and flagged segment by
    segment, with indices continuing across the boundary."""
    wl = workload("tiny", L=40000, n_plant=40)
    print("case tiny L=40000", flush=True)
    x = batch(wl, steps=1)
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl)
    score_o, _, _ = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    check(wl, x, score_g, idx_g, flag_g, n_vl, score_o)


@pytest.mark.parametrize("L", [40000, 70000])
def test_select_tied_across_segments(L):
    """Every score equal over two or three segments: the equal keys are ranked
    in position order across segments (the lowest n_vl positions)."""
    wl = workload("tiny", L=L)
    x = batch(wl, steps=1)
    s_in = torch.full((wl.B, wl.Hkv, wl.L), 1.0e9, dtype=torch.float32, device="cuda")
    score_g, idx_g, flag_g, n_vl = gpu_select(x, wl, score_in=s_in)
    _own_topk_exact(wl, score_g, idx_g, flag_g, n_vl)
    assert np.array_equal(idx_g[0, 0], np.arange(n_vl))


def test_select_ties_at_the_cut():
    """A block of equal scores straddling the cut-off: only the lowest of
    them are taken, the higher ones not (ranking inside and across threads'
    words)."""
    wl = workload("llama31_8b", L=9000)
    x = batch(wl, steps=1)
    rng = np.random.default_rng(3)
    n_nw = wl.L - wl.W
    n_vl = O.n_vertical(wl.rho, n_nw)
    base = rng.uniform(0.0, 1.0, size=(wl.B, wl.Hkv, wl.L)).astype(np.float32)
    # n_vl - 100 positions clearly above, 400 tied at the cut, the rest below
    perm = rng.permutation(n_nw)
    for b in range(wl.B):
        for g in range(wl.Hkv):
            base[b, g, perm[:n_vl - 100]] = 1.0e9 + 1.0e3
            base[b, g, perm[n_vl - 100:n_vl + 300]] = 1.0e9
            base[b, g, perm[n_vl + 300:]] = 1.0e6
    s_in = torch.from_numpy(base).to("cuda")
    score_g, idx_g, flag_g, n_vl2 = gpu_select(x, wl, score_in=s_in)
    assert n_vl2 == n_vl
    _own_topk_exact(wl, score_g, idx_g, flag_g, n_vl)
