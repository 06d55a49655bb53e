"""GPU checks of paged K4V4 slots (a pool of 32-slot blocks shared by all
units, a page table per unit, blocks handed out in a shuffled order): every
entry point reads and writes the same logical cache as with contiguous
slots, so pack, fused and plain decode steps and the decode-time refresh
give bit-identical results; a ragged batch whose sequences own only the
blocks their lengths need matches the oracle per sequence."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, workload
from oracle import hq_oracle as O

from gpu_util import assert_unit_equal, check_decode, dev, gpu_pack, unit_from_gpu

pytestmark = pytest.mark.gpu

T = 4


def _flags(wl, x):
    n_nw = max(0, wl.L - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    f = np.zeros((wl.B, wl.Hkv, wl.L), np.uint8)
    for b in range(wl.B):
        pl = x["plant"][b]
        f[b, :, pl[pl < n_nw][:n_vl]] = 1
    return f


def _same_cache(c, p, wl, tag):
    for b in range(wl.B):
        for g in range(wl.Hkv):
            n = int(c.t["n_q"][b, g])
            assert n == int(p.t["n_q"][b, g]), tag
            for a, q in zip(c.k4_unit(b, g), p.k4_unit(b, g)):
                assert torch.equal(a[:n].contiguous().view(torch.uint8), q[:n].contiguous().view(torch.uint8)), tag
    for k in ("kvl", "vvl", "vl_pos", "kwin", "vwin", "kstg", "vstg", "n_q", "n_vl", "n_stg"):
        if c.t[k] is not None:
            assert torch.equal(c.t[k], p.t[k]), f"{tag} {k}"


CASES = [
    ("tiny", {"B": 2, "L": 1500}, 4, 4),
    ("qwen3_32b", {"B": 1, "L": 700}, 4, 4),      # G = 8: the general decode path
    ("tiny", {"L": 900}, 8, 4),                   # another width: the LDS-tile path
    ("tiny", {"L": 300, "W": 0}, 4, 4),
]


@pytest.mark.parametrize("name,over,kb,vb", CASES)
def test_paged_equals_contiguous(name, over, kb, vb):
    wl = workload(name, **over)
    print(f"case {name} {over} K{kb}V{vb}", flush=True)
    x = batch(wl, steps=2 * T + 1)
    L, W = wl.L, wl.W
    flags = _flags(wl, x)
    c = gpu_pack(x, L, W, wl.rho, flags, L_max=L + 2 * T + 2, extra_vl=2, k_bits=kb, v_bits=vb)
    p = H.HybridCache.allocate_paged(wl.B, wl.Hq, wl.Hkv, W, wl.rho, L + 2 * T + 2, extra_vl=2, k_bits=kb,
                                     v_bits=vb, shuffle_seed=11)
    H.hq_quant_pack(p.dims, dev(x["K"][:, :, :L]), dev(x["V"][:, :, :L]), L, dev(flags), p)
    torch.cuda.synchronize()
    _same_cache(c, p, wl, "after pack")
    oc, op = (torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda") for _ in range(2))
    lc, lp = (torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda") for _ in range(2))
    wc = H.workspace(c.dims, H.HQ_OP_DECODE, L + 2 * T + 1)
    wp = H.workspace(p.dims, H.HQ_OP_DECODE, L + 2 * T + 1)
    for s in range(2 * T):
        t = L + s
        k, v, q = dev(x["k_dec"][s]), dev(x["v_dec"][s]), dev(x["q_dec"][s])
        if s < T:        # fused steps, then plain merge + decode
            H.hq_decode_step(c.dims, c, t, k, v, q, oc, wc, lse=lc)
            H.hq_decode_step(p.dims, p, t, k, v, q, op, wp, lse=lp)
        else:
            for cache, o, l, w in ((c, oc, lc, wc), (p, op, lp, wp)):
                H.hq_append_merge(cache.dims, cache, t, k, v)
                H.hq_decode_attn(cache.dims, cache, t, q, o, w, lse=l)
        torch.cuda.synchronize()
        assert torch.equal(oc.view(torch.int16), op.view(torch.int16)), f"step {s}"
        assert torch.equal(lc, lp), f"step {s}"
    _same_cache(c, p, wl, "after the steps")
    # the decode-time refresh over both
    t = L + 2 * T
    nb = min(64, t + 1)
    rng = np.random.default_rng(3)
    qb = dev(rng.standard_normal((wl.B, wl.Hq, nb, 128)).astype(np.float16))
    lse = dev(rng.uniform(4.0, 8.0, (wl.B, wl.Hq, nb)).astype(np.float32))
    n_vl = O.n_vertical(wl.rho, max(0, t - W))
    res = []
    for cache in (c, p):
        score = torch.zeros((wl.B, wl.Hkv, t + 1), dtype=torch.float32, device="cuda")
        idx = torch.full((wl.B, wl.Hkv, max(1, n_vl)), -1, dtype=torch.int32, device="cuda")
        flag = torch.zeros((wl.B, wl.Hkv, t + 1), dtype=torch.uint8, device="cuda")
        cut = torch.zeros((wl.B, wl.Hkv), dtype=torch.float32, device="cuda")
        H.hq_refresh_hybrid(cache.dims, cache, t, qb, lse, score, idx, flag, cut)
        res.append((score, idx, flag, cut))
    torch.cuda.synchronize()
    for a, b_ in zip(*res):
        assert torch.equal(a, b_)


def test_paged_ragged_batch():
    """Sequences of 1500, 300 and 60 tokens own 46, 6 and 0 blocks per KV
    head instead of the longest one's 46 each; merge + decode at each
    sequence's own position against the oracle, caches bit-exact."""
    wl = workload("tiny", B=3, L=1500)
    lengths = [1500, 300, 60]
    x = batch(wl, steps=T + 1)
    B, Hkv, G, W = wl.B, wl.Hkv, wl.G, wl.W
    L_cap = max(lengths) + T + 1
    p = H.HybridCache.allocate_paged(B, wl.Hq, Hkv, W, wl.rho, L_cap, extra_vl=T + 1,
                                     seq_L_max=[Lb + T + 1 for Lb in lengths], shuffle_seed=5)
    full = H.HybridCache.allocate(B, wl.Hq, Hkv, W, wl.rho, L_cap, extra_vl=T + 1)
    assert p.t["kq"].shape[0] < full.t["kq"].shape[0] * full.t["kq"].shape[1] * full.t["kq"].shape[2] // 2
    del full
    refs = []
    for b, Lb in enumerate(lengths):
        n_vl = O.n_vertical(wl.rho, max(0, Lb - W))
        flag = np.zeros((1, Hkv, Lb), np.uint8)
        pl = x["plant"][b]
        flag[0, :, pl[pl < max(0, Lb - W)][:n_vl]] = 1
        v = p.view(b)
        H.hq_quant_pack(v.dims, dev(x["K"][b:b + 1, :, :Lb]), dev(x["V"][b:b + 1, :, :Lb]), Lb, dev(flag), v)
        refs.append([O.quant_pack_unit(x["K"][b, g, :Lb], x["V"][b, g, :Lb], Lb, W, flag[0, g])
                     for g in range(Hkv)])
    ws = H.workspace(p.dims, H.HQ_OP_DECODE, L_cap)
    out = torch.empty((B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, wl.Hq), dtype=torch.float32, device="cuda")
    for s in range(T):
        t = np.array([Lb + s for Lb in lengths], np.int32)
        H.hq_decode_step_ragged(p.dims, p, dev(t), int(t.max()), dev(x["k_dec"][s]), dev(x["v_dec"][s]),
                                dev(x["q_dec"][s]), out, ws, lse=lse)
        torch.cuda.synchronize()
        ref = np.zeros((B, wl.Hq, 128))
        ref_l = np.zeros((B, wl.Hq))
        for b in range(B):
            for g in range(Hkv):
                O.append_merge_unit(refs[b][g], int(t[b]), x["k_dec"][s, b, g], x["v_dec"][s, b, g])
                ref[b, g * G:(g + 1) * G], ref_l[b, g * G:(g + 1) * G] = O.decode_fused(
                    refs[b][g], x["q_dec"][s][b, g * G:(g + 1) * G], int(t[b]))
        check_decode(out.cpu().numpy(), lse.cpu().numpy(), ref, ref_l, tag=f"step {s}")
    t = np.array([Lb + T for Lb in lengths], np.int32)
    H.hq_append_merge_ragged(p.dims, p, dev(t), int(t.max()), dev(x["k_dec"][T]), dev(x["v_dec"][T]))
    torch.cuda.synchronize()
    for b in range(B):
        for g in range(Hkv):
            O.append_merge_unit(refs[b][g], int(t[b]), x["k_dec"][T, b, g], x["v_dec"][T, b, g])
            assert_unit_equal(unit_from_gpu(p, b, g), refs[b][g], int(t[b]), W, tag=f"b{b} g{g}")
