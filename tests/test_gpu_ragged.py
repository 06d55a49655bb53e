"""GPU parity of a ragged batch (each sequence at its own position): caches
built one sequence at a time on B = 1 views, then hq_append_merge_ragged and
hq_decode_attn_ragged against the oracle run per sequence at its own
position (bit-exact caches; decode within max-abs 2e-3 / rel-L2 1e-3); with
equal lengths the ragged calls equal the plain ones bit for bit."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, workload
from oracle import hq_oracle as O

from gpu_util import assert_unit_equal, check_decode, dev, unit_from_gpu

pytestmark = pytest.mark.gpu


def _build(wl, x, lengths, T, kb=4, vb=4):
    B, Hkv = wl.B, wl.Hkv
    L_max = max(lengths)
    cache = H.HybridCache.allocate(B, wl.Hq, Hkv, wl.W, wl.rho, L_max + T, extra_vl=T, k_bits=kb, v_bits=vb)
    refs = []
    for b, Lb in enumerate(lengths):
        n_nw = max(0, Lb - wl.W)
        n_vl = O.n_vertical(wl.rho, n_nw)
        flag = np.zeros((1, Hkv, Lb), np.uint8)
        plant = x["plant"][b]
        flag[0, :, plant[plant < n_nw][:n_vl]] = 1
        v = cache.view(b)
        H.hq_quant_pack(v.dims, dev(x["K"][b:b + 1, :, :Lb]), dev(x["V"][b:b + 1, :, :Lb]), Lb, dev(flag), v)
        refs.append([O.quant_pack_unit(x["K"][b, g, :Lb], x["V"][b, g, :Lb], Lb, wl.W, flag[0, g], kb, vb)
                     for g in range(Hkv)])
    return cache, refs


@pytest.mark.parametrize("name,over,lengths,kbvb", [
    ("tiny", {"B": 3, "L": 1500}, [1500, 700, 1100], (4, 4)),
    ("tiny", {"B": 4, "L": 1200}, [1200, 60, 1, 300], (4, 4)),        # shorter than the window, and one token
    ("qwen3_32b", {"B": 2, "L": 1500}, [1500, 1000], (4, 4)),         # G = 8: the general decode path
    ("tiny", {"B": 3, "L": 1500}, [1500, 700, 1100], (8, 4)),         # another width
])
def test_ragged_merge_and_decode(name, over, lengths, kbvb):
    wl = workload(name, **over)
    print(f"case {name} {over} {lengths} K{kbvb[0]}V{kbvb[1]}", flush=True)
    T = 4
    x = batch(wl, steps=T)
    cache, refs = _build(wl, x, lengths, T, *kbvb)
    B, Hkv, G = wl.B, wl.Hkv, wl.G
    L_max = max(lengths)
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, L_max + T)
    out = torch.empty((B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, wl.Hq), dtype=torch.float32, device="cuda")
    for s in range(T):
        t = np.array([Lb + s for Lb in lengths], np.int32)
        H.hq_append_merge_ragged(cache.dims, cache, dev(t), int(t.max()), dev(x["k_dec"][s]), dev(x["v_dec"][s]))
        for b in range(B):
            for g in range(Hkv):
                O.append_merge_unit(refs[b][g], int(t[b]), x["k_dec"][s, b, g], x["v_dec"][s, b, g])
        q = x["q_dec"][s]
        H.hq_decode_attn_ragged(cache.dims, cache, dev(t), int(t.max()), dev(q), out, ws, lse=lse)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        ref = np.zeros((B, wl.Hq, 128))
        ref_l = np.zeros((B, wl.Hq))
        for b in range(B):
            for g in range(Hkv):
                ref[b, g * G:(g + 1) * G], ref_l[b, g * G:(g + 1) * G] = O.decode_fused(
                    refs[b][g], q[b, g * G:(g + 1) * G], int(t[b]))
        check_decode(o, l, ref, ref_l, tag=f"step {s}")
    for b in range(B):
        for g in range(Hkv):
            assert_unit_equal(unit_from_gpu(cache, b, g), refs[b][g], lengths[b] + T - 1, wl.W, tag=f"b{b} g{g}")


def test_ragged_equals_plain_for_equal_lengths():
    wl = workload("llama31_8b", B=2, L=3000)
    x = batch(wl, steps=1)
    c1, _ = _build(wl, x, [3000, 3000], 1)
    c2 = c1.clone()
    t = torch.full((2,), 3000, dtype=torch.int32, device="cuda")
    H.hq_append_merge(c1.dims, c1, 3000, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    H.hq_append_merge_ragged(c2.dims, c2, t, 3000, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    q = dev(x["q_dec"][0])
    outs = []
    for c, ragged in ((c1, False), (c2, True)):
        ws = H.workspace(c.dims, H.HQ_OP_DECODE, 3001)
        out = torch.empty((2, wl.Hq, 128), dtype=torch.float16, device="cuda")
        if ragged:
            H.hq_decode_attn_ragged(c.dims, c, t, 3000, q, out, ws)
        else:
            H.hq_decode_attn(c.dims, c, 3000, q, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))
    for k in c1.t:
        if c1.t[k] is not None:
            assert torch.equal(c1.t[k], c2.t[k]), k


@pytest.mark.parametrize("name,over,lengths", [
    ("tiny", {"B": 3, "L": 1500}, [1500, 700, 1100]),
    ("tiny", {"B": 4, "L": 1200}, [1200, 60, 1, 300]),
    ("qwen3_32b", {"B": 2, "L": 1500}, [1500, 1000]),
])
def test_ragged_step(name, over, lengths):
    """hq_decode_step_ragged: every sequence merges and attends at its own
    position in one launch; outputs against the oracle's merge + decode per
    sequence, then one plain ragged merge on both sides and the caches
    compared bit for bit."""
    wl = workload(name, **over)
    print(f"case {name} {over} {lengths} (step)", flush=True)
    T = 4
    x = batch(wl, steps=T + 1)
    cache, refs = _build(wl, x, lengths, T + 1)
    B, Hkv, G = wl.B, wl.Hkv, wl.G
    L_max = max(lengths)
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, L_max + T + 1)
    out = torch.empty((B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, wl.Hq), dtype=torch.float32, device="cuda")
    for s in range(T + 1):
        t = np.array([Lb + s for Lb in lengths], np.int32)
        if s < T:
            H.hq_decode_step_ragged(cache.dims, cache, dev(t), int(t.max()), dev(x["k_dec"][s]),
                                    dev(x["v_dec"][s]), dev(x["q_dec"][s]), out, ws, lse=lse)
        else:
            H.hq_append_merge_ragged(cache.dims, cache, dev(t), int(t.max()), dev(x["k_dec"][s]),
                                     dev(x["v_dec"][s]))
        for b in range(B):
            for g in range(Hkv):
                O.append_merge_unit(refs[b][g], int(t[b]), x["k_dec"][s, b, g], x["v_dec"][s, b, g])
        if s == T:
            break
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        ref = np.zeros((B, wl.Hq, 128))
        ref_l = np.zeros((B, wl.Hq))
        for b in range(B):
            for g in range(Hkv):
                ref[b, g * G:(g + 1) * G], ref_l[b, g * G:(g + 1) * G] = O.decode_fused(
                    refs[b][g], x["q_dec"][s][b, g * G:(g + 1) * G], int(t[b]))
        check_decode(o, l, ref, ref_l, tag=f"step {s}")
    torch.cuda.synchronize()
    for b in range(B):
        for g in range(Hkv):
            assert_unit_equal(unit_from_gpu(cache, b, g), refs[b][g], lengths[b] + T, wl.W, tag=f"b{b} g{g}")
