"""GPU parity of hq_decode_step (the staging merge of the new token and the
decode attention in one launch) against the oracle's append_merge then
decode: outputs within max-abs 2e-3 / rel-L2 1e-3 every step, the cache
bit-exact at the end; and equal, bit for bit, to hq_append_merge +
hq_decode_attn on the GPU."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, workload
from oracle import hq_oracle as O

from gpu_util import assert_unit_equal, check_decode, dev, gpu_pack, unit_from_gpu

pytestmark = pytest.mark.gpu

T = 6


def _flags(wl, x):
    B, Hkv, L = wl.B, wl.Hkv, wl.L
    n_nw = max(0, L - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    f = np.zeros((B, Hkv, L), np.uint8)
    for b in range(B):
        pl = x["plant"][b]
        f[b, :, pl[pl < n_nw][:n_vl]] = 1
    return f


def _evict(wl, s, mode):
    if not mode or not mode.startswith("promote"):
        return None
    e = np.zeros((wl.B, wl.Hkv), np.uint8)
    e.flat[s % 2::2] = 1                   # every other unit promotes, alternating by step
    return e


CASES = [
    ("tiny", {"L": 1500}, 4, 4, None),                     # G = 4: the grouped-column path
    ("qwen3_32b", {"L": 700, "B": 2}, 4, 4, None),         # G = 8: the general path
    ("tiny", {"L": 900}, 8, 4, None),                      # another width (LDS-tile path)
    ("tiny", {"L": 1100}, 4, 2, None),                     # K4V2 at G = 4: grouped path, 2-bit V codes
    ("tiny", {"L": 1000}, 2, 4, None),                     # K2V4 at G = 4: grouped path, 2-bit K codes
    ("tiny", {"L": 700}, 2, 2, "promote"),                 # K2V2, with promotions
    ("tiny", {"L": 300, "W": 0}, 4, 4, None),              # no window: the new token itself leaves
    ("tiny", {"L": 60}, 4, 4, None),                       # the window is not full yet
    ("tiny", {"L": 800}, 4, 4, "promote"),                 # leaving tokens promoted to lines
    ("llama31_8b", {"L": 4096}, 4, 4, "promote"),          # 8 KV heads
    ("tiny", {"L": 800}, 4, 4, "promote-full"),            # no room for lines: promoted tokens stay K4V4
]


@pytest.mark.parametrize("name,over,kb,vb,mode", CASES)
def test_step_parity(name, over, kb, vb, mode):
    wl = workload(name, **over)
    print(f"case {name} {over} K{kb}V{vb} {mode}", flush=True)
    x = batch(wl, steps=T + 1)
    L, W = wl.L, wl.W
    flags = _flags(wl, x)
    extra = T + 2
    if mode == "promote-full":
        # one free line slot per unit: the first promotion fits, later ones
        # are turned away (negative extra: fewer slots than rho would give)
        extra = int(flags.sum(axis=2).max()) + 1 - O.n_vertical(wl.rho, L + T + 2 - W)
    cache = gpu_pack(x, L, W, wl.rho, flags, L_max=L + T + 2, extra_vl=extra, k_bits=kb, v_bits=vb)
    refs = O.quant_pack(x["K"][:, :, :L], x["V"][:, :, :L], L, W, flags, kb, vb)
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, L + T + 1)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    prev = None                                   # the promotion flags of the previous step
    # a flagged token becomes a line only while the unit's line region has
    # room (the library's capacity rule; the oracle's cache has no capacity)
    room = np.array([[cache.dims.cap_vl - refs[b][g]["vl_pos"].size for g in range(wl.Hkv)]
                     for b in range(wl.B)])
    refused = 0
    for s in range(T):
        t = L + s
        ev = _evict(wl, s, mode)
        H.hq_decode_step(cache.dims, cache, t, dev(x["k_dec"][s]), dev(x["v_dec"][s]), dev(x["q_dec"][s]),
                         out, ws, lse=lse, evict_is_vl=dev(ev) if ev is not None else None)
        torch.cuda.synchronize()
        # the oracle merges the token leaving at t - 1 - W now; the step let
        # the token at t - 1 - W leave at the end of the previous step
        O.append_merge(refs, t, x["k_dec"][s], x["v_dec"][s], prev)
        ref_o, ref_l = O.decode(refs, x["q_dec"][s], t)
        check_decode(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, tag=f"step {s}")
        if ev is not None and L + s - W >= 0:
            kept = ev & (room > 0)
            refused += int(ev.sum() - kept.sum())
            room -= kept
            ev = kept
        prev = ev
    # one plain merge on both sides: the caches then hold the same staged token
    t = L + T
    H.hq_append_merge(cache.dims, cache, t, dev(x["k_dec"][T]), dev(x["v_dec"][T]))
    O.append_merge(refs, t, x["k_dec"][T], x["v_dec"][T], prev)
    torch.cuda.synchronize()
    for b in range(wl.B):
        for g in range(wl.Hkv):
            assert_unit_equal(unit_from_gpu(cache, b, g), refs[b][g], t, W, tag=f"b{b} g{g}")
    if mode == "promote-full":
        assert refused > 0                        # the full region did turn promotions away


@pytest.mark.parametrize("name,over", [("tiny", {"L": 1500}), ("qwen3_32b", {"L": 900, "B": 2}),
                                       ("tiny", {"L": 200, "W": 0}),
                                       # G = 1, 2, 3 (the step's own fold at G = 3 with at
                                       # most 32 splits, the shared fold otherwise)
                                       ("tiny", {"L": 1500, "Hq": 2}), ("tiny", {"L": 1500, "Hq": 4}),
                                       ("tiny", {"L": 1500, "Hq": 6}), ("tiny", {"L": 8192, "Hq": 6})])
def test_step_equals_merge_then_decode(name, over):
    wl = workload(name, **over)
    x = batch(wl, steps=T)
    L, W = wl.L, wl.W
    flags = _flags(wl, x)
    c1 = gpu_pack(x, L, W, wl.rho, flags, L_max=L + T + 2, extra_vl=2)
    c2 = c1.clone()
    ws1 = H.workspace(c1.dims, H.HQ_OP_DECODE, L + T + 1)
    ws2 = H.workspace(c2.dims, H.HQ_OP_DECODE, L + T + 1)
    o1 = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    o2 = torch.empty_like(o1)
    l1 = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    for s in range(T):
        t = L + s
        k, v, q = dev(x["k_dec"][s]), dev(x["v_dec"][s]), dev(x["q_dec"][s])
        H.hq_decode_step(c1.dims, c1, t, k, v, q, o1, ws1, lse=l1)
        # the unfused pair attends the same tokens: its merge at t moves the
        # token at t - 1 that the previous step already moved
        H.hq_append_merge(c2.dims, c2, t, k, v)
        H.hq_decode_attn(c2.dims, c2, t, q, o2, ws2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"step {s}"
        assert torch.equal(l1, l2), f"step {s}"


def test_step_refuses_units_with_a_staged_token():
    """hq_decode_step needs nothing staged.  With a token staged in sequence 0
    only (a plain hq_append_merge on its B = 1 view), the step refuses
    sequence 0's units (NaN out and lse, their cache bytes unchanged) and
    steps sequence 1 exactly as it does on a cache where nothing is staged."""
    wl = workload("tiny", B=2, L=600)
    x = batch(wl, steps=2)
    L, W = wl.L, wl.W
    flags = _flags(wl, x)
    c = gpu_pack(x, L, W, wl.rho, flags, L_max=L + 4, extra_vl=2)
    ref = c.clone()
    v0 = c.view(0)
    H.hq_append_merge(v0.dims, v0, L, dev(x["k_dec"][0][:1]), dev(x["v_dec"][0][:1]))
    torch.cuda.synchronize()
    before = {k: v[0].clone() for k, v in c.t.items() if v is not None and k != "k4_pages"}
    k, v, q = dev(x["k_dec"][1]), dev(x["v_dec"][1]), dev(x["q_dec"][1])
    outs = []
    for cc in (c, ref):
        o = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
        ls = torch.zeros((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
        H.hq_decode_step(cc.dims, cc, L, k, v, q, o, H.workspace(cc.dims, H.HQ_OP_DECODE, L + 4), lse=ls)
        outs.append((o, ls))
    torch.cuda.synchronize()
    (o, ls), (o_ref, ls_ref) = outs
    assert torch.isnan(o[0]).all() and torch.isnan(ls[0]).all()
    for key, val in before.items():
        assert torch.equal(c.t[key][0].view(torch.uint8), val.view(torch.uint8)), key
    assert torch.equal(o[1].view(torch.int16), o_ref[1].view(torch.int16))
    assert torch.equal(ls[1], ls_ref[1])
    for key, val in c.t.items():
        if val is not None and key != "k4_pages":
            assert torch.equal(val[1].view(torch.uint8), ref.t[key][1].view(torch.uint8)), key
