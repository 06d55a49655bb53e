"""GPU check of hq_decode_attn_noalloc (the decode for callers that cannot
allocate: its counters and partial records in the library's static per-GPU
scratch) against hq_decode_attn with a caller workspace, through the C ABI:
bit-equal outputs and LSE, and within the decode tolerance of the fp64
oracle, on consecutive calls of different sizes (the second one smaller)."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, workload
from oracle import hq_oracle as O

from gpu_util import check_decode, dev, gpu_pack, oracle_decode_on

pytestmark = pytest.mark.gpu


def _case(name, **over):
    wl = workload(name, **over)
    x = batch(wl, steps=1)
    n_nw = max(0, wl.L - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    flags = np.zeros((wl.B, wl.Hkv, wl.L), np.uint8)
    for b in range(wl.B):
        pl = x["plant"][b]
        flags[b, :, pl[pl < n_nw][:n_vl]] = 1
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + 2)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    torch.cuda.synchronize()
    return wl, x, cache


def _run(wl, x, cache, units):
    L = wl.L
    q = dev(x["q_dec"][0])
    shape = (wl.B, wl.Hq, 128)
    o_ws = torch.empty(shape, dtype=torch.float16, device="cuda")
    o_na = torch.full(shape, 7.0, dtype=torch.float16, device="cuda")
    l_ws = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    l_na = torch.full((wl.B, wl.Hq), 7.0, dtype=torch.float32, device="cuda")
    H.hq_decode_attn(cache.dims, cache, L, q, o_ws, H.workspace(cache.dims, H.HQ_OP_DECODE, L), lse=l_ws)
    H.hq_decode_attn_noalloc(cache.dims, cache, L, q, o_na, lse=l_na)
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
    assert torch.equal(l_na, l_ws)
    ref, ref_lse = oracle_decode_on(cache, L, x["q_dec"][0], units=units)
    G = wl.G
    pick = lambda a: np.concatenate([a[b, g * G:(g + 1) * G].reshape(-1) for b, g in units])
    check_decode(pick(o_na.cpu().numpy()), pick(l_na.cpu().numpy()), pick(ref), pick(ref_lse), tag="noalloc")


def test_noalloc_decode_matches_workspace_decode():
    # a Llama-shaped layer at an 8K prefix, then the smaller tiny layer, then
    # a two-sequence GQA-8 layer: the counters of each call start at zero
    for name, over, units in (("llama31_8b", {"L": 8192}, [(0, 0), (0, 5)]),
                              ("tiny", {}, [(0, 0), (0, 1)]),
                              ("qwen3_32b", {"B": 2, "L": 3000}, [(0, 2), (1, 7)])):
        print(f"case {name} {over}", flush=True)
        wl, x, cache = _case(name, **over)
        _run(wl, x, cache, units)
