"""GPU parity of the other strict low-bit widths (K8V8, K4V2, K2V4 and the
rest of {2, 4, 8} x {2, 4, 8}) against the fp64 oracle: pack and merge
bit-exact (codes, {scale, min}, positions), decode within the same
tolerances as K4V4 (max-abs 2e-3, rel-L2 1e-3 against the oracle on the
GPU-built cache, exactly dequantised), and the decode-time refresh over
b-bit keys to the same 2e-5 as over K4V4 keys."""
import math

import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, workload
from oracle import hq_oracle as O

from gpu_util import (SCORE_RTOL, assert_unit_equal, check_decode, dev, gpu_decode, gpu_pack, oracle_decode_on,
                      score_bounds, unit_from_gpu)

pytestmark = pytest.mark.gpu

WIDTHS = [(8, 8), (4, 2), (2, 4), (2, 2), (8, 4), (4, 8), (2, 8), (8, 2)]


def _flags(wl, x):
    n_nw = max(0, wl.L - wl.W)
    n_vl = O.n_vertical(wl.rho, n_nw)
    f = np.zeros((wl.B, wl.Hkv, wl.L), np.uint8)
    for b in range(wl.B):
        f[b, :, x["plant"][b][:n_vl]] = 1
    return f


@pytest.mark.parametrize("kb,vb", WIDTHS, ids=[f"K{k}V{v}" for k, v in WIDTHS])
def test_pack_and_merge_bit_exact(kb, vb):
    wl = workload("tiny", L=1500)
    print(f"case K{kb}V{vb}", flush=True)
    T = 6
    x = batch(wl, steps=T)
    flags = _flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T, extra_vl=T, k_bits=kb, v_bits=vb)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags, kb, vb)
    for b in range(wl.B):
        for g in range(wl.Hkv):
            gc = unit_from_gpu(cache, b, g)
            assert gc["kq"].shape[1] == 16 * kb and gc["vq"].shape[1] == 16 * vb
            assert_unit_equal(gc, ref[b][g], wl.L, wl.W, tag=f"pack b{b} g{g}")
    for s in range(T):
        t = wl.L + s
        ev = np.full((wl.B, wl.Hkv), 1 if s == 3 else 0, np.uint8)
        H.hq_append_merge(cache.dims, cache, t, dev(x["k_dec"][s]), dev(x["v_dec"][s]), evict_is_vl=dev(ev))
        O.append_merge(ref, t, x["k_dec"][s], x["v_dec"][s], ev)
    torch.cuda.synchronize()
    for b in range(wl.B):
        for g in range(wl.Hkv):
            assert_unit_equal(unit_from_gpu(cache, b, g), ref[b][g], wl.L + T - 1, wl.W, tag=f"merge b{b} g{g}")


DECODE_CASES = [
    ("tiny", {}), ("llama31_8b", {"L": 4097}), ("qwen3_32b", {"B": 2, "L": 1800}),
    ("glm4_9b", {"B": 2, "L": 2000, "rho": 0.05}), ("tiny", {"W": 0, "rho": 0.0}), ("tiny", {"L": 40}),
]


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 2), (2, 4), (2, 2)], ids=["K8V8", "K4V2", "K2V4", "K2V2"])
@pytest.mark.parametrize("name,over", DECODE_CASES, ids=[f"{n}-{o}" for n, o in DECODE_CASES])
def test_decode_parity(name, over, kb, vb):
    wl = workload(name, **over)
    print(f"case {name} {over} K{kb}V{vb}", flush=True)
    x = batch(wl, steps=1)
    flags = _flags(wl, x) if wl.L else np.zeros((wl.B, wl.Hkv, 0), np.uint8)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + 1, k_bits=kb, v_bits=vb)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    q = x["q_dec"][0]
    out, lse = gpu_decode(cache, wl.L, q)
    ref, ref_lse = oracle_decode_on(cache, wl.L, q)
    check_decode(out, lse, ref, ref_lse, tag=f"{name} {over} K{kb}V{vb}")


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 2), (2, 4)], ids=["K8V8", "K4V2", "K2V4"])
def test_decode_full_size_llama_layer(kb, vb):
    """Llama-3.1-8B-shaped layer at a 32K prefix: every unit."""
    wl = workload("llama31_8b")
    print(f"case llama31_8b full K{kb}V{vb}", flush=True)
    x = batch(wl, steps=1)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, _flags(wl, x), L_max=wl.L + 1, k_bits=kb, v_bits=vb)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    q = x["q_dec"][0]
    out, lse = gpu_decode(cache, wl.L, q)
    ref, ref_lse = oracle_decode_on(cache, wl.L, q)
    check_decode(out, lse, ref, ref_lse, tag=f"full K{kb}V{vb}")


@pytest.mark.parametrize("kb", [2, 8])
def test_refresh_over_b_bit_keys(kb):
    """The decode-time refresh dequantises b-bit keys to fp16 like K4V4 ones."""
    wl = workload("llama31_8b", L=3000)
    print(f"case refresh K{kb}", flush=True)
    T = 2
    x = batch(wl, steps=T)
    flags = _flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T, k_bits=kb, v_bits=4)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags, kb, 4)
    for s in range(T):
        H.hq_append_merge(cache.dims, cache, wl.L + s, dev(x["k_dec"][s]), dev(x["v_dec"][s]))
        O.append_merge(ref, wl.L + s, x["k_dec"][s], x["v_dec"][s])
    t = wl.L + T - 1
    G, nb = wl.G, 64
    qb = np.ascontiguousarray(x["qbuf"])
    lse = np.full((wl.B, wl.Hq, nb), 7.0)
    n_vl = O.n_vertical(wl.rho, t - wl.W)
    score = torch.zeros((wl.B, wl.Hkv, t + 1), dtype=torch.float32, device="cuda")
    idx = torch.zeros((wl.B, wl.Hkv, n_vl), dtype=torch.int32, device="cuda")
    flag = torch.zeros((wl.B, wl.Hkv, t + 1), dtype=torch.uint8, device="cuda")
    cut = torch.zeros((wl.B, wl.Hkv), dtype=torch.float32, device="cuda")
    H.hq_refresh_hybrid(cache.dims, cache, t, dev(qb), dev(lse.astype(np.float32)), score, idx, flag, cut)
    torch.cuda.synchronize()
    sg = score.cpu().numpy()
    for b in range(wl.B):
        for g in range(wl.Hkv):
            so = np.zeros(t + 1)
            O.refresh_hybrid_unit(ref[b][g], t, qb[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G], wl.rho, so)
            # the bound of the fp16 rounding of each dequantised key element
            bpos, bnd = score_bounds(ref[b][g], t, qb[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G])
            tol = SCORE_RTOL * so
            tol[bpos] += bnd
            err = np.abs(sg[b, g] - so)
            assert np.all(err <= tol), f"b{b} g{g} err {np.max(err - tol):.2e} over the bound"
