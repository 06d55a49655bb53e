"""GPU parity of hq_quant_pack and hq_append_merge: bit-exact against the
oracle on the same seeded inputs (codes, {scale, min}, positions, vertical
lines, window ring, staging, counters)."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import workload, batch
from oracle import hq_oracle as O

from gpu_util import assert_unit_equal, dev, gpu_pack, unit_from_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # name, overrides, steps
    ("tiny", {}),
    ("llama31_8b", {"L": 3001}),
    ("qwen3_8b", {"B": 2, "L": 2050}),
    ("glm4_9b", {"B": 2, "L": 1500, "rho": 0.10}),
    ("qwen3_32b", {"B": 2, "L": 1333}),
    ("tiny", {"L": 100}),              # prefix shorter than the window
    ("tiny", {"L": 128}),              # prefix exactly the window
    ("tiny", {"W": 0}),                # no window: strict low-bit + lines
    ("tiny", {"rho": 0.0, "W": 0}),    # strict K4V4
    ("tiny", {"rho": 1.0}),            # every non-window token FP16
    ("tiny", {"L": 1}),
    ("tiny", {"L": 0}),
]


def _flags(wl, x):
    if wl.L == 0:
        return np.zeros((wl.B, wl.Hkv, 0), np.uint8)
    _, _, f = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    return f


@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{o}" for n, o in CASES])
def test_pack_bit_exact(name, over):
    wl = workload(name, **over)
    print(f"case {name} {over}", flush=True)
    x = batch(wl, steps=1)
    flags = _flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags)
    for b in range(wl.B):
        for g in range(wl.Hkv):
            gc = unit_from_gpu(cache, b, g)
            assert int(cache.t["n_stg"][b, g]) == 0
            assert_unit_equal(gc, ref[b][g], wl.L, wl.W, tag=f"b{b} g{g}")


def test_pack_full_size_llama_layer():
    """Llama-3.1-8B-shaped layer at full size (L = 32768): every unit."""
    wl = workload("llama31_8b")
    x = batch(wl, steps=1)
    flags = _flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags)
    for g in range(wl.Hkv):
        assert int(cache.t["n_vl"][0, g]) == 1632 and int(cache.t["n_q"][0, g]) == 31008
        assert_unit_equal(unit_from_gpu(cache, 0, g), ref[0][g], wl.L, wl.W, tag=f"g{g}")


def test_pack_vertical_overflow_goes_to_k4():
    """Flagged positions beyond the vertical-line capacity are stored as K4V4."""
    wl = workload("tiny", L=600)
    x = batch(wl, steps=1)
    flags = np.zeros((1, wl.Hkv, wl.L), np.uint8)
    flags[:, :, 10:60:2] = 1                                # 25 flags
    cache = H.HybridCache.allocate(1, wl.Hq, wl.Hkv, wl.W, 0.01, wl.L)   # cap_vl = 4
    cap_vl = cache.dims.cap_vl
    H.hq_quant_pack(cache.dims, dev(x["K"]), dev(x["V"]), wl.L, dev(flags), cache)
    torch.cuda.synchronize()
    eff = flags.copy()
    for g in range(wl.Hkv):
        on = np.nonzero(eff[0, g])[0]
        eff[0, g, on[cap_vl:]] = 0
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, eff)
    for g in range(wl.Hkv):
        assert int(cache.t["n_vl"][0, g]) == cap_vl
        assert_unit_equal(unit_from_gpu(cache, 0, g), ref[0][g], wl.L, wl.W)


def test_quantiser_special_groups():
    """Groups with subnormal, zero and constant ranges, exact ties, large
    magnitudes and -0: the GPU codes and meta equal the oracle's."""
    L, W = 64, 0
    rng = np.random.default_rng(0)
    K = np.zeros((1, 1, L, 128), np.float16)
    K[0, 0, 0] = 3.0                                          # constant
    K[0, 0, 1, :32] = np.array([0, 15] + [k + 0.5 for k in range(15)] + [7] * 15, np.float16)
    K[0, 0, 2, :4] = np.array([0, 22 * 2.0 ** -24, 11 * 2.0 ** -24, 2.0 ** -24], np.float16)
    K[0, 0, 3, :2] = np.array([0, 7 * 2.0 ** -24], np.float16)
    K[0, 0, 4] = np.float16(-0.0)
    K[0, 0, 5, :64] = np.float16(60000)
    K[0, 0, 5, 64:] = np.float16(-60000)
    K[0, 0, 6:] = (rng.standard_normal((L - 6, 128)) * rng.uniform(1e-5, 100, (L - 6, 1))).astype(np.float16)
    V = K[:, :, ::-1].copy()
    x = {"K": K, "V": V, "qbuf": np.zeros((1, 1, 1, 128), np.float16)}
    flags = np.zeros((1, 1, L), np.uint8)
    cache = gpu_pack(x, L, W, 0.0, flags)
    ref = O.quant_pack(K, V, L, W, flags)
    assert_unit_equal(unit_from_gpu(cache, 0, 0), ref[0][0], L, W)


@pytest.mark.parametrize("name,over,T,ev_every", [
    ("tiny", {}, 40, 0),
    ("tiny", {"L": 60}, 100, 0),          # window fills up while streaming
    ("tiny", {"W": 0}, 20, 0),
    ("tiny", {}, 30, 7),                  # every 7th leaving token promoted to FP16
    ("qwen3_32b", {"B": 2, "L": 700}, 12, 0),
])
def test_merge_streaming_bit_exact(name, over, T, ev_every):
    wl = workload(name, **over)
    print(f"case {name} {over} T={T}", flush=True)
    x = batch(wl, steps=T)
    flags = _flags(wl, x)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T, extra_vl=T)
    ref = O.quant_pack(x["K"], x["V"], wl.L, wl.W, flags)
    # the oracle's VL region has no capacity limit; the GPU one has room for T
    for t in range(T):
        pos = wl.L + t
        ev = None
        if ev_every and t % ev_every == 3:
            ev = np.ones((wl.B, wl.Hkv), np.uint8)
        H.hq_append_merge(cache.dims, cache, pos, dev(x["k_dec"][t]), dev(x["v_dec"][t]),
                          evict_is_vl=dev(ev) if ev is not None else None)
        O.append_merge(ref, pos, x["k_dec"][t], x["v_dec"][t], ev)
        if t in (0, 1, T // 2, T - 1):
            torch.cuda.synchronize()
            for b in range(wl.B):
                for g in range(wl.Hkv):
                    gc = unit_from_gpu(cache, b, g)
                    assert int(cache.t["n_stg"][b, g]) == 1
                    assert_unit_equal(gc, ref[b][g], pos, wl.W, tag=f"t{t} b{b} g{g}")


def _tie_rows(n_tok, bits, seed):
    """fp16 token rows whose groups put many values exactly on, or just
    beside, half-integer quotients (x - min) / scale: the float32 estimate of
    the quantiser must hand those to the exact decision."""
    rng = np.random.default_rng(seed)
    qmax = 2 ** bits - 1
    X = np.zeros((n_tok, 128), np.float64)
    scales = [2.0 ** -8, 1.0, 4.0, 2.0 ** -12]
    mins = [0.0, -0.75, 0.5]
    for t in range(n_tok):
        for g in range(4):
            s = scales[(t + g) % len(scales)]
            m = mins[(3 * t + g) % len(mins)] * s
            k = rng.integers(0, qmax, 32).astype(np.float64)
            off = rng.choice([0.5, 0.5, 0.5, 0.0, 0.5 + 2.0 ** -7, 0.5 - 2.0 ** -7], 32)
            v = m + (k + off) * s
            v[0], v[1] = m, m + qmax * s
            X[t, 32 * g:32 * g + 32] = v
    return X.astype(np.float16)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_and_merge_tie_rich_groups(bits):
    """Pack (W = 0: every token quantised) and streamed merges of tie-rich
    tokens, K and V at the same width: codes, scales and minimums bit-exact
    against the oracle."""
    L, T = 300, 40
    K = _tie_rows(L + T, bits, 1)
    V = _tie_rows(L + T, bits, 2)
    x = {"K": K[None, None], "V": V[None, None], "qbuf": np.zeros((1, 1, 1, 128), np.float16)}
    flags = np.zeros((1, 1, L + T), np.uint8)
    cache = gpu_pack(x, L, 0, 0.0, flags, L_max=L + T + 1, k_bits=bits, v_bits=bits)
    ref = O.quant_pack_unit(K[:L], V[:L], L, 0, flags[0, 0, :L], bits, bits)
    for t in range(L, L + T):
        H.hq_append_merge(cache.dims, cache, t, dev(K[None, None, t]), dev(V[None, None, t]))
        O.append_merge_unit(ref, t, K[t], V[t])
    torch.cuda.synchronize()
    assert_unit_equal(unit_from_gpu(cache, 0, 0), ref, L + T - 1, 0, tag=f"{bits}-bit")
