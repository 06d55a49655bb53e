"""Host-side checks of the multi-layer cache and the capacity plan (no GPU:
the buffers are allocated on the CPU, no kernel runs)."""
import ctypes

import pytest

import hybrid_precision_attention_amd as H
from hybrid_precision_attention_amd import model_cache as M
from hybrid_precision_attention_amd import _binding as B


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 8), (2, 4), (4, 2)])
def test_plan_bytes_match_the_allocation(kb, vb):
    shape = M.ModelShape("small", 3, 8, 2, 128)
    mc = H.ModelCache(shape, 2, 1500, 64, 0.05, k_bits=kb, v_bits_fn=lambda l: vb, device="cpu")
    assert len(mc) == 3
    want = 2 * M.cache_bytes_per_sequence(shape, 1500, 64, 0.05, kb, lambda l: vb)
    assert mc.nbytes() == want


def test_per_layer_value_widths():
    shape = M.ModelShape("small", 4, 8, 2, 128)
    mc = H.ModelCache(shape, 1, 600, 32, 0.1, v_bits_fn=lambda l: 2 if l % 2 else 4, device="cpu")
    assert [c.dims.v_bits for c in mc.layers] == [4, 2, 4, 2]
    assert [c.t["vq"].shape[-1] for c in mc.layers] == [64, 32, 64, 32]
    assert all(c.dims.k_bits == 4 for c in mc.layers)


def test_capacity_plan_32k():
    """Qwen3-8B-shaped, 32K prefix, W = 128, rho = 5 %: the K4V4 hybrid cache
    as allocated (every non-window position may be quantised, positions
    stored) is 0.373x of an fp16 cache (0.349x algorithmic), so about 2.6x
    the batch fits."""
    plan = M.plan_capacity(M.QWEN3_8B, 32768, 128, 0.05, hbm_bytes=288 * 10 ** 9)
    ratio = plan["hybrid_bytes_per_seq"] / plan["fp16_bytes_per_seq"]
    assert 0.37 < ratio < 0.38
    assert plan["max_batch_hybrid"] >= 2.6 * plan["max_batch_fp16"]
    # an 80 GB GPU: the fp16 cache fits 12 sequences next to the weights, the
    # hybrid one 35
    p80 = M.plan_capacity(M.QWEN3_8B, 32768, 128, 0.05, hbm_bytes=80 * 10 ** 9)
    assert p80["max_batch_fp16"] < 16 <= p80["max_batch_hybrid"]


def test_view_is_one_sequence():
    c = H.HybridCache.allocate(3, 8, 2, 32, 0.05, 500, device="cpu")
    v = c.view(1)
    assert v.dims.B == 1 and v.dims.Hkv == 2
    assert v.t["kq"].data_ptr() == c.t["kq"][1].data_ptr()
    assert v.t["n_q"].shape == (1, 2)


P = 1 << 24


def test_ragged_validation():
    d = B.make_dims(2, 32, 8, 128, 0.05, 32640, 1632, 1)
    c = B.hq_cache()
    for i, (n, _) in enumerate(B.hq_cache._fields_):
        setattr(c, n, (1 << 20) + 4096 * i)
    f = H.lib.hq_decode_attn_ragged
    need = H.hq_workspace_bytes(d, H.HQ_OP_DECODE, 32768)
    assert f(ctypes.byref(d), ctypes.byref(c), None, 100, P, P, None, P, need, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(c), P, -1, P, P, None, P, need, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(c), P + 4, 100, P, P, None, P, need, None) == -3
    assert f(ctypes.byref(d), ctypes.byref(c), P, 100, P, P, None, None, need, None) == -5
    g = H.lib.hq_append_merge_ragged
    assert g(ctypes.byref(d), ctypes.byref(c), None, 100, P, P, None, None) == -1
    assert g(ctypes.byref(d), ctypes.byref(c), P, 40000, P, P, None, None) == -4   # cap_q < t_max - W


def test_paged_bytes_match_a_paged_allocation():
    """The paged byte model equals what HybridCache.allocate_paged allocates
    (on the CPU): per-sequence blocks, the shared spare block aside."""
    import hybrid_precision_attention_amd as H
    from hybrid_precision_attention_amd.model_cache import paged_layer_bytes_per_sequence, ModelShape
    shape = ModelShape("toy", 1, 8, 2, 128, 0)
    lens = [1500, 300, 60]
    L_cap = 1600
    c = H.HybridCache.allocate_paged(3, 8, 2, 128, 0.05, L_cap, extra_vl=3, seq_L_max=lens, device="cpu")
    spare = 32 * (64 + 64 + 16 + 16 + 4)            # one spare block of the pool (K4V4 rows and positions)
    want = sum(paged_layer_bytes_per_sequence(shape, Lb, L_cap, 128, 0.05, extra_vl=3) for Lb in lens)
    assert c.nbytes() - spare == want
    # a short sequence pays for its own K4V4 blocks only (the window and the
    # line region are sized by the cap for every sequence)
    assert paged_layer_bytes_per_sequence(shape, 300, L_cap, 128, 0.05) < \
        paged_layer_bytes_per_sequence(shape, 1500, L_cap, 128, 0.05) / 2
