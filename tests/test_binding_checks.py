"""The binding's own checks, before any library call: the C ABI takes plain
pointers, so the binding compares every tensor's size with what the call
reads or writes, and a cache call's dims with the cache's buffers.  These
run on the CPU: each case fails its check before a pointer is taken."""
import pytest
import torch

import hybrid_precision_attention_amd as H
from hybrid_precision_attention_amd import _binding as Bd

B, Hq, Hkv, W, RHO, L = 2, 8, 2, 16, 0.1, 96


@pytest.fixture(scope="module")
def cache():
    return H.HybridCache.allocate(B, Hq, Hkv, W, RHO, L, device="cpu")


def h(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def test_token_and_query_sizes(cache):
    d = cache.dims
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="k_new holds"):
        H.hq_append_merge(d, cache, L, h(B, Hkv, 127), h(B, Hkv, 128))
    with pytest.raises(ValueError, match="evict_is_vl holds"):
        H.hq_append_merge(d, cache, L, h(B, Hkv, 128), h(B, Hkv, 128),
                          evict_is_vl=torch.zeros(B * Hkv - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="q holds"):
        H.hq_decode_attn(d, cache, L, h(B, Hq - 1, 128), h(B, Hq, 128), ws)
    with pytest.raises(ValueError, match="lse holds"):
        H.hq_decode_attn(d, cache, L, h(B, Hq, 128), h(B, Hq, 128), ws,
                         lse=torch.zeros(B * Hq - 1))
    with pytest.raises(ValueError, match="out holds"):
        H.hq_decode_step(d, cache, L, h(B, Hkv, 128), h(B, Hkv, 128), h(B, Hq, 128), h(B, Hq, 64), ws)
    with pytest.raises(ValueError, match="t_seq holds"):
        H.hq_decode_step_ragged(d, cache, torch.zeros(B - 1, dtype=torch.int32), L, h(B, Hkv, 128),
                                h(B, Hkv, 128), h(B, Hq, 128), h(B, Hq, 128), ws)
    with pytest.raises(ValueError, match="L_seq holds"):
        H.hq_decode_attn_ragged(d, cache, torch.zeros(B - 1, dtype=torch.int32), L, h(B, Hq, 128),
                                h(B, Hq, 128), ws)
    # every size right: the check passes and the CPU tensor is refused next
    with pytest.raises(ValueError, match="device tensor"):
        H.hq_decode_attn(d, cache, L, h(B, Hq, 128), h(B, Hq, 128), ws)


def test_prefix_sizes(cache):
    d = cache.dims
    with pytest.raises(ValueError, match="k holds"):
        H.hq_quant_pack(d, h(B, Hkv, L - 1, 128), h(B, Hkv, L, 128), L, None, cache)
    with pytest.raises(ValueError, match="vl_flag holds"):
        H.hq_quant_pack(d, h(B, Hkv, L, 128), h(B, Hkv, L, 128), L,
                        torch.zeros(B * Hkv * L - 1, dtype=torch.uint8), cache)
    sd = H.make_dims(B, Hq, Hkv, W, RHO)
    n_vl = H.n_vertical(RHO, L - W)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    args = dict(score=torch.zeros(B, Hkv, L), vl_idx=torch.zeros(B, Hkv, n_vl, dtype=torch.int32),
                vl_flag=torch.zeros(B, Hkv, L, dtype=torch.uint8))
    with pytest.raises(ValueError, match="qbuf must be"):
        H.hq_select_vertical(sd, h(B, Hq, 64), h(B, Hkv, L, 128), L, ws=ws, **args)
    with pytest.raises(ValueError, match="vl_idx holds"):
        H.hq_select_vertical(sd, h(B, Hq, 8, 128), h(B, Hkv, L, 128), L, args["score"],
                             torch.zeros(B, Hkv, n_vl - 1, dtype=torch.int32), args["vl_flag"], ws)
    with pytest.raises(ValueError, match="k holds"):
        H.hq_prefill_attn(sd, h(B, Hq, L, 128), h(B, Hkv, L, 64), h(B, Hkv, L, 128), L, None,
                          h(B, Hq, L, 128), ws)
    with pytest.raises(ValueError, match="lse holds"):
        H.hq_prefill_attn(sd, h(B, Hq, L, 128), h(B, Hkv, L, 128), h(B, Hkv, L, 128), L, None,
                          h(B, Hq, L, 128), ws, lse=torch.zeros(B, Hq, L - 1))


def test_dims_must_describe_the_cache(cache):
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    other = H.make_dims(B, Hq, Hkv, W, RHO, cap_q=cache.dims.cap_q + 32, cap_vl=cache.dims.cap_vl,
                        cap_stg=cache.dims.cap_stg)
    with pytest.raises(ValueError, match="cap_q"):
        H.hq_decode_attn(other, cache, L, h(B, Hq, 128), h(B, Hq, 128), ws)
    wide = H.make_dims(B, Hq, Hkv, W, RHO, cap_q=cache.dims.cap_q, cap_vl=cache.dims.cap_vl,
                       cap_stg=cache.dims.cap_stg, k_bits=8)
    with pytest.raises(ValueError, match="k_bits"):
        H.hq_append_merge(wide, cache, L, h(B, Hkv, 128), h(B, Hkv, 128))
    one = cache.view(1)
    with pytest.raises(ValueError, match="dims.B"):
        H.hq_append_merge(cache.dims, one, L, h(B, Hkv, 128), h(B, Hkv, 128))
    # unset widths (0) mean 4 bits, as in the C ABI
    same = H.make_dims(B, Hq, Hkv, W, RHO, cap_q=cache.dims.cap_q, cap_vl=cache.dims.cap_vl,
                       cap_stg=cache.dims.cap_stg, k_bits=0, v_bits=0)
    Bd._same_cache(same, cache)
