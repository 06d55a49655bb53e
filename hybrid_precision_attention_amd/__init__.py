"""MI355X-native hybrid K4V4/FP16 decode attention (HyQuant's decode path).

The compute lives in libhq.so (hand-written HIP kernels for gfx950 behind a C
ABI, declared in include/hq.h); this package is the ctypes binding.
"""
from ._binding import (HQError, HybridCache, bind_decode, bind_merge, bind_step, HQ_OP_DECODE, HQ_OP_PREFILL,
                       HQ_OP_SELECT, hq_append_merge, hq_append_merge_ragged, hq_append_merge_scored,
                       hq_cache, hq_decode_attn, hq_decode_attn_noalloc, hq_decode_attn_ragged, hq_decode_step, hq_decode_step_ragged, hq_dims, hq_prefill_attn,
                       hq_quant_int8, hq_quant_pack, hq_refresh_hybrid, hq_select_vertical,
                       hq_status_string, hq_workspace_bytes, lib, make_dims, n_vertical, workspace)
from .model_cache import ModelCache, ModelShape, plan_capacity

__all__ = ["HQError", "HybridCache", "bind_decode", "bind_merge", "bind_step", "HQ_OP_DECODE", "HQ_OP_PREFILL",
           "HQ_OP_SELECT", "hq_append_merge", "hq_append_merge_ragged", "hq_append_merge_scored",
           "hq_cache", "hq_decode_attn", "hq_decode_attn_noalloc", "hq_decode_attn_ragged", "hq_decode_step", "hq_decode_step_ragged", "hq_dims", "hq_prefill_attn",
           "hq_quant_int8", "hq_quant_pack", "hq_refresh_hybrid", "hq_select_vertical",
           "hq_status_string", "hq_workspace_bytes", "lib", "make_dims", "n_vertical", "workspace",
           "ModelCache", "ModelShape", "plan_capacity"]
