"""A model's hybrid caches, one per layer, and the batch capacity of one GPU.

The pages run whole models with one hybrid cache per layer (HyQuant README,
Quick Start: ``DStageKVCache(num_layers, k_bits, v_bits_fn, window_size,
top_ratio)``) and report the batch a 32K prefix allows on one GPU (agihunt
digest, results paragraph; README, Highlights).  The library's ABI is per
layer; this module only allocates the per-layer buffers (``HybridCache``),
keeps each layer's dims (its own value width through ``v_bits_fn``), and
does the byte arithmetic of a capacity plan.  Every cache operation runs in
libhq's kernels through the per-layer calls.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional

from ._binding import HybridCache, n_vertical

GROUP = 32


@dataclass(frozen=True)
class ModelShape:
    """Attention shape of a decoder: layers, query / KV heads, head_dim, and
    the bytes its weights take (16-bit), for a capacity plan."""
    name: str
    layers: int
    Hq: int
    Hkv: int
    d: int = 128
    weight_bytes: int = 0


# shapes of the models the pages evaluate (public configurations)
LLAMA31_8B = ModelShape("Llama-3.1-8B-shaped", 32, 32, 8, 128, 16_060_000_000)
QWEN3_8B = ModelShape("Qwen3-8B-shaped", 36, 32, 8, 128, 16_380_000_000)
QWEN3_32B = ModelShape("Qwen3-32B-shaped", 64, 64, 8, 128, 65_500_000_000)
GLM4_9B = ModelShape("GLM-4-9B-shaped", 40, 32, 2, 128, 18_800_000_000)


def layer_bytes_per_sequence(shape: ModelShape, L_max: int, W: int, rho: float, k_bits: int = 4,
                             v_bits: int = 4, extra_vl: int = 0, cap_stg: int = 1) -> int:
    """Bytes one sequence's hybrid cache takes in one layer, with the
    capacities ``HybridCache.allocate`` gives a prefix of up to L_max tokens:
    every non-window position may be quantised (codes, {scale, min} per group
    for K and V, position), the vertical-line region holds the top-rho set
    plus ``extra_vl`` promotions (fp16 K and V, position), the window ring and
    the staging slots are fp16, and three int32 counters."""
    d = shape.d
    n_nw = max(0, L_max - W)
    cap_q = max(1, n_nw)
    cap_vl = max(1, n_vertical(rho, n_nw) + extra_vl)
    q_tok = d * k_bits // 8 + d * v_bits // 8 + 2 * (d // GROUP) * 2 * 2 + 4
    f_tok = 2 * d * 2
    per_unit = cap_q * q_tok + cap_vl * (f_tok + 4) + W * f_tok + max(1, cap_stg) * f_tok + 3 * 4
    return shape.Hkv * per_unit


def cache_bytes_per_sequence(shape: ModelShape, L_max: int, W: int, rho: float, k_bits: int = 4,
                             v_bits_fn: Optional[Callable[[int], int]] = None, extra_vl: int = 0) -> int:
    vb = v_bits_fn or (lambda _l: 4)
    return sum(layer_bytes_per_sequence(shape, L_max, W, rho, k_bits, vb(l), extra_vl)
               for l in range(shape.layers))


def paged_layer_bytes_per_sequence(shape: ModelShape, L_seq: int, L_cap: int, W: int, rho: float,
                                   k_bits: int = 4, v_bits: int = 4, extra_vl: int = 0, cap_stg: int = 1) -> int:
    """Bytes one sequence of up to L_seq tokens takes in one layer of a
    paged cache whose longest sequence may reach L_cap
    (``HybridCache.allocate_paged``): K4V4 blocks of 32 slots only for its
    own non-window positions, plus its page table; the vertical-line region,
    window ring, staging slots and counters as in a contiguous cache of
    L_cap tokens."""
    d = shape.d
    n_nw_cap = max(0, L_cap - W)
    npb = max(1, -(-n_nw_cap // 32))
    blocks = -(-max(0, L_seq - W) // 32)
    cap_vl = max(1, n_vertical(rho, n_nw_cap) + extra_vl)
    q_tok = d * k_bits // 8 + d * v_bits // 8 + 2 * (d // GROUP) * 2 * 2 + 4
    f_tok = 2 * d * 2
    per_unit = (blocks * 32 * q_tok + npb * 4 + cap_vl * (f_tok + 4) + W * f_tok
                + max(1, cap_stg) * f_tok + 3 * 4)
    return shape.Hkv * per_unit


def fp16_cache_bytes_per_sequence(shape: ModelShape, L: int) -> int:
    """A plain fp16 K/V cache of L tokens over all layers."""
    return shape.layers * shape.Hkv * L * shape.d * 2 * 2


def plan_capacity(shape: ModelShape, L_max: int, W: int, rho: float, hbm_bytes: int,
                  reserve_bytes: int = 0, k_bits: int = 4,
                  v_bits_fn: Optional[Callable[[int], int]] = None, extra_vl: int = 0) -> dict:
    """Largest batch of L_max-token sequences whose hybrid caches fit next to
    the weights and a reserve, and the same for an fp16 cache."""
    free = hbm_bytes - shape.weight_bytes - reserve_bytes
    hyb = cache_bytes_per_sequence(shape, L_max, W, rho, k_bits, v_bits_fn, extra_vl)
    fp16 = fp16_cache_bytes_per_sequence(shape, L_max)
    return {"model": shape.name, "L": L_max, "hybrid_bytes_per_seq": hyb, "fp16_bytes_per_seq": fp16,
            "free_bytes": free, "max_batch_hybrid": max(0, free // hyb),
            "max_batch_fp16": max(0, free // fp16)}


class ModelCache:
    """Per-layer hybrid caches of a batch of B sequences of up to L_max
    tokens.  Layer l stores k_bits-bit keys and v_bits_fn(l)-bit values."""

    def __init__(self, shape: ModelShape, B: int, L_max: int, W: int, rho: float, k_bits: int = 4,
                 v_bits_fn: Optional[Callable[[int], int]] = None, extra_vl: int = 0,
                 device="cuda"):
        vb = v_bits_fn or (lambda _l: 4)
        self.shape, self.B, self.L_max, self.W, self.rho = shape, B, L_max, W, rho
        self.layers: List[HybridCache] = [
            HybridCache.allocate(B, shape.Hq, shape.Hkv, W, rho, L_max, extra_vl=extra_vl,
                                 device=device, k_bits=k_bits, v_bits=vb(l))
            for l in range(shape.layers)]

    def __len__(self) -> int:
        return len(self.layers)

    def __getitem__(self, l: int) -> HybridCache:
        return self.layers[l]

    def nbytes(self) -> int:
        return sum(c.nbytes() for c in self.layers)
