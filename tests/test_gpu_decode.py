"""GPU parity of hq_decode_attn against the fp64 oracle run on the GPU-built
cache (exactly dequantised): max-abs <= 2e-3 and rel-L2 <= 1e-3 on the
output, 1e-3 on the logsumexp; bit-identical reruns."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import workload, batch
from oracle import hq_oracle as O

from gpu_util import assert_unit_equal, check_decode, dev, gpu_decode, gpu_pack, oracle_decode_on, unit_from_gpu

pytestmark = pytest.mark.gpu


def _setup(wl, T=1):
    x = batch(wl, steps=T)
    if wl.L:
        _, _, flags = O.select_vertical(x["K"], x["qbuf"], wl.L, wl.W, wl.rho)
    else:
        flags = np.zeros((wl.B, wl.Hkv, 0), np.uint8)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + T)
    return x, cache


CASES = [
    ("tiny", {}),
    ("llama31_8b", {"L": 4097}),
    ("qwen3_8b", {"B": 3, "L": 2500}),
    ("glm4_9b", {"B": 2, "L": 3000, "rho": 0.01}),
    ("glm4_9b", {"B": 2, "L": 1024, "rho": 0.10}),
    ("qwen3_32b", {"B": 2, "L": 1800}),
    ("tiny", {"L": 100}),
    ("tiny", {"L": 0}),                 # only the staged token
    ("tiny", {"L": 1}),
    ("tiny", {"W": 0}),
    ("tiny", {"W": 0, "rho": 0.0}),     # strict K4V4 (dequantise-then-attend)
    ("tiny", {"rho": 1.0}),             # full precision
    ("llama31_8b", {"L": 700, "W": 1000}),   # window covers the prefix
    ("tiny", {"Hq": 2}),                # G = 1: eight partials per output in the fold
    ("tiny", {"Hq": 4}),                # G = 2: four
    ("tiny", {"Hq": 6}),                # G = 3: two, met by a lane exchange
    ("tiny", {"Hq": 6, "L": 8192}),     # G = 3 with more than 32 splits: batches, LDS combine
    ("llama31_8b", {"L": 4097, "Hq": 24}),   # G = 3 at 8 KV heads
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{o}" for n, o in CASES])
def test_decode_parity(name, over):
    wl = workload(name, **over)
    print(f"case {name} {over}", flush=True)
    x, cache = _setup(wl)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    q = x["q_dec"][0]
    out, lse = gpu_decode(cache, wl.L, q)
    ref, ref_lse = oracle_decode_on(cache, wl.L, q)
    check_decode(out, lse, ref, ref_lse, tag=f"{name} {over}")


def test_decode_without_staged_token():
    """Right after the pack nothing is staged: the query sees the prefix only."""
    wl = workload("tiny", L=777)
    x, cache = _setup(wl)
    q = x["q_dec"][0]
    out, lse = gpu_decode(cache, wl.L, q)
    ref, ref_lse = oracle_decode_on(cache, wl.L, q)
    check_decode(out, lse, ref, ref_lse)


def test_decode_full_size_llama_layer():
    """The benchmark's launch configuration: B=1, 32/8 heads, L=32768."""
    wl = workload("llama31_8b")
    x, cache = _setup(wl)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(x["k_dec"][0]), dev(x["v_dec"][0]))
    q = x["q_dec"][0]
    out, lse = gpu_decode(cache, wl.L, q)
    ref, ref_lse = oracle_decode_on(cache, wl.L, q)
    check_decode(out, lse, ref, ref_lse)


def test_decode_deterministic():
    wl = workload("qwen3_8b", B=2, L=3000)
    x, cache = _setup(wl)
    q = x["q_dec"][0]
    a = gpu_decode(cache, wl.L, q)
    b = gpu_decode(cache, wl.L, q)
    assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_decode_streaming_steps():
    """Streaming decode (merge, then decode) stays within tolerance at steps
    0, 1, 63 and 127 of a Qwen3-32B-shaped run (reduced prefix and batch)."""
    wl = workload("qwen3_32b", B=2, L=2000)
    T = 128
    x, cache = _setup(wl, T=T)
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, wl.L + T)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    for t in range(T):
        pos = wl.L + t
        H.hq_append_merge(cache.dims, cache, pos, dev(x["k_dec"][t]), dev(x["v_dec"][t]))
        H.hq_decode_attn(cache.dims, cache, pos, dev(x["q_dec"][t]), out, ws, lse=lse)
        if t in (0, 1, 63, 127):
            torch.cuda.synchronize()
            ref, ref_lse = oracle_decode_on(cache, pos, x["q_dec"][t])
            check_decode(out.cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, tag=f"step {t}")


def test_step_full_size_llama_layer():
    """hq_decode_step in the benchmark's launch configuration (B=1, 32/8
    heads, L=32768): two steps equal, bit for bit, hq_append_merge +
    hq_decode_attn on a copy of the cache, which the oracle checks."""
    wl = workload("llama31_8b")
    T = 2
    x, c1 = _setup(wl, T=T)
    c2 = c1.clone()
    ws1 = H.workspace(c1.dims, H.HQ_OP_DECODE, wl.L + T)
    ws2 = H.workspace(c2.dims, H.HQ_OP_DECODE, wl.L + T)
    o1 = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    o2 = torch.empty_like(o1)
    l1 = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    for s in range(T):
        t = wl.L + s
        k, v, q = dev(x["k_dec"][s]), dev(x["v_dec"][s]), dev(x["q_dec"][s])
        H.hq_decode_step(c1.dims, c1, t, k, v, q, o1, ws1, lse=l1)
        H.hq_append_merge(c2.dims, c2, t, k, v)
        H.hq_decode_attn(c2.dims, c2, t, q, o2, ws2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"step {s}"
        assert torch.equal(l1, l2), f"step {s}"
        ref, ref_lse = oracle_decode_on(c2, t, x["q_dec"][s])
        check_decode(o2.cpu().numpy(), l2.cpu().numpy(), ref, ref_lse, tag=f"step {s}")


def test_decode_full_size_qwen3_8b_batch32_sampled():
    """The batch sweep's largest launch: Qwen3-8B-shaped layer, B=32,
    L=32768 (256 units, the split plan of that size).  Four seeded sequences
    are tiled over the batch (units are independent); the oracle checks
    sampled units, one from each tile group and head."""
    wl = workload("qwen3_8b")
    assert wl.B == 32 and wl.L == 32768
    xs = batch(wl, steps=1, seqs=[0, 1, 2, 3])
    _, _, f4 = O.select_vertical(xs["K"], xs["qbuf"], wl.L, wl.W, wl.rho)
    rep = wl.B // 4
    x = {"K": np.concatenate([xs["K"]] * rep), "V": np.concatenate([xs["V"]] * rep),
         "qbuf": np.concatenate([xs["qbuf"]] * rep)}
    flags = np.concatenate([f4] * rep)
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, flags, L_max=wl.L + 1)
    del x
    k_new = np.concatenate([xs["k_dec"][0]] * rep)
    v_new = np.concatenate([xs["v_dec"][0]] * rep)
    q = np.concatenate([xs["q_dec"][0]] * rep)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(k_new), dev(v_new))
    out, lse = gpu_decode(cache, wl.L, q)
    units = [(0, 0), (5, 3), (18, 6), (31, 7)]
    ref, ref_lse = oracle_decode_on(cache, wl.L, q, units=units)
    G = wl.G
    # the output bound applies to the checked output as a whole (the sampled
    # units together), as it applies to a whole call's output elsewhere
    pick = lambda a: np.stack([a[b, g * G:(g + 1) * G] for b, g in units])
    check_decode(pick(out), pick(lse), pick(ref), pick(ref_lse), tag="sampled units")


@pytest.mark.parametrize("name,seqs,units,rho", [
    # Qwen3-32B-shaped, B=32, 64/8 heads (G = 8, the general path): four
    # seeded sequences tiled over the batch, one sampled unit per tile group
    ("qwen3_32b", [0, 1, 2, 3], [(0, 0), (9, 2), (22, 5), (31, 7)], 0.05),
    # GLM-4-9B-shaped, B=8, 32/2 heads (G = 16): every sequence its own seed,
    # at the grid's three line ratios
    ("glm4_9b", list(range(8)), [(0, 0), (3, 1), (6, 0), (7, 1)], 0.05),
    ("glm4_9b", list(range(8)), [(1, 0), (2, 1), (5, 1), (7, 0)], 0.01),
    ("glm4_9b", list(range(8)), [(0, 1), (4, 0), (6, 1), (7, 1)], 0.10),
])
def test_decode_full_size_sampled(name, seqs, units, rho):
    """The streaming and GQA-16 runs' decode at full size (L=32768, the
    split plan of that launch), checked by the oracle on sampled units."""
    wl = workload(name, rho=rho)
    print(f"case {name} rho={rho}", flush=True)
    assert wl.L == 32768
    xs = batch(wl, steps=1, seqs=seqs)
    _, _, f = O.select_vertical(xs["K"], xs["qbuf"], wl.L, wl.W, wl.rho)
    rep = wl.B // len(seqs)
    x = {"K": np.concatenate([xs["K"]] * rep), "V": np.concatenate([xs["V"]] * rep),
         "qbuf": np.concatenate([xs["qbuf"]] * rep)}
    cache = gpu_pack(x, wl.L, wl.W, wl.rho, np.concatenate([f] * rep), L_max=wl.L + 1)
    del x
    k_new = np.concatenate([xs["k_dec"][0]] * rep)
    v_new = np.concatenate([xs["v_dec"][0]] * rep)
    q = np.concatenate([xs["q_dec"][0]] * rep)
    H.hq_append_merge(cache.dims, cache, wl.L, dev(k_new), dev(v_new))
    out, lse = gpu_decode(cache, wl.L, q)
    ref, ref_lse = oracle_decode_on(cache, wl.L, q, units=units)
    G = wl.G
    pick = lambda a: np.stack([a[b, g * G:(g + 1) * G] for b, g in units])
    check_decode(pick(out), pick(lse), pick(ref), pick(ref_lse), tag=f"{name} sampled units")


def test_streaming_full_size_qwen3_32b_sampled():
    """The benchmark's streaming run at full size: Qwen3-32B-shaped layer,
    B=32, 64/8 heads, L0=32768, W=128, rho=5%, 128 hq_decode_step calls.
    Four seeded sequences (prefix and decode tokens) are tiled over the batch
    (units are independent); the oracle packs and streams the sampled units on
    its own.  Outputs at steps 0, 1, 63 and 127 within the decode tolerance;
    after one more plain merge on both sides, the sampled units' caches are
    bit-exact."""
    wl = workload("qwen3_32b")
    assert wl.B == 32 and wl.L == 32768 and wl.Hq == 64 and wl.Hkv == 8
    T, L, W, G = 128, wl.L, wl.W, wl.G
    print("case qwen3_32b streaming, full size", flush=True)
    xs = batch(wl, steps=T + 1, seqs=[0, 1, 2, 3])
    _, _, f4 = O.select_vertical(xs["K"], xs["qbuf"], L, W, wl.rho)
    rep = wl.B // 4
    tile = lambda a: np.ascontiguousarray(np.concatenate([a] * rep))
    x = {"K": tile(xs["K"]), "V": tile(xs["V"]), "qbuf": tile(xs["qbuf"])}
    cache = gpu_pack(x, L, W, wl.rho, tile(f4), L_max=L + T + 1)
    del x
    units = [(0, 0), (9, 2), (22, 5), (31, 7)]
    refs = {(b, g): O.quant_pack_unit(xs["K"][b % 4, g], xs["V"][b % 4, g], L, W, f4[b % 4, g])
            for b, g in units}
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, L + T)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    for s in range(T):
        t = L + s
        q = tile(xs["q_dec"][s])
        H.hq_decode_step(cache.dims, cache, t, dev(tile(xs["k_dec"][s])), dev(tile(xs["v_dec"][s])), dev(q),
                         out, ws, lse=lse)
        for b, g in units:
            O.append_merge_unit(refs[(b, g)], t, xs["k_dec"][s, b % 4, g], xs["v_dec"][s, b % 4, g])
        if s in (0, 1, 63, 127):
            torch.cuda.synchronize()
            o, lg = out.cpu().numpy(), lse.cpu().numpy()
            ro, rl = zip(*(O.decode_fused(refs[(b, g)], q[b, g * G:(g + 1) * G], t) for b, g in units))
            pick = lambda a: np.stack([a[b, g * G:(g + 1) * G] for b, g in units])
            check_decode(pick(o), pick(lg), np.stack(ro), np.stack(rl), tag=f"step {s}")
    t = L + T
    H.hq_append_merge(cache.dims, cache, t, dev(tile(xs["k_dec"][T])), dev(tile(xs["v_dec"][T])))
    for b, g in units:
        O.append_merge_unit(refs[(b, g)], t, xs["k_dec"][T, b % 4, g], xs["v_dec"][T, b % 4, g])
    torch.cuda.synchronize()
    for b, g in units:
        assert_unit_equal(unit_from_gpu(cache, b, g), refs[(b, g)], t, W, tag=f"b{b} g{g}")



def test_step_large_batch_64bit_offsets():
    """Byte offsets past 2^31 in the K4V4 arrays: the Qwen3-8B-shaped layer
    at B=160, L=32768 (1280 units, so kq and vq each hold 2.67 GB), built by
    hq_quant_pack, stepped once by hq_decode_step and then given one plain
    merge.  Four seeded sequences are tiled on the device; the oracle packs
    and merges sampled units on its own, the last unit at the highest
    offsets.  The step's outputs lie within the decode tolerance and the
    sampled units' caches are bit-exact at the end."""
    wl = workload("qwen3_8b", B=160)
    L, W, G = wl.L, wl.W, wl.G
    print("case qwen3_8b B=160, 64-bit offsets", flush=True)
    xs = batch(wl, steps=2, seqs=[0, 1, 2, 3])
    _, _, f4 = O.select_vertical(xs["K"], xs["qbuf"], L, W, wl.rho)
    rep = wl.B // 4
    cache = H.HybridCache.allocate(wl.B, wl.Hq, wl.Hkv, W, wl.rho, L + 2)
    kq = cache.t["kq"]
    assert kq.numel() * kq.element_size() > 2 ** 31
    K = dev(xs["K"]).repeat(rep, 1, 1, 1)
    V = dev(xs["V"]).repeat(rep, 1, 1, 1)
    F = dev(f4).repeat(rep, 1, 1)
    H.hq_quant_pack(cache.dims, K, V, L, F, cache)
    del K, V, F
    tile = lambda a: np.ascontiguousarray(np.concatenate([a] * rep))
    q = tile(xs["q_dec"][0])
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, L + 1)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    H.hq_decode_step(cache.dims, cache, L, dev(tile(xs["k_dec"][0])), dev(tile(xs["v_dec"][0])), dev(q),
                     out, ws, lse=lse)
    H.hq_append_merge(cache.dims, cache, L + 1, dev(tile(xs["k_dec"][1])), dev(tile(xs["v_dec"][1])))
    torch.cuda.synchronize()
    units = [(0, 0), (81, 5), (130, 2), (159, 7)]
    refs = {(b, g): O.quant_pack_unit(xs["K"][b % 4, g], xs["V"][b % 4, g], L, W, f4[b % 4, g])
            for b, g in units}
    for b, g in units:
        O.append_merge_unit(refs[(b, g)], L, xs["k_dec"][0, b % 4, g], xs["v_dec"][0, b % 4, g])
    ro, rl = zip(*(O.decode_fused(refs[(b, g)], q[b, g * G:(g + 1) * G], L) for b, g in units))
    o, lg = out.cpu().numpy(), lse.cpu().numpy()
    pick = lambda a: np.stack([a[b, g * G:(g + 1) * G] for b, g in units])
    check_decode(pick(o), pick(lg), np.stack(ro), np.stack(rl), tag="B=160 sampled units")
    for b, g in units:
        O.append_merge_unit(refs[(b, g)], L + 1, xs["k_dec"][1, b % 4, g], xs["v_dec"][1, b % 4, g])
        assert_unit_equal(unit_from_gpu(cache, b, g), refs[(b, g)], L + 1, W, tag=f"b{b} g{g}")
