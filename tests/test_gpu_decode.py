"""GPU parity of hq_decode_attn against the fp64 oracle run on the GPU-built
cache (exactly dequantised): max-abs <= 2e-3 and rel-L2 <= 1e-3 on the
output, 1e-3 on the logsumexp; bit-identical reruns."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import workload, batch
from oracle import hq_oracle as O

from gpu_util import check_decode, dev, gpu_decode, gpu_pack, oracle_decode_on

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
