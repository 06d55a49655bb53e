"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and bring its cache back in the oracle's per-unit form."""
import math

import numpy as np
import torch

import hybrid_precision_attention_amd as H
from oracle import hq_oracle as O

# decode-output tolerances (max-abs and relative L2 against the fp64 oracle)
MAX_ABS = 2e-3
REL_L2 = 1e-3
LSE_ABS = 1e-3


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_pack(x, L, W, rho, flags, L_max=None, extra_vl=0, k_bits=4, v_bits=4):
    """Pack the prefix with the HIP kernel; returns the HybridCache."""
    B, Hkv = x["K"].shape[:2]
    Hq = x["qbuf"].shape[1]
    cache = H.HybridCache.allocate(B, Hq, Hkv, W, rho, L_max if L_max is not None else L,
                                   extra_vl=extra_vl, k_bits=k_bits, v_bits=v_bits)
    K = dev(x["K"][:, :, :L]) if L else None
    V = dev(x["V"][:, :, :L]) if L else None
    F = dev(flags[:, :, :L]) if L else None
    H.hq_quant_pack(cache.dims, K, V, L, F, cache)
    torch.cuda.synchronize()
    return cache


def unit_from_gpu(cache, b, g):
    """One unit of the GPU cache as an oracle cache dict (valid rows only)."""
    pools = ("kq", "vq", "kq_meta", "vq_meta", "q_pos")
    t = {k: (v[b, g].cpu().numpy() if v is not None else None) for k, v in cache.t.items()
         if k not in pools and k != "k4_pages"}
    t.update({k: v.cpu().numpy() for k, v in zip(pools, cache.k4_unit(b, g))})
    n_q, n_vl, n_stg = int(t["n_q"]), int(t["n_vl"]), int(t["n_stg"])
    W = cache.dims.W
    c = O.empty_unit_cache(128, W, cache.dims.k_bits, cache.dims.v_bits)
    c["kq"], c["vq"] = t["kq"][:n_q], t["vq"][:n_q]
    c["kq_meta"], c["vq_meta"] = t["kq_meta"][:n_q], t["vq_meta"][:n_q]
    c["q_pos"] = t["q_pos"][:n_q]
    c["kvl"], c["vvl"], c["vl_pos"] = t["kvl"][:n_vl], t["vvl"][:n_vl], t["vl_pos"][:n_vl]
    if W:
        c["kwin"], c["vwin"] = t["kwin"], t["vwin"]
    c["kstg"], c["vstg"] = t["kstg"][:n_stg], t["vstg"][:n_stg]
    return c


def assert_unit_equal(gc, oc, L, W, tag=""):
    """Bit-exact comparison of one unit: K4V4 codes/meta/positions, vertical
    lines, the valid window slots, and the staged token."""
    for key in ("kq", "vq", "kq_meta", "vq_meta", "q_pos", "kvl", "vvl", "vl_pos"):
        a, b = gc[key], oc[key]
        assert a.shape == b.shape, f"{tag} {key} shape {a.shape} vs {b.shape}"
        if a.size:
            bad = np.nonzero(a.view(np.uint8).reshape(a.shape[0], -1)
                             != b.view(np.uint8).reshape(b.shape[0], -1))
            assert bad[0].size == 0, f"{tag} {key}: first mismatch row {bad[0][:5]}"
    if W:
        n_win = min(W, L)
        slots = np.arange(L - n_win, L) % W
        assert np.array_equal(gc["kwin"][slots].view(np.uint16), oc["kwin"][slots].view(np.uint16)), tag
        assert np.array_equal(gc["vwin"][slots].view(np.uint16), oc["vwin"][slots].view(np.uint16)), tag
    assert gc["kstg"].shape[0] == oc["kstg"].shape[0], tag
    assert np.array_equal(gc["kstg"].view(np.uint16), oc["kstg"].view(np.uint16)), tag
    assert np.array_equal(gc["vstg"].view(np.uint16), oc["vstg"].view(np.uint16)), tag


def check_decode(out_gpu, lse_gpu, out_ref, lse_ref, tag=""):
    o = out_gpu.astype(np.float64)
    err = np.abs(o - out_ref)
    rel = np.linalg.norm(o - out_ref) / max(np.linalg.norm(out_ref), 1e-300)
    assert err.max() <= MAX_ABS, f"{tag} max-abs {err.max():.3e}"
    assert rel <= REL_L2, f"{tag} rel-L2 {rel:.3e}"
    if lse_gpu is not None:
        le = np.abs(lse_gpu.astype(np.float64) - lse_ref).max()
        assert le <= LSE_ABS, f"{tag} lse max-abs {le:.3e}"
    return err.max(), rel


def gpu_decode(cache, L, q, lse=True):
    B, Hq = q.shape[:2]
    ws = H.workspace(cache.dims, H.HQ_OP_DECODE, L)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    lt = torch.empty((B, Hq), dtype=torch.float32, device="cuda") if lse else None
    H.hq_decode_attn(cache.dims, cache, L, dev(q), out, ws, lse=lt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lt.cpu().numpy() if lse else None)


def oracle_decode_on(cache, L, q, units=None):
    """Oracle decode over the GPU-produced cache (exactly dequantised)."""
    B, Hq = q.shape[:2]
    Hkv = cache.dims.Hkv
    G = Hq // Hkv
    out = np.full((B, Hq, 128), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in range(B):
        for g in range(Hkv):
            if units is not None and (b, g) not in units:
                continue
            c = unit_from_gpu(cache, b, g)
            out[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G] = O.decode_fused(
                c, q[b, g * G:(g + 1) * G], L)
    return out, lse


# Bound of a refresh's GPU score against the oracle's (the decode-time refresh
# feeds the matrix cores each dequantised K4V4 key element rounded to fp16).
SCORE_RTOL = 2e-5          # fp32 MFMA + exp2 of exact fp16 keys against fp64
U16 = 2.0 ** -11           # fp16 unit roundoff
SUB16 = 2.0 ** -25         # half the spacing of fp16 subnormals


def score_bounds(c, t, q, lse, lse_tol=0.0):
    """Per cached position i, a bound on |GPU - oracle| of one refresh's
    increment: sum over rows r (head, buffered query) of p_ri (exp(b_ri) - 1),
    where p_ri = exp(tau q_r.k_i - lse_r) on the oracle's exact keys (causal),
    b_ri = tau sum_e |q_re| (u |k_ie| + 2^-25) for a K4V4 key (the fp16
    rounding of its dequantised elements) and 0 for an FP16 key, plus lse_tol
    when the GPU's row normalisers differ from the oracle's by up to that.
    Returns (positions, bounds)."""
    G, nb, d = q.shape
    pos, keys = O.hybrid_keys(c, t)
    k4 = np.zeros(len(pos), bool)
    k4[:c["q_pos"].shape[0]] = True                     # K4V4 slots come first
    rows = t - nb + 1 + np.arange(nb)
    tau = 1.0 / math.sqrt(d)
    kabs = np.where(k4[:, None], U16 * np.abs(keys) + SUB16, 0.0)
    out = np.zeros(len(pos))
    for h in range(G):
        qh = q[h].astype(np.float64)
        z = tau * (qh @ keys.T)
        p = np.exp(z - lse[h][:, None]) * (pos[None, :] <= rows[:, None])
        beta = tau * (np.abs(qh) @ kabs.T) + lse_tol
        out += (p * np.expm1(beta)).sum(axis=0)
    return pos, out
