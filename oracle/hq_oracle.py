"""Plain fp64 CPU oracle of HyQuant's decode-time hybrid K4V4/FP16 attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The GPU library
never calls it, and it shares no code with the GPU path: it is written from
the method's description, slowly and in float64, so that a reader can check
each step against the pages by eye.

Sources (page title, then the passage):
  [D]  agihunt.info digest "HyQuant: Hybrid-Precision Quantization for LLM
       Attention" -- method paragraph (three-way key partition, column-mass
       score, top-rho over the non-window prefix, <=64 buffered FP16 queries,
       refresh every 64 tokens) and decode paragraph (fused dequantisation in
       the attention scan, vertical lines fixed after the prefill tail, new
       tokens staged then merged into the hybrid layout).
  [R]  HyQuant README (gitlite.dev mirror) -- "Overview" items 1 and 3
       (running column-mass score; K4V4 + FP16 vertical-line/window cache with
       an online softmax over quantised blocks), "Overhead" (query-buffer
       size, ~15 % KV growth), "Mode reference" (dense / strict low-bit /
       hybrid_full modes, window_size and top_ratio).
  [H]  Hugging Face paper page mirror -- author comment (top-5 % keys plus a
       128-token window; FP16 vertical lines and window, the rest K4V4).

Readings where the pages are silent (each is listed with its reason in the
design notes): softmax scale 1/sqrt(d); column mass = softmax probabilities
of each buffered query's full causal row, summed over the query heads of a
KV group and over the buffered queries, kept for non-window columns only;
n_vl = floor(rho * |non-window| + 1e-6); ties at the cut-off go to the lower
position; the K4V4 group layout is asymmetric uint4 over groups of 32
consecutive head_dim elements of one token, fp16 {scale, min} per group,
scale = fp16(range / 15), codes = round-half-even((x - min) / scale) clamped
to [0, 15] (all codes 0 when the scale is 0), two codes per byte with the
lower-index element in the low nibble; the other strict low-bit widths of
the mode table (K8V8, K4V2, K2V4) use the same rule with 2^b - 1 steps and
8/b codes per byte, lowest-index element in the lowest bits, K and V widths
chosen independently; the decode token is not part of the window -- it sits
in an FP16 staging slot and attends to itself; the prefill's low-bit QK is
symmetric INT8 per token row (scale fp32(amax/127), code round-half-even of
127 x / amax), its FP16 keys are the vertical lines and each query's own
W-window, and its P V is FP16 for every key.

Parity unpinned: none of the functions below; every one has a pin in
tests/test_oracle_*.py (closed forms, brute force, library routines).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

GROUP = 32          # head_dim elements per quantisation group
QMAX = 15           # largest 4-bit code
KV_BITS = (2, 4, 8) # code widths of the strict low-bit caches [R Mode reference]
NB_MAX = 64         # buffered queries for the column-mass estimate [D], [R Overhead]


# --------------------------------------------------------------------------
# O1: the three-way key partition [D method paragraph]
# --------------------------------------------------------------------------
def softmax_scale(d: int) -> float:
    """Scale of the attention logits (reading: the standard 1/sqrt(d))."""
    return 1.0 / math.sqrt(d)


def partition(L: int, W: int):
    """Prefix positions 0..L-1 split into the non-window prefix [0, n_nw) and
    the most recent window [n_nw, L).  Returns (n_nw, window positions)."""
    n_nw = max(0, L - W)
    return n_nw, np.arange(n_nw, L, dtype=np.int64)


def n_vertical(rho: float, n_nw: int) -> int:
    """Size of the vertical-line set: top-rho of the non-window prefix [D].
    The 1e-6 absorbs binary representation error of rho (0.29*100 is
    28.999999999999996)."""
    return int(math.floor(rho * n_nw + 1e-6))


# --------------------------------------------------------------------------
# O2: column attention mass [D method paragraph; R Overview item 1]
# --------------------------------------------------------------------------
def buffered_positions(L: int, nb: int) -> np.ndarray:
    """The buffered queries are the last nb prefix positions (prefill tail)."""
    return np.arange(L - nb, L, dtype=np.int64)


def attention_rows(K: np.ndarray, qs: np.ndarray, pos: np.ndarray, d: int):
    """Causal softmax rows of queries ``qs`` [n][d] (at positions ``pos``)
    over keys K[0..L) in fp64.  Returns (probabilities [n][L], lse [n]),
    lse in natural log."""
    Kd = K.astype(np.float64)
    z = softmax_scale(d) * (qs.astype(np.float64) @ Kd.T)          # [n][L]
    keys = np.arange(K.shape[0])
    z = np.where(keys[None, :] <= pos[:, None], z, -np.inf)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    s = e.sum(axis=1, keepdims=True)
    lse = (zmax + np.log(s))[:, 0]
    return e / s, lse


def column_mass_unit(K: np.ndarray, qgrp: np.ndarray, L: int, W: int) -> np.ndarray:
    """Delta of the column-mass score of one (sequence, KV head).

    K [L][d] fp16; qgrp [G][nb][d] fp16 = the buffered queries of the G query
    heads sharing this KV head.  Every buffered query's causal softmax row is
    computed over all its keys (window included) and the probabilities of the
    non-window columns are summed over heads and queries.  Returns [n_nw].
    """
    G, nb, d = qgrp.shape
    n_nw, _ = partition(L, W)
    pos = buffered_positions(L, nb)
    dc = np.zeros(n_nw, dtype=np.float64)
    for h in range(G):
        a, _ = attention_rows(K[:L], qgrp[h], pos, d)
        dc += a[:, :n_nw].sum(axis=0)
    return dc


def column_mass_given_lse_unit(K: np.ndarray, qgrp: np.ndarray, lse: np.ndarray, L: int,
                               W: int) -> np.ndarray:
    """The column-mass delta with each buffered row normalised by a given
    natural-log LSE (lse [G][nb]) instead of its own: exp(tau q.k_i - lse)
    summed over the heads and rows, causal, non-window columns [n_nw].  With
    the rows' own LSE this is column_mass_unit; a caller may supply LSE rows
    it already has (the prefill's)."""
    G, nb, d = qgrp.shape
    n_nw, _ = partition(L, W)
    pos = buffered_positions(L, nb)
    tau = softmax_scale(d)
    Kd = K[:L].astype(np.float64)
    keys = np.arange(L)
    dc = np.zeros(n_nw, dtype=np.float64)
    for h in range(G):
        z = tau * (qgrp[h].astype(np.float64) @ Kd.T)
        a = np.where(keys[None, :] <= pos[:, None], np.exp(z - lse[h][:, None]), 0.0)
        dc += a[:, :n_nw].sum(axis=0)
    return dc


def row_lse_unit(K: np.ndarray, qgrp: np.ndarray, L: int) -> np.ndarray:
    """Natural-log LSE of each buffered query's causal row: [G][nb]."""
    G, nb, d = qgrp.shape
    pos = buffered_positions(L, nb)
    return np.stack([attention_rows(K[:L], qgrp[h], pos, d)[1] for h in range(G)])


# --------------------------------------------------------------------------
# O3: top-rho selection [D method paragraph]
# --------------------------------------------------------------------------
def top_rho(c: np.ndarray, n_vl: int) -> np.ndarray:
    """Positions of the n_vl largest scores c[0..n); ties to the lower
    position.  Returned ascending."""
    n = c.shape[0]
    order = np.lexsort((np.arange(n), -c))          # by -c, then position
    return np.sort(order[:n_vl]).astype(np.int64)


def select_vertical_unit(K, qgrp, L, W, rho, score_in=None):
    """Running score update c <- c + delta and the top-rho set over the
    non-window prefix.  Returns (score [L] fp64, vl positions, vl_flag [L])."""
    n_nw, _ = partition(L, W)
    score = np.zeros(L, np.float64) if score_in is None else score_in.astype(np.float64).copy()
    score[:n_nw] += column_mass_unit(K, qgrp, L, W)
    vl = top_rho(score[:n_nw], n_vertical(rho, n_nw))
    flag = np.zeros(L, np.uint8)
    flag[vl] = 1
    return score, vl, flag


# --------------------------------------------------------------------------
# O4/O5: K4V4 quantisation and packing [R Overview item 3; H author comment]
# --------------------------------------------------------------------------
def quantize_groups(X: np.ndarray, bits: int = 4):
    """Asymmetric b-bit quantisation of tokens X [n][d] (fp16), one group per
    32 consecutive head_dim elements (b = 4 for K4V4; 2 and 8 for the other
    strict low-bit caches of [R Mode reference], same rule with 2^b - 1
    steps).

    min m and max M of the group; scale s = fp16(round-to-nearest-even of
    (M - m) / (2^b - 1)); a zero minimum or a zero scale is stored as +0;
    code = clamp(round-half-even((x - m) / s), 0, 2^b - 1), all 0 when
    s == 0.  Every step is exact in fp64 before its single rounding.
    Returns codes uint8 [n][d], scale fp16 [n][d/32], min fp16 [n][d/32].
    """
    assert bits in KV_BITS
    qmax = (1 << bits) - 1
    n, d = X.shape
    x = X.astype(np.float64).reshape(n, d // GROUP, GROUP)
    m = x.min(axis=2) + 0.0        # a zero minimum is stored as +0
    M = x.max(axis=2)
    s16 = (((M - m) + 0.0) / qmax).astype(np.float16)   # a zero range gives scale +0
    s = s16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((x - m[:, :, None]) / s[:, :, None])
    q = np.where(s[:, :, None] > 0, np.clip(q, 0, qmax), 0)
    return q.reshape(n, d).astype(np.uint8), s16, m.astype(np.float16)


def pack_codes(codes: np.ndarray, bits: int = 4) -> np.ndarray:
    """b-bit codes [n][d] into bytes [n][d*b/8]: 8/b codes per byte, the
    lower-index element in the lower bits (element (8/b) j + r of byte j at
    bits b r .. b r + b - 1)."""
    per = 8 // bits
    n, d = codes.shape
    out = np.zeros((n, d // per), np.uint16)
    for r in range(per):
        out |= codes[:, r::per].astype(np.uint16) << (bits * r)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int = 4) -> np.ndarray:
    per = 8 // bits
    n, h = packed.shape
    out = np.empty((n, per * h), np.uint8)
    for r in range(per):
        out[:, r::per] = (packed >> (bits * r)) & ((1 << bits) - 1)
    return out


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, element 2j in the low nibble, 2j+1 in the high."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    n, h = packed.shape
    out = np.empty((n, 2 * h), np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def make_meta(scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """Per-token metadata [n][d/32][2] fp16: {scale, min} for each group."""
    return np.stack([scale, mn], axis=-1).astype(np.float16)


def dequantize(packed: np.ndarray, meta: np.ndarray, bits: int = 4) -> np.ndarray:
    """x_hat = code * scale + min, in fp64: [n][d]."""
    c = unpack_codes(packed, bits).astype(np.float64)
    n, d = c.shape
    s = meta[:, :, 0].astype(np.float64)
    m = meta[:, :, 1].astype(np.float64)
    return (c.reshape(n, d // GROUP, GROUP) * s[:, :, None] + m[:, :, None]).reshape(n, d)


def quantize_pack_tokens(X: np.ndarray, bits: int = 4):
    codes, s, m = quantize_groups(X, bits)
    return pack_codes(codes, bits), make_meta(s, m)


# --------------------------------------------------------------------------
# The hybrid cache of one (sequence, KV head) and its construction
# --------------------------------------------------------------------------
def empty_unit_cache(d: int, W: int, k_bits: int = 4, v_bits: int = 4) -> Dict:
    """One unit's hybrid cache; the quantised region holds k_bits-bit keys
    and v_bits-bit values (K4V4 by default)."""
    return {
        "kq": np.zeros((0, d * k_bits // 8), np.uint8), "vq": np.zeros((0, d * v_bits // 8), np.uint8),
        "kq_meta": np.zeros((0, d // GROUP, 2), np.float16),
        "vq_meta": np.zeros((0, d // GROUP, 2), np.float16),
        "q_pos": np.zeros(0, np.int32),
        "kvl": np.zeros((0, d), np.float16), "vvl": np.zeros((0, d), np.float16),
        "vl_pos": np.zeros(0, np.int32),
        "kwin": np.zeros((W, d), np.float16), "vwin": np.zeros((W, d), np.float16),
        "kstg": np.zeros((0, d), np.float16), "vstg": np.zeros((0, d), np.float16),
        "stg_pos": np.zeros(0, np.int32),
        "W": W, "d": d, "k_bits": k_bits, "v_bits": v_bits,
    }


def quant_pack_unit(K: np.ndarray, V: np.ndarray, L: int, W: int,
                    vl_flag: np.ndarray, k_bits: int = 4, v_bits: int = 4) -> Dict:
    """Build the hybrid cache of one unit after the prefill tail [D decode
    paragraph; R Overview item 3]: vertical-line tokens (flag set, non-window)
    keep FP16 K and V in ascending position; the window [L-W, L) goes to an
    FP16 ring (slot = position mod W); every other prefix token is quantised
    and stored in ascending position.  Nothing is staged."""
    d = K.shape[1]
    n_nw, win = partition(L, W)
    flag = np.asarray(vl_flag[:n_nw]).astype(bool)
    qpos = np.nonzero(~flag)[0].astype(np.int32)
    vpos = np.nonzero(flag)[0].astype(np.int32)
    cache = empty_unit_cache(d, W, k_bits, v_bits)
    cache["kq"], cache["kq_meta"] = quantize_pack_tokens(K[qpos], k_bits)
    cache["vq"], cache["vq_meta"] = quantize_pack_tokens(V[qpos], v_bits)
    cache["q_pos"] = qpos
    cache["kvl"], cache["vvl"], cache["vl_pos"] = K[vpos].copy(), V[vpos].copy(), vpos
    for p in win:
        cache["kwin"][p % W] = K[p]
        cache["vwin"][p % W] = V[p]
    return cache


# --------------------------------------------------------------------------
# O7: staging and merge of new tokens [D decode paragraph]
# --------------------------------------------------------------------------
def append_merge_unit(cache: Dict, t: int, k_new: np.ndarray, v_new: np.ndarray,
                      evict_is_vl: bool = False) -> None:
    """New token at position t.  The token staged by the previous call
    (position t-1) is merged into the window ring at slot (t-1) mod W; the
    token that slot held (position t-1-W) leaves the window and is appended
    to the FP16 vertical-line region if flagged, else quantised and appended
    to the K4V4 region.  With W = 0 the staged token itself leaves.  Then the
    new token is staged.  In place."""
    W = cache["W"]
    if cache["stg_pos"].size:
        p = int(cache["stg_pos"][0])
        ks, vs = cache["kstg"][0].copy(), cache["vstg"][0].copy()
        if W > 0:
            slot = p % W
            ev = p - W
            if ev >= 0:
                ek, evv = cache["kwin"][slot].copy(), cache["vwin"][slot].copy()
                _evict(cache, ev, ek, evv, evict_is_vl)
            cache["kwin"][slot] = ks
            cache["vwin"][slot] = vs
        else:
            _evict(cache, p, ks, vs, evict_is_vl)
    cache["kstg"] = k_new[None, :].astype(np.float16).copy()
    cache["vstg"] = v_new[None, :].astype(np.float16).copy()
    cache["stg_pos"] = np.array([t], np.int32)


def _evict(cache, pos, k, v, to_vl):
    if to_vl:
        cache["kvl"] = np.concatenate([cache["kvl"], k[None]])
        cache["vvl"] = np.concatenate([cache["vvl"], v[None]])
        cache["vl_pos"] = np.concatenate([cache["vl_pos"], np.array([pos], np.int32)])
    else:
        kb, km = quantize_pack_tokens(k[None], cache.get("k_bits", 4))
        vb, vm = quantize_pack_tokens(v[None], cache.get("v_bits", 4))
        cache["kq"] = np.concatenate([cache["kq"], kb])
        cache["kq_meta"] = np.concatenate([cache["kq_meta"], km])
        cache["vq"] = np.concatenate([cache["vq"], vb])
        cache["vq_meta"] = np.concatenate([cache["vq_meta"], vm])
        cache["q_pos"] = np.concatenate([cache["q_pos"], np.array([pos], np.int32)])


# --------------------------------------------------------------------------
# O6/O9: decode attention over the hybrid cache [D decode paragraph;
#        R Overview item 3]
# --------------------------------------------------------------------------
def hybrid_regions(cache: Dict, L: int):
    """The key/value regions one decode query at position L attends to, as
    fp64 arrays: K4V4 slots (dequantised), vertical lines, window (positions
    [max(0, L-W), L)), staging.  Returns a list of (name, positions, K, V)."""
    W = cache["W"]
    out = [("k4", cache["q_pos"].astype(np.int64),
            dequantize(cache["kq"], cache["kq_meta"], cache.get("k_bits", 4)),
            dequantize(cache["vq"], cache["vq_meta"], cache.get("v_bits", 4))),
           ("vl", cache["vl_pos"].astype(np.int64),
            cache["kvl"].astype(np.float64), cache["vvl"].astype(np.float64))]
    if W > 0:
        wpos = np.arange(max(0, L - W), L, dtype=np.int64)
        slots = wpos % W
        out.append(("win", wpos, cache["kwin"][slots].astype(np.float64),
                    cache["vwin"][slots].astype(np.float64)))
    out.append(("stg", cache["stg_pos"].astype(np.int64),
                cache["kstg"].astype(np.float64), cache["vstg"].astype(np.float64)))
    return out


def decode_unfused(cache: Dict, q: np.ndarray, L: int):
    """O9-i: materialise the hybrid keys/values in fp64, then plain softmax
    attention.  q [G][d].  Returns (o [G][d], lse [G] natural log)."""
    regs = hybrid_regions(cache, L)
    Kt = np.concatenate([r[2] for r in regs])
    Vt = np.concatenate([r[3] for r in regs])
    z = softmax_scale(q.shape[1]) * (q.astype(np.float64) @ Kt.T)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    s = e.sum(axis=1, keepdims=True)
    return (e @ Vt) / s, (zmax + np.log(s))[:, 0]


def decode_fused(cache: Dict, q: np.ndarray, L: int, tile: int = 256):
    """O9-ii: one online softmax over the regions, K4V4 tiles dequantised one
    tile at a time (no full-precision cache), then VL, window and staging."""
    G, d = q.shape
    qd = q.astype(np.float64)
    tau = softmax_scale(d)
    m = np.full(G, -np.inf)
    l = np.zeros(G)
    acc = np.zeros((G, d))

    def absorb(Kt, Vt):
        nonlocal m, l, acc
        if Kt.shape[0] == 0:
            return
        z = tau * (qd @ Kt.T)
        m_new = np.maximum(m, z.max(axis=1))
        alpha = np.exp(m - m_new)
        p = np.exp(z - m_new[:, None])
        l = l * alpha + p.sum(axis=1)
        acc = acc * alpha[:, None] + p @ Vt
        m = m_new

    n_q = cache["kq"].shape[0]
    for t0 in range(0, n_q, tile):
        sl = slice(t0, min(n_q, t0 + tile))
        absorb(dequantize(cache["kq"][sl], cache["kq_meta"][sl], cache.get("k_bits", 4)),
               dequantize(cache["vq"][sl], cache["vq_meta"][sl], cache.get("v_bits", 4)))
    for name, _, Kr, Vr in hybrid_regions(cache, L)[1:]:
        absorb(Kr, Vr)
    return acc / l[:, None], m + np.log(l)


# --------------------------------------------------------------------------
# Batch drivers (loops over units; kvh of query head h is h // G)
# --------------------------------------------------------------------------
def select_vertical(K, qbuf, L, W, rho, score_in=None):
    """K [B][Hkv][L][d], qbuf [B][Hq][nb][d].  Returns score [B][Hkv][L],
    list of VL index arrays [B][Hkv], vl_flag [B][Hkv][L]."""
    B, Hkv = K.shape[:2]
    G = qbuf.shape[1] // Hkv
    score = np.zeros((B, Hkv, L))
    flags = np.zeros((B, Hkv, L), np.uint8)
    idx = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        for g in range(Hkv):
            s_in = None if score_in is None else score_in[b, g]
            score[b, g], idx[b][g], flags[b, g] = select_vertical_unit(
                K[b, g], qbuf[b, g * G:(g + 1) * G], L, W, rho, s_in)
    return score, idx, flags


def quant_pack(K, V, L, W, vl_flag, k_bits: int = 4, v_bits: int = 4) -> List[List[Dict]]:
    B, Hkv = K.shape[:2]
    return [[quant_pack_unit(K[b, g], V[b, g], L, W, vl_flag[b, g], k_bits, v_bits)
             for g in range(Hkv)] for b in range(B)]


def append_merge(caches, t, k_new, v_new, evict_is_vl=None) -> None:
    for b, row in enumerate(caches):
        for g, c in enumerate(row):
            ev = False if evict_is_vl is None else bool(evict_is_vl[b, g])
            append_merge_unit(c, t, k_new[b, g], v_new[b, g], ev)


def decode(caches, q, L, fused=True):
    """q [B][Hq][d] -> (out [B][Hq][d] fp64, lse [B][Hq])."""
    B, Hq, d = q.shape
    Hkv = len(caches[0])
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    f = decode_fused if fused else decode_unfused
    for b in range(B):
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G] = f(
                caches[b][g], q[b, g * G:(g + 1) * G], L)
    return out, lse


# --------------------------------------------------------------------------
# Decode-time running refresh [D method paragraph: running column-mass score
# from at most 64 buffered queries, refreshed every 64 tokens; R Overview
# item 1].  Readings: the buffered queries are the last nb decode queries;
# each row's normaliser is the LSE its decode step produced (one pass over
# the keys); the keys are the hybrid cache as stored at refresh time, a
# K4V4 key taken as the fp16 rounding of code * scale + min (the compute
# type of the attention scan); every cached position accumulates (window and
# staged tokens too, since their mass decides promotion when they leave the
# window); the cut-off is the n_vl-th largest running score over the
# non-window prefix; a token leaving the window becomes a vertical line when
# its running score reaches the cut-off.
# --------------------------------------------------------------------------
def hybrid_keys(cache: Dict, t: int):
    """Positions and keys [n][d] (fp64) of every key cached at decode
    position t: the K4V4 slots as their exact dequantisation code * scale +
    min (the key the cache holds, as decode attention takes it), then the
    FP16 vertical lines, window and staged token."""
    regs = hybrid_regions(cache, t)
    return np.concatenate([r[1] for r in regs]), np.concatenate([r[2] for r in regs])


def refresh_hybrid_unit(cache: Dict, t: int, qgrp: np.ndarray, lse: np.ndarray,
                        rho: float, score: np.ndarray):
    """One refresh at decode position t (the staged token).  qgrp [G][nb][d]
    are the last nb decode queries (positions t - nb + 1 .. t), lse [G][nb]
    the natural-log LSE of each at its own decode step.  For every cached key
    at position i, exp(tau q.k_i - lse) of every row with i <= its position
    is added to score[i] (in place).  Returns (cut, vl positions): the n_vl-th
    largest running score over [0, t - W) (+inf when n_vl = 0) and the top-rho
    set there (ascending, ties to the lower position)."""
    G, nb, d = qgrp.shape
    W = cache["W"]
    tau = softmax_scale(d)
    pos, keys = hybrid_keys(cache, t)
    rows_pos = t - nb + 1 + np.arange(nb)
    for h in range(G):
        z = tau * (qgrp[h].astype(np.float64) @ keys.T)            # [nb][n]
        a = np.exp(z - lse[h][:, None]) * (pos[None, :] <= rows_pos[:, None])
        score[pos] += a.sum(axis=0)
    n_nw = max(0, t - W)
    n_vl = n_vertical(rho, n_nw)
    if n_vl == 0:
        return math.inf, np.zeros(0, np.int64)
    sel = top_rho(score[:n_nw], n_vl)
    return float(score[sel].min()), sel


def append_merge_scored_unit(cache: Dict, t: int, k_new: np.ndarray, v_new: np.ndarray,
                             score: np.ndarray, cut: float) -> bool:
    """append_merge_unit where the token leaving the window (position
    t - 1 - W, or t - 1 with no window) becomes a vertical line exactly when
    score[pos] >= cut.  Returns that decision (False when nothing leaves)."""
    W = cache["W"]
    ev = -1
    if cache["stg_pos"].size:
        p = int(cache["stg_pos"][0])
        ev = p - W if W > 0 else p
    promote = ev >= 0 and bool(score[ev] >= cut)
    append_merge_unit(cache, t, k_new, v_new, promote)
    return promote


# --------------------------------------------------------------------------
# Prefill: one fused hybrid-precision attention [D method paragraph, the
# prefill sentences; R Overview item 2; R repository layout, the ops listing
# (INT8-QK + FP16-PV prefill attention with window / vertical variants)].
# Readings: the low-bit path quantises Q and K to symmetric INT8 per token
# row (one scale per row of d elements): scale = fp32(amax / 127), code =
# round-half-even(x / (amax / 127)) in exact arithmetic, i.e. of 127 x / amax
# (all codes 0 and scale 0 when amax = 0); a key is kept in FP16 for query p
# when it is a vertical line or lies in the query's own window (p - i < W),
# else its logit is tau * (q8 . k8) * scale_q * scale_k; causal (i <= p);
# P V runs in FP16 for every key, so the oracle takes the exact softmax times
# V; the LSE (natural log) is over the hybrid logits.
# --------------------------------------------------------------------------
def int8_quantize_rows(X: np.ndarray):
    """Symmetric per-row INT8 of fp16 rows X [..][d].  Returns (codes int8
    [..][d], scales float32 [..]).  127 x is exact in float64 and a single
    correctly rounded division cannot cross a half-integer (the exact
    quotient is a ratio of 18- and 11-bit integers), so rint gives the exact
    round-half-even code."""
    Xd = X.astype(np.float64)
    amax = np.abs(Xd).max(axis=-1, keepdims=True)
    safe = np.where(amax > 0.0, amax, 1.0)
    codes = np.where(amax > 0.0, np.rint(127.0 * Xd / safe), 0.0) + 0.0
    scales = (amax[..., 0] / 127.0).astype(np.float32)
    return codes.astype(np.int8), scales


def prefill_fp16_mask(pos: np.ndarray, L: int, W: int, vl_flag: np.ndarray) -> np.ndarray:
    """[n][L] bool: key i is taken in FP16 by the query at position pos[r]
    (i <= pos[r], and i is a vertical line or pos[r] - i < W)."""
    p = np.asarray(pos, np.int64)[:, None]
    i = np.arange(L)[None, :]
    return (i <= p) & (((p - i) < W) | (np.asarray(vl_flag)[None, :L] != 0))


def prefill_rows_unit(Qr: np.ndarray, pos: np.ndarray, K: np.ndarray, V: np.ndarray,
                      vl_flag: Optional[np.ndarray], W: int):
    """Causal prefill attention of one unit for the queries at positions pos
    (Qr [G][n][d], the queries of those positions; K, V [L][d] fp16; vl_flag
    [L] or None: no vertical lines).  Returns (O [G][n][d], lse [G][n]) in
    float64."""
    G, n, d = Qr.shape
    L = K.shape[0]
    tau = softmax_scale(d)
    pos = np.asarray(pos, np.int64)
    flag = np.zeros(L, np.uint8) if vl_flag is None else np.asarray(vl_flag)
    q8, sq = int8_quantize_rows(Qr)
    k8, sk = int8_quantize_rows(K)
    hi = prefill_fp16_mask(pos, L, W, flag)
    causal = np.arange(L)[None, :] <= pos[:, None]
    Kd, Vd = K.astype(np.float64), V.astype(np.float64)
    k8d = k8.astype(np.float64)
    O = np.zeros((G, n, d))
    lse = np.zeros((G, n))
    for h in range(G):
        z_hi = tau * (Qr[h].astype(np.float64) @ Kd.T)
        z_lo = tau * (q8[h].astype(np.float64) @ k8d.T) * sq[h].astype(np.float64)[:, None] \
            * sk.astype(np.float64)[None, :]
        z = np.where(hi, z_hi, z_lo)
        z[~causal] = -np.inf
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        s = e.sum(axis=1)
        O[h] = (e @ Vd) / s[:, None]
        lse[h] = m + np.log(s)
    return O, lse


def prefill_hybrid_unit(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                        vl_flag: Optional[np.ndarray], W: int):
    """Every query of the prefix: Q [G][L][d].  Returns (O [G][L][d],
    lse [G][L])."""
    return prefill_rows_unit(Q, np.arange(Q.shape[1]), K, V, vl_flag, W)


def prefill_hybrid(Q, K, V, vl_flag, W):
    """Batch driver: Q [B][Hq][L][d], K, V [B][Hkv][L][d], vl_flag
    [B][Hkv][L] or None.  Query head h uses KV head h // (Hq / Hkv)."""
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, Hq, L, d))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for g in range(Hkv):
            f = None if vl_flag is None else vl_flag[b, g]
            O[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G] = prefill_hybrid_unit(
                Q[b, g * G:(g + 1) * G], K[b, g], V[b, g], f, W)
    return O, lse


# --------------------------------------------------------------------------
# Byte accounting [R Overhead; D limitations paragraph]
# --------------------------------------------------------------------------
def k4v4_bytes_per_token(d: int = 128) -> int:
    """K and V codes (d/2 bytes each) + K and V {scale, min} fp16 per group."""
    return 2 * (d // 2) + 2 * (d // GROUP) * 2 * 2


def fp16_bytes_per_token(d: int = 128) -> int:
    return 2 * d * 2


def query_buffer_bytes(Hq: int, d: int, nb: int = NB_MAX) -> int:
    """FP16 query buffer of the column-mass estimate [R Overhead]."""
    return nb * Hq * d * 2


def kv_growth_vs_strict(rho: float, code_bits: float = 4.0, hi_bits: float = 16.0) -> float:
    """Relative growth of the non-window KV when a fraction rho of tokens is
    kept at hi_bits per element instead of code_bits [D limitations; R
    Overhead].  Pure 4-bit accounting (code_bits = 4) gives rho*12/4."""
    return (rho * hi_bits + (1 - rho) * code_bits) / code_bits - 1.0


def decode_step_bytes(B: int, Hq: int, Hkv: int, d: int, n_q: int, n_vl: int,
                      n_win: int, n_stg: int) -> int:
    """Algorithmic HBM bytes of one decode step: every unit reads each K4V4
    token once and each FP16 token (vertical line, window, staging) once;
    plus the fp16 query in and output out."""
    per_unit = (k4v4_bytes_per_token(d) * n_q
                + fp16_bytes_per_token(d) * (n_vl + n_win + n_stg))
    return B * Hkv * per_unit + B * Hq * d * 2 * 2
