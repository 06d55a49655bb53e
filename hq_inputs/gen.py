"""Seeded generators for the five decode-attention workloads.

The workloads follow the shapes the HyQuant pages report their measurements
on (decode-kernel latency at 1K-32K prefixes, a batch-capacity run at a 32K
prefix; HyQuant README, "Efficiency: decode attention kernel latency", and the
agihunt digest, results paragraph) with the attention-map structure the
method is built around: a few "vertical-line" key positions that nearly every
query attends to (agihunt digest, method paragraph).  There are no trained
weights, so the lines are planted: a unit vector u per KV head is added with a
strength ``a`` to the keys at the planted positions and with strength 1.5 to
every query, which makes those keys dominate the column attention mass.

Recipe (one sequence b of workload number c):
  * RNG ``numpy.random.Generator(PCG64(10000*c + b))``;
  * draw order: u [Hkv][d] (normal, then normalised per KV head); K [Hkv][L][d];
    V [Hkv][L][d]; the buffered queries [Hq][nb][d]; the planted positions
    (without replacement from the non-window prefix minus the sinks); their
    strengths; then for each decode step t: k, v [Hkv][d] and q [Hq][d];
  * values are float32 N(0,1); planting is applied in float32; the result is
    rounded to fp16 (round to nearest even).  Workloads flagged ``bf16`` are
    rounded to bf16 first, then to fp16.
  * prefill queries of every prefix position (``prefill_queries``): their own
    stream, ``PCG64(SeedSequence([number, b, 7]))``, drawn as Q [Hq][L][d]
    N(0,1) plus 1.5 u of the query's KV head (u as above), then rounded the
    same way.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one decode-attention workload."""
    name: str
    number: int             # seed namespace (seed = 10000*number + b)
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int                  # prefix length; the decode token sits at position L
    W: int                  # local FP16 window
    rho: float              # vertical-line ratio of the non-window prefix
    n_plant: int            # planted vertical lines (besides the sinks)
    sinks: bool             # also plant positions 0..3
    strength: tuple         # (lo, hi): a ~ U(lo, hi); lo == hi -> fixed
    bf16: bool = False      # round to bf16 before fp16
    steps: int = 1          # decode steps drawn

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nb(self) -> int:
        """Buffered queries: at most 64, the last nb prefix positions."""
        return min(64, self.L)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _plant_count(frac: float, L: int) -> int:
    return int(np.floor(frac * L))


WORKLOADS = {
    # 1: tiny decode step, one layer (GQA 4): sinks + 4 random lines, a = 4
    "tiny": Workload("tiny", 1, B=1, Hq=8, Hkv=2, d=128, L=1024, W=128, rho=0.05,
                     n_plant=4, sinks=True, strength=(4.0, 4.0)),
    # 2: Llama-3.1-8B-shaped layer: 1 % of positions + 4 sinks
    "llama31_8b": Workload("llama31_8b", 2, B=1, Hq=32, Hkv=8, d=128, L=32768,
                           W=128, rho=0.05, n_plant=_plant_count(0.01, 32768),
                           sinks=True, strength=(4.0, 4.0)),
    # 3: Qwen3-8B-shaped batch sweep, bf16-rounded values (B in {1,4,16,32})
    "qwen3_8b": Workload("qwen3_8b", 3, B=32, Hq=32, Hkv=8, d=128, L=32768,
                         W=128, rho=0.05, n_plant=_plant_count(0.01, 32768),
                         sinks=True, strength=(4.0, 4.0), bf16=True),
    # 4: GLM-4-9B-shaped GQA-16 sweep: 2 % of positions, a ~ U(2, 6)
    "glm4_9b": Workload("glm4_9b", 4, B=8, Hq=32, Hkv=2, d=128, L=32768, W=128,
                        rho=0.05, n_plant=_plant_count(0.02, 32768), sinks=False,
                        strength=(2.0, 6.0)),
    # 5: Qwen3-32B-shaped streaming decode: 3 % of positions, 128 steps
    "qwen3_32b": Workload("qwen3_32b", 5, B=32, Hq=64, Hkv=8, d=128, L=32768,
                          W=128, rho=0.05, n_plant=_plant_count(0.03, 32768),
                          sinks=False, strength=(4.0, 4.0), steps=128),
}


def workload(name: str, **overrides) -> Workload:
    """Named workload, optionally with some fields replaced (e.g. a smaller L).

    When L is overridden and ``n_plant`` is not, the planted count is scaled
    with L in the workload's own proportion (the tiny workload keeps 4).
    """
    base = WORKLOADS[name]
    if "L" in overrides and "n_plant" not in overrides and name != "tiny":
        frac = base.n_plant / base.L
        overrides["n_plant"] = _plant_count(frac, overrides["L"])
    return base.replace(**overrides)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (round to nearest even) -> float32, by bit manipulation."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def _to_fp16(x: np.ndarray, bf16: bool) -> np.ndarray:
    if bf16:
        x = bf16_round(x)
    return x.astype(np.float16)


def unit_vectors(rng: np.random.Generator, Hkv: int, d: int) -> np.ndarray:
    u = rng.standard_normal((Hkv, d), dtype=np.float32)
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def sequence(wl: Workload, b: int, steps: Optional[int] = None) -> dict:
    """All inputs of sequence ``b``: prefix K/V, buffered queries, decode tokens.

    Returns fp16 arrays ``K``, ``V`` [Hkv][L][d], ``qbuf`` [Hq][nb][d],
    ``k_dec``, ``v_dec`` [T][Hkv][d], ``q_dec`` [T][Hq][d] and the planted
    positions ``plant`` (ascending int64) with their float32 ``strength``.
    """
    T = wl.steps if steps is None else steps
    Hkv, Hq, d, L, W, G, nb = wl.Hkv, wl.Hq, wl.d, wl.L, wl.W, wl.G, wl.nb
    rng = np.random.Generator(np.random.PCG64(10000 * wl.number + b))
    u = unit_vectors(rng, Hkv, d)
    K = rng.standard_normal((Hkv, L, d), dtype=np.float32)
    V = rng.standard_normal((Hkv, L, d), dtype=np.float32)
    qbuf = rng.standard_normal((Hq, nb, d), dtype=np.float32)

    n_nw = max(0, L - W)
    sinks = [p for p in range(4) if wl.sinks and p < n_nw]
    cand = np.setdiff1d(np.arange(n_nw, dtype=np.int64), np.array(sinks, dtype=np.int64))
    n_rand = min(wl.n_plant, cand.size)
    rand = rng.choice(cand, size=n_rand, replace=False) if n_rand else np.zeros(0, np.int64)
    lo, hi = wl.strength
    strength_rand = (rng.uniform(lo, hi, size=n_rand).astype(np.float32) if hi > lo
                     else np.full(n_rand, lo, dtype=np.float32))
    plant = np.concatenate([np.array(sinks, dtype=np.int64), rand.astype(np.int64)])
    strength = np.concatenate([np.full(len(sinks), lo if hi == lo else (lo + hi) / 2,
                                       dtype=np.float32), strength_rand])
    order = np.argsort(plant, kind="stable")
    plant, strength = plant[order], strength[order]

    if plant.size:
        K[:, plant, :] += strength[None, :, None] * u[:, None, :]
    qbuf += 1.5 * np.repeat(u, G, axis=0)[:, None, :]

    k_dec = np.empty((T, Hkv, d), dtype=np.float32)
    v_dec = np.empty((T, Hkv, d), dtype=np.float32)
    q_dec = np.empty((T, Hq, d), dtype=np.float32)
    for t in range(T):
        k_dec[t] = rng.standard_normal((Hkv, d), dtype=np.float32)
        v_dec[t] = rng.standard_normal((Hkv, d), dtype=np.float32)
        q_dec[t] = rng.standard_normal((Hq, d), dtype=np.float32)
    q_dec += 1.5 * np.repeat(u, G, axis=0)[None, :, :]

    f = lambda x: _to_fp16(x, wl.bf16)
    return {"K": f(K), "V": f(V), "qbuf": f(qbuf), "k_dec": f(k_dec),
            "v_dec": f(v_dec), "q_dec": f(q_dec), "plant": plant,
            "strength": strength}


def batch(wl: Workload, steps: Optional[int] = None,
          seqs: Optional[Sequence[int]] = None) -> dict:
    """Stack ``sequence`` over the batch: K, V [B][Hkv][L][d], qbuf [B][Hq][nb][d],
    k_dec, v_dec [T][B][Hkv][d], q_dec [T][B][Hq][d]; plant is a list per b."""
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    per = [sequence(wl, b, steps) for b in seqs]
    out = {k: np.stack([p[k] for p in per]) for k in ("K", "V", "qbuf")}
    for k in ("k_dec", "v_dec", "q_dec"):
        out[k] = np.stack([p[k] for p in per], axis=1)
    out["plant"] = [p["plant"] for p in per]
    out["strength"] = [p["strength"] for p in per]
    return out


def prefill_queries(wl: Workload, b: int) -> np.ndarray:
    """Queries of every prefix position of sequence ``b``, fp16 [Hq][L][d]:
    N(0,1) from their own stream plus 1.5 u of the KV head (the vector the
    planted keys carry), so that the planted lines draw attention in the
    prefill as in decode."""
    u = unit_vectors(np.random.Generator(np.random.PCG64(10000 * wl.number + b)), wl.Hkv, wl.d)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.number, b, 7])))
    Q = rng.standard_normal((wl.Hq, wl.L, wl.d), dtype=np.float32)
    Q += 1.5 * np.repeat(u, wl.G, axis=0)[:, None, :]
    return _to_fp16(Q, wl.bf16)
