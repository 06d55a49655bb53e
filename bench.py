#!/usr/bin/env python3
"""Benchmark of the hybrid K4V4/FP16 decode-attention path on one MI355X.

A timed *step* is one streaming decode step of the whole hot path, one
hq_decode_step launch: the staging merge of the new token (the token leaving
the window quantised or promoted, the new one into the ring) and the decode
attention (split-K fused scan + in-kernel log-sum-exp merge).  The first step
of every 64-step period of the timed window also runs the vertical-line
refresh hq_select_vertical over 64 buffered queries (the pages' refresh
cadence), so K timed steps hold ceil(K / 64) refreshes.  The same steps
without the refresh (``step_us_decode_only``) and as two launches
(hq_append_merge, then hq_decode_attn; ``step_us_unfused``) are timed too,
and ``step_us_amortized_64`` is the decode-only step plus 1/64 of the
measured refresh.  hq_quant_pack, which builds the cache once after the
prefill, is timed on its own and reported beside the step.

The cache footprint of one small-batch layer fits in the 256 MB Infinity
Cache, so the step rotates over R independent cache replicas (R * footprint
>= 1 GiB) to measure HBM rather than cache bandwidth.

Beside the step, with the sweeps on (default): the batch sweep of the
Qwen3-8B-shaped layer (B = 1, 4, 16, 32), the other code widths, a context
sweep of the Llama-shaped layer (L = 1K .. 32K), a grid of the
GLM-4-9B-shaped GQA-16 layer (B = 8, L = 1K .. 32K, rho = 1, 5, 10 %, with
the selection, its one-pass form and the decode-time refresh timed at 32K),
a Qwen3-32B-shaped layer streaming 128 tokens at B = 32, the read ceiling,
the prefill attention and the capacity runs.

Prints one JSON line.  ``value`` is the effective HBM bandwidth of the timed
window: the algorithmic bytes of the launches it ran (what the method must
move: 160 B per K4V4 token and 512 B per FP16 token per KV head, q in, out,
merge traffic, and both selection passes over the dense keys for each
refresh) divided by the window's measured time, so value * ms_per_step * K
equals those bytes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid K4V4 decode-attn µs/step + HBM GB/s (% of peak) at L=32K, B=1..32"
PEAK_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
PEAK_I8_TOPS = 5000.0
REFRESH = 64
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "decode_traffic*.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--workload", default="llama31_8b")
    p.add_argument("--B", type=int, default=None, help="batch override (e.g. the qwen3_8b sweep)")
    p.add_argument("--rho", type=float, default=None)
    p.add_argument("--L", type=int, default=None)
    p.add_argument("--replicas", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--decode-only", action="store_true",
                   help="time only hq_decode_attn launches (profiling runs)")
    p.add_argument("--no-capacity", action="store_true",
                   help="skip the whole-model capacity run (36 layers at the largest 32K batch)")
    p.add_argument("--capacity-only", action="store_true",
                   help="print only the capacity run's JSON object")
    p.add_argument("--prefill-only", action="store_true",
                   help="print only the prefill timing's JSON object")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill attention timing")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the decode batch sweep and the streaming-read ceiling")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="run a plain device copy of this many bytes (counter calibration) and exit")
    return p.parse_args()


def src_hash():
    import hashlib
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "hybrid_precision_attention_amd", "csrc", "decode_attn.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def graph_upload(g, torch):
    """Upload an instantiated graph before its timed replay (hipGraphUpload)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    st = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError(f"hipGraphUpload failed ({st})")


def load_traffic(wl_name, B):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs
    (profiles/decode_traffic*.txt), or None when none was taken on this
    kernel source and workload."""
    import glob
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        kv = {}
        with open(path) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256_16") != src_hash():
            continue
        if kv.get("workload") != wl_name or int(kv.get("B", -1)) != B:
            continue
        try:
            return float(kv["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            return None
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by "
              "(sequence, KV head) with no exchange, so N GPUs are N independent copies.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_bytes:
        n = args.copy_bytes // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 3}))
        return

    import hybrid_precision_attention_amd as H
    from hq_inputs import workload, batch

    if args.capacity_only:
        print(json.dumps({"capacity": capacity_run(H, torch),
                          "capacity_ragged_paged": capacity_ragged_run(H, torch)}))
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_timing(H, torch)}))
        return

    over = {}
    if args.B is not None:
        over["B"] = args.B
    if args.rho is not None:
        over["rho"] = args.rho
    if args.L is not None:
        over["L"] = args.L
    wl = workload(args.workload, **over)
    B, Hq, Hkv, d, L, W = wl.B, wl.Hq, wl.Hkv, wl.d, wl.L, wl.W
    G = Hq // Hkv
    U = B * Hkv
    dev = torch.device("cuda")
    torch.manual_seed(0)

    # ---- inputs (seeded, synthetic) and the one-time cache build ----------
    t0 = time.time()
    x = batch(wl, steps=1)
    K = torch.from_numpy(x["K"]).to(dev)
    V = torch.from_numpy(x["V"]).to(dev)
    qbuf = torch.from_numpy(x["qbuf"]).to(dev)
    del x
    gen_s = time.time() - t0
    n_nw = max(0, L - W)
    n_vl = H.n_vertical(wl.rho, n_nw)
    total_steps = args.warmup + args.steps
    dims_sel = H.make_dims(B, Hq, Hkv, W, wl.rho)
    ws_sel = H.workspace(dims_sel, H.HQ_OP_SELECT, L)
    score = torch.zeros((B, Hkv, L), dtype=torch.float32, device=dev)
    vl_idx = torch.zeros((B, Hkv, max(1, n_vl)), dtype=torch.int32, device=dev)
    vl_flag = torch.zeros((B, Hkv, L), dtype=torch.uint8, device=dev)
    H.hq_select_vertical(dims_sel, qbuf, K, L, score, vl_idx, vl_flag, ws_sel)

    per_unit_fp16 = 512 * (n_vl + min(W, L) + 1)
    footprint = U * (160 * (n_nw - n_vl) + per_unit_fp16)
    R = args.replicas or max(1, math.ceil((1 << 30) / max(footprint, 1)))
    # positions a replica may advance: warm-up, the timed steps, the same
    # number unfused, the per-row merges and the refresh timing
    L_max = L + total_steps + 3 * args.steps + 64 + 16
    base = H.HybridCache.allocate(B, Hq, Hkv, W, wl.rho, L_max)
    H.hq_quant_pack(base.dims, K, V, L, vl_flag, base)
    torch.cuda.synchronize()
    caches = [base] + [base.clone() for _ in range(R - 1)]
    dims = base.dims
    ws = [H.workspace(dims, H.HQ_OP_DECODE, L_max) for _ in range(R)]
    pos = [L] * R
    pool = 64
    gk = torch.Generator(device=dev).manual_seed(1)
    k_new = torch.randn((pool, B, Hkv, d), generator=gk, device=dev).half()
    v_new = torch.randn((pool, B, Hkv, d), generator=gk, device=dev).half()
    q_new = torch.randn((pool, B, Hq, d), generator=gk, device=dev).half()
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    # dense keys for the refresh, rotated too (64 MiB per layer at L = 32K)
    k_bytes = K.numel() * 2
    R_sel = max(1, min(8, math.ceil((512 << 20) / k_bytes)))
    K_rep = [K] + [K.clone() for _ in range(R_sel - 1)]
    del V

    kp = [k_new[j].data_ptr() for j in range(pool)]
    vp = [v_new[j].data_ptr() for j in range(pool)]
    qp = [q_new[j].data_ptr() for j in range(pool)]

    def make_step(stream, fused=True):
        """Step function launching on ``stream`` (pointer arguments marshalled
        once): hq_decode_step, or (fused=False) hq_append_merge then
        hq_decode_attn, which attend the same tokens."""
        dec = [H.bind_decode(dims, caches[r], q_new[0], out, ws[r], lse=lse, stream=stream)
               for r in range(R)]
        mrg = [H.bind_merge(dims, caches[r], stream=stream) for r in range(R)]
        stp = [H.bind_step(dims, caches[r], q_new[0], out, ws[r], lse=lse, stream=stream)
               for r in range(R)]

        def step(i, refresh=False):
            r = i % R
            t = pos[r]
            j = i % pool
            if fused:
                stp[r](t, kp[j], vp[j], qp[j])
            else:
                mrg[r](t, kp[j], vp[j])
                dec[r](t, qp[j])
            pos[r] = t + 1
            if refresh:
                H.hq_select_vertical(dims_sel, qbuf, K_rep[(i // REFRESH) % R_sel], L, score,
                                     vl_idx, vl_flag, ws_sel, stream=stream)
        return step, dec

    if args.decode_only:
        _, dec = make_step(torch.cuda.current_stream())
        for i in range(total_steps):
            r = i % R
            dec[r](pos[r], qp[i % pool])
        torch.cuda.synchronize()
        print(json.dumps({"decode_only_launches": total_steps, "replicas": R}))
        return

    eager_step, _ = make_step(torch.cuda.current_stream())
    for i in range(args.warmup):
        eager_step(i, refresh=(i % REFRESH == 0))
    torch.cuda.synchronize()

    # The K timed steps are captured once into a HIP graph (through torch) and
    # replayed once, so the host's per-launch cost stays out of the step time.
    def capture(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body(torch.cuda.current_stream())
        graph_upload(g, torch)
        return g

    # The refresh runs at the first step of every 64-step period of the timed
    # window (the pages' cadence), so K timed steps hold ceil(K / 64)
    # refreshes and `value` counts exactly the bytes those launches move.
    n_refresh = sum(1 for k in range(args.steps) if k % REFRESH == 0)

    def timed_steps(stream):
        st, _ = make_step(stream)
        for k in range(args.steps):
            st(args.warmup + k, refresh=(k % REFRESH == 0))
    g_steps = capture(timed_steps)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    start.record()
    g_steps.replay()
    stop.record()
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps

    # the same number of decode steps without the refresh: one launch each,
    # and the merge and the decode as two launches
    def plain_steps(fused):
        def body(stream):
            st, _ = make_step(stream, fused=fused)
            for k in range(args.steps):
                st(args.warmup + (2 if fused else 3) * args.steps + k)
        g = capture(body)
        torch.cuda.synchronize()
        start.record()
        g.replay()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps
    ms_step_plain = plain_steps(True)
    ms_step_unfused = plain_steps(False)

    # Average decode launch duration: the same decode launches back to back
    # (rotating replicas, current positions), replayed from a graph between
    # HIP events on the launching stream.
    n_dec = args.steps

    def dec_body(stream):
        _, dec = make_step(stream)
        for i in range(n_dec):
            r = i % R
            dec[r](pos[r], qp[i % pool])
    g_dec = capture(dec_body)
    g_dec.replay()                                  # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_dec.replay()
    e1.record()
    torch.cuda.synchronize()
    dec_avg_ms = e0.elapsed_time(e1) / n_dec

    # ---- per-row timings (each on its own, same rotation) -----------------
    def time_loop(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # the refresh as the step runs it: launches replayed from a HIP graph
    n_sel = 2 * R_sel

    def sel_body(stream):
        for i in range(n_sel):
            H.hq_select_vertical(dims_sel, qbuf, K_rep[i % R_sel], L, score, vl_idx, vl_flag,
                                 ws_sel, stream=stream)
    g_sel = capture(sel_body)
    g_sel.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_sel.replay()
    e1.record()
    torch.cuda.synchronize()
    sel_ms = e0.elapsed_time(e1) / n_sel
    del g_sel
    spare = H.HybridCache.allocate(B, Hq, Hkv, W, wl.rho, L_max)
    pack_ms = time_loop(lambda i: H.hq_quant_pack(spare.dims, K_rep[i % R_sel], K_rep[(i + 1) % R_sel],
                                                  L, vl_flag, spare), 4)

    mrg = [H.bind_merge(dims, caches[r]) for r in range(R)]

    def merge_only(i):
        r = i % R
        mrg[r](pos[r], kp[i % pool], vp[i % pool])
        pos[r] += 1
    merge_ms = time_loop(merge_only, 64)
    torch.cuda.synchronize()
    refresh = refresh_timing(H, torch, wl, dims, caches, pos, qbuf, capture)

    # ---- algorithmic bytes ------------------------------------------------
    n_q_mid = (n_nw - n_vl) + (args.warmup + args.steps // 2) // R
    dec_bytes = U * (160 * n_q_mid + 512 * (n_vl + min(W, L) + 1)) + B * Hq * d * 2 * 2
    # the merge reads the leaving token and writes its K4V4 slot and the new
    # token's ring slot (the new token's read is in the decode's bytes)
    merge_bytes = U * (512 + 160 + 512)
    sel_bytes = 2 * U * L * d * 2 + B * Hq * wl.nb * d * 2 * 2 + U * n_nw * 4 * 2 + U * L
    # what the timed graph executed: K steps and n_refresh refreshes
    timed_bytes = args.steps * (dec_bytes + merge_bytes) + n_refresh * sel_bytes
    value = timed_bytes / (total_ms * 1e-3) / 1e9
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    traffic = load_traffic(wl.name, B)

    # selection: HBM (two passes over K) and MFMA (S = K Q^T twice) use
    sel_flops = 2 * 2 * (U * L) * (G * wl.nb) * d
    sel_util = {"hbm_gbs": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(sel_bytes / (sel_ms * 1e-3) / 1e9 / PEAK_GBS, 4),
                "mfma_tflops": round(sel_flops / (sel_ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(sel_flops / (sel_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}

    # ---- CPU baseline: the oracle on a bounded sample ---------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, base, H, torch)

    # ---- the metric's batch sweep, the read ceiling, prefill, capacity ----
    # (the step's own buffers are released first)
    if not (args.no_sweep and args.no_prefill and args.no_capacity):
        del caches, ws, K_rep, base, spare
        torch.cuda.empty_cache()
    sweep, ceiling, widths, contexts, gqa16, streaming, mfma = None, None, None, None, None, None, None
    if not args.no_sweep:
        sweep = decode_sweep(H, torch, workload)
        widths = width_sweep(H, torch, workload)
        contexts = context_sweep(H, torch, workload)
        gqa16 = gqa16_grid(H, torch, workload)
        streaming = streaming_run(H, torch, workload)
        ceiling = read_ceiling(torch, 4 << 30)
        ceiling["at_decode_footprint"] = read_ceiling_footprint(torch, dec_bytes)
        mfma = mfma_rate(torch)
    prefill = None if args.no_prefill else prefill_timing(H, torch)
    capacity = None if args.no_capacity else capacity_run(H, torch)
    capacity_ragged = None if args.no_capacity else capacity_ragged_run(H, torch)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{wl.name}-shaped layer", "B": B, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "L": L, "W": W, "rho": wl.rho, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "decode_kernel (hq_decode_attn)",
                     "bytes_per_launch": dec_bytes, "avg_launch_us": round(dec_avg_ms * 1e3, 2)},
        "cpu_baseline": cpu,
        "step_us": round(ms_step * 1e3, 2), "timed_host_s": round(t_host, 4),
        "timed_bytes": timed_bytes, "refreshes_timed": n_refresh,
        "step_us_decode_only": round(ms_step_plain * 1e3, 2),
        "step_us_unfused": round(ms_step_unfused * 1e3, 2),
        # the step at the pages' cadence, one refresh per 64 decode steps
        "step_us_amortized_64": round((ms_step_plain + sel_ms / REFRESH) * 1e3, 2),
        "timing": (f"{args.steps} steps (one hq_decode_step each; hq_select_vertical at the first step of "
                   f"every 64-step period: {n_refresh} in the window) captured as one HIP graph, replayed once "
                   f"between HIP events; value = the bytes of those launches / the graph's time"),
        "rows_us": {"decode": round(dec_avg_ms * 1e3, 2), "merge": round(merge_ms * 1e3, 2),
                    "select": round(sel_ms * 1e3, 2), "pack": round(pack_ms * 1e3, 2)},
        # the selection's share of the amortised step: hq_select_vertical (rows
        # a1-a3, two passes over the dense keys) as the step runs it, and the
        # decode-time refresh over the hybrid cache in its place
        "select_share": {"per_refresh_vs_step": round(sel_ms / ms_step_plain, 4),
                         "amortized": round(sel_ms / (sel_ms + REFRESH * ms_step_plain), 4),
                         "amortized_decode_time_refresh": round(
                             refresh["us"] * 1e-3 / (refresh["us"] * 1e-3 + REFRESH * ms_step_plain), 4)},
        "select_util": sel_util,
        "decode_time_refresh": refresh,
        "b_sweep": sweep,
        "kv_width_sweep": widths,
        "context_sweep": contexts,
        "gqa16_grid": gqa16,
        "streaming_qwen3_32b": streaming,
        "read_ceiling": ceiling,
        "mfma_rate": mfma,
        "prefill": prefill,
        "capacity": capacity,
        "capacity_ragged_paged": capacity_ragged,
        "replicas": R, "input_gen_s": round(gen_s, 1),
    }
    if ceiling:
        rec["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceiling["read_gbs"], 4)
        fp = ceiling["at_decode_footprint"]
        rec["roofline"]["frac_of_ceiling_at_footprint"] = round(achieved / fp["read_gbs"], 4)
    print(json.dumps(rec))


def refresh_timing(H, torch, wl, dims, caches, pos, qbuf, capture):
    """hq_refresh_hybrid (the decode-time running refresh over the hybrid
    cache, every 64 tokens) at the cache each replica holds now: average of
    back-to-back calls over the replicas, replayed from a HIP graph."""
    B, Hq, Hkv, d, W = wl.B, wl.Hq, wl.Hkv, wl.d, wl.W
    U, G, nb = B * Hkv, Hq // Hkv, qbuf.shape[2]
    R = len(caches)
    ld = max(pos) + 1
    lse = torch.full((B, Hq, nb), 8.0, dtype=torch.float32, device="cuda")
    score = torch.zeros((B, Hkv, ld), dtype=torch.float32, device="cuda")
    flag = torch.zeros((B, Hkv, ld), dtype=torch.uint8, device="cuda")
    cut = torch.zeros((B, Hkv), dtype=torch.float32, device="cuda")
    n_vl_max = H.n_vertical(wl.rho, max(0, ld - W))
    idx = torch.zeros((B, Hkv, max(1, n_vl_max)), dtype=torch.int32, device="cuda")
    ts = [p - 1 for p in pos]                      # each replica's staged position
    n = 2 * R

    def body(stream):
        for i in range(n):
            r = i % R
            H.hq_refresh_hybrid(dims, caches[r], ts[r], qbuf, lse, score, idx, flag, cut, stream=stream)
    g = capture(body)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    t = ts[0]
    n_nw = max(0, t - W)
    n_vl = H.n_vertical(wl.rho, n_nw)
    n_q = n_nw - n_vl
    n_f = n_vl + min(W, t) + 1
    # keys only: K4V4 codes + {scale, min} + position (84 B), FP16 key (256 B,
    # + 4 B position for a vertical line); the score read and written, the
    # top-k pass over it (score read, flags written), queries and LSE in
    byts = (U * (84 * n_q + 256 * n_f + 4 * n_vl + 8 * (t + 1) + 5 * n_nw)
            + B * Hq * nb * (d * 2 + 4))
    flops = 2 * U * (t + 1) * G * nb * d
    return {"us": round(us, 2), "t": t, "nb": nb,
            "hbm_gbs": round(byts / (us * 1e-6) / 1e9, 1),
            "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_F16_TFLOPS, 4),
            "bytes": byts, "flops": flops,
            "per_step_us": round(us / REFRESH, 3)}


def capture_graph(torch, body):
    """body(stream) captured into a HIP graph (through torch) and uploaded."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body(torch.cuda.current_stream())
    graph_upload(g, torch)
    return g


def replay_stats(g, torch, n, reps=5):
    """Per-launch µs of a graph of n launches (already replayed once): the
    median and p90 over `reps` replays, each between HIP events."""
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / n)
    ts.sort()
    return ts[len(ts) // 2], ts[min(len(ts) - 1, math.ceil(0.9 * len(ts)) - 1)]


def graph_decode_us(H, torch, dims, caches, wss, L, q, out, n, reps=5):
    """(median, p90) of the average duration of n back-to-back hq_decode_attn
    launches over the rotating caches, replayed from a captured graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        calls = [H.bind_decode(dims, c, q, out, w, stream=st) for c, w in zip(caches, wss)]
        for i in range(n):
            calls[i % len(calls)](L)
    graph_upload(g, torch)
    g.replay()
    torch.cuda.synchronize()
    return replay_stats(g, torch, n, reps)


def decode_sweep(H, torch, workload, Bs=(1, 4, 16, 32)):
    """The metric's batch sweep on the Qwen3-8B-shaped layer (32/8 heads,
    L = 32768, W = 128, rho = 5 %): decode launches only, caches built on the
    device from bf16-rounded N(0,1) keys and values (timing inputs; parity is
    covered by the tests), each then holding one staged token as in a step."""
    pts = [decode_point(H, torch, workload, B) for B in Bs]
    for p in pts:
        # HBM bytes of the launch from the committed counter runs, where one
        # was taken at this batch on the current decode source
        t = load_traffic("qwen3_8b", p["B"])
        if t is not None:
            p["traffic"] = t
            p["traffic_over_algorithmic"] = round(t / p["bytes"], 4)
    return pts


def width_sweep(H, torch, workload, points=((1, 8, 8), (1, 4, 2), (1, 2, 4), (32, 8, 8), (32, 4, 2), (32, 2, 4))):
    """Decode of the other strict low-bit caches (K8V8, K4V2, K2V4, with
    vertical lines and window) on the same layer: µs and GB/s of each width's
    own algorithmic bytes (16 (k_bits + v_bits) + 32 per quantised token)."""
    return [decode_point(H, torch, workload, B, kb, vb) for B, kb, vb in points]


def context_sweep(H, torch, workload, Ls=(1024, 2048, 4096, 8192, 16384, 32768)):
    """Decode of the Llama-3.1-8B-shaped layer (B = 1) at the prefix lengths
    of the pages' latency table, for comparison with its shape only."""
    return [decode_point(H, torch, workload, 1, name="llama31_8b", L=L) for L in Ls]


def gqa16_grid(H, torch, workload, Ls=(1024, 4096, 16384, 32768), rhos=(0.01, 0.05, 0.10)):
    """GLM-4-9B-shaped layer (32 query heads on 2 KV heads, B = 8): decode
    µs and GB/s over prefix length and rho; at L = 32K the selection is timed
    too (its two passes are MFMA-heavy at 16 query heads per KV head)."""
    return [decode_point(H, torch, workload, 8, name="glm4_9b", select=(L == max(Ls)), L=L, rho=r)
            for L in Ls for r in rhos]


def streaming_run(H, torch, workload, steps=128):
    """A Qwen3-32B-shaped layer (B = 32, 64/8 heads) streaming 128 tokens
    from a 32K prefix: per-step µs of the merge and the decode on their own,
    of the two as separate launches, and of hq_decode_step, each from a graph
    of the 128 steps replayed once on a fresh copy of the cache (one launch
    moves 1.5 GB, past the Infinity Cache)."""
    wl = workload("qwen3_32b")
    B, Hq, Hkv, L, W, rho, d = wl.B, wl.Hq, wl.Hkv, wl.L, wl.W, wl.rho, 128
    U = B * Hkv
    g = torch.Generator(device="cuda").manual_seed(32)
    K = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
    V = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
    qb = torch.randn((B, Hq, 64, d), generator=g, device="cuda").half()
    dims_s = H.make_dims(B, Hq, Hkv, W, rho)
    n_nw = L - W
    n_vl = H.n_vertical(rho, n_nw)
    score = torch.zeros((B, Hkv, L), device="cuda")
    idx = torch.zeros((B, Hkv, n_vl), dtype=torch.int32, device="cuda")
    flag = torch.zeros((B, Hkv, L), dtype=torch.uint8, device="cuda")
    H.hq_select_vertical(dims_s, qb, K, L, score, idx, flag, H.workspace(dims_s, H.HQ_OP_SELECT, L))
    base = H.HybridCache.allocate(B, Hq, Hkv, W, rho, L + steps + 2)
    H.hq_quant_pack(base.dims, K, V, L, flag, base)
    del K, V, qb, score, idx, flag
    kn = torch.randn((steps, B, Hkv, d), generator=g, device="cuda").half()
    vn = torch.randn((steps, B, Hkv, d), generator=g, device="cuda").half()
    qn = torch.randn((steps, B, Hq, d), generator=g, device="cuda").half()
    out = torch.empty((B, Hq, d), dtype=torch.float16, device="cuda")
    dims = base.dims
    ws = H.workspace(dims, H.HQ_OP_DECODE, L + steps + 2)
    kp = [kn[i].data_ptr() for i in range(steps)]
    vp = [vn[i].data_ptr() for i in range(steps)]
    qp = [qn[i].data_ptr() for i in range(steps)]
    # warm every kernel once on a throwaway copy
    w = base.clone()
    H.hq_decode_step(dims, w, L, kn[0], vn[0], qn[0], out, ws)
    H.hq_append_merge(dims, w, L + 1, kn[1], vn[1])
    H.hq_decode_attn(dims, w, L + 1, qn[1], out, ws)
    torch.cuda.synchronize()
    del w

    def once(body):
        c = base.clone()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            body(c, torch.cuda.current_stream())
        graph_upload(gr, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        del gr
        return us, c

    def fused(c, st):
        f = H.bind_step(dims, c, qn[0], out, ws, stream=st)
        for i in range(steps):
            f(L + i, kp[i], vp[i], qp[i])

    def unfused(c, st):
        m = H.bind_merge(dims, c, stream=st)
        dq = H.bind_decode(dims, c, qn[0], out, ws, stream=st)
        for i in range(steps):
            m(L + i, kp[i], vp[i])
            dq(L + i, qp[i])

    def merges(c, st):
        m = H.bind_merge(dims, c, stream=st)
        for i in range(steps):
            m(L + i, kp[i], vp[i])

    step_us, _ = once(fused)
    unfused_us, _ = once(unfused)
    merge_us, cm = once(merges)

    def decodes(c, st):
        dq = H.bind_decode(dims, cm, qn[0], out, ws, stream=st)
        for i in range(steps):
            dq(L + steps - 1, qp[i])
    decode_us, _ = once(decodes)
    # algorithmic bytes at the middle of the run: the decode reads the K4V4
    # tokens, the FP16 lines, window and staged token, q in and out; the merge
    # reads the leaving token and writes its K4V4 slot and the ring slot
    n_q_mid = (n_nw - n_vl) + steps // 2
    dec_bytes = U * (160 * n_q_mid + 512 * (n_vl + W + 1)) + B * Hq * d * 4
    merge_bytes = U * (512 + 160 + 512)
    res = {"workload": "Qwen3-32B-shaped layer, B=32, 64/8 heads, 128 steps from L=32768", "W": W,
           "rho": rho, "steps": steps, "step_us": round(step_us, 2), "unfused_us": round(unfused_us, 2),
           "decode_us": round(decode_us, 2), "merge_us": round(merge_us, 2),
           "step_GBs": round((dec_bytes + merge_bytes) / (step_us * 1e-6) / 1e9, 1),
           "decode_GBs": round(dec_bytes / (decode_us * 1e-6) / 1e9, 1),
           "decode_frac": round(dec_bytes / (decode_us * 1e-6) / 1e9 / PEAK_GBS, 4),
           "bytes_per_step": dec_bytes + merge_bytes,
           "timing": "each variant: the 128 steps as one graph, replayed once on a fresh copy of the cache"}
    del base, cm, kn, vn, qn, ws
    torch.cuda.empty_cache()
    return res


_PLANTED = {}                      # planted host inputs of the last selection-timed shape


def decode_point(H, torch, workload, B, kb=4, vb=4, name="qwen3_8b", select=False, **over):
    """Decode launches of one workload shape (the named layer at batch B,
    with overrides such as L and rho): cache built on the device from
    bf16-rounded N(0,1) keys and values by select + pack + one merge, then
    rotated over replicas of at least 1 GiB in all; µs (median and p90 over
    graph replays) and GB/s of the algorithmic bytes.  With select=True the
    selection over the same prefix is timed too, with its share of the step
    at one refresh per 64 decodes; its keys, values and buffered queries are
    then the workload's planted ones (hq_inputs)."""
    d = 128
    if True:
        wl = workload(name, B=B, **over)
        Hq, Hkv, L, W, rho = wl.Hq, wl.Hkv, wl.L, wl.W, wl.rho
        U = B * Hkv
        g = torch.Generator(device="cuda").manual_seed(1000 + B)
        if select and name != "qwen3_8b":
            # the selection's timing depends on the score distribution (the
            # top-k brackets its cut-off from a sample): the workload's own
            # planted generator, shared by the points of one shape
            key = (name, B, L)
            if key not in _PLANTED:
                _PLANTED.clear()
                from hq_inputs import batch
                x = batch(wl, steps=1)
                _PLANTED[key] = tuple(torch.from_numpy(np.ascontiguousarray(x[k])) for k in ("K", "V", "qbuf"))
            K, V, qb = (t.to("cuda") for t in _PLANTED[key])
        else:
            K = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
            V = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
            qb = torch.randn((B, Hq, 64, d), generator=g, device="cuda").half()
        dims_s = H.make_dims(B, Hq, Hkv, W, rho)
        n_nw = L - W
        n_vl = H.n_vertical(rho, n_nw)
        score = torch.zeros((B, Hkv, L), device="cuda")
        idx = torch.zeros((B, Hkv, n_vl), dtype=torch.int32, device="cuda")
        flag = torch.zeros((B, Hkv, L), dtype=torch.uint8, device="cuda")
        ws_s = H.workspace(dims_s, H.HQ_OP_SELECT, L)
        H.hq_select_vertical(dims_s, qb, K, L, score, idx, flag, ws_s)
        sel_us = sel1_us = None
        if select:
            # both passes, and the column-mass pass alone with the rows' LSE
            # handed over as the producing attention would (a constant here:
            # timing only)
            lse_c = torch.full((B, Hq, 64), 8.0, dtype=torch.float32, device="cuda")

            def sel_graph(lse_in):
                torch.cuda.synchronize()
                gs = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gs):
                    st = torch.cuda.current_stream()
                    for _ in range(8):
                        H.hq_select_vertical(dims_s, qb, K, L, score, idx, flag, ws_s, lse=lse_in, stream=st)
                graph_upload(gs, torch)
                gs.replay()
                torch.cuda.synchronize()
                return replay_stats(gs, torch, 8, 3)[0]
            sel_us = sel_graph(None)
            sel1_us = sel_graph(lse_c)
            H.hq_select_vertical(dims_s, qb, K, L, score, idx, flag, ws_s)
            qb_keep = qb
        base = H.HybridCache.allocate(B, Hq, Hkv, W, rho, L + 8, k_bits=kb, v_bits=vb)
        H.hq_quant_pack(base.dims, K, V, L, flag, base)
        H.hq_append_merge(base.dims, base, L, K[:, :, 0].contiguous(), V[:, :, 0].contiguous())
        del K, V, qb, score, idx, flag
        q_tok = 16 * (kb + vb) + 32
        footprint = U * (q_tok * (n_nw - n_vl) + 512 * (n_vl + W + 1))
        R = min(256, max(1, math.ceil((1 << 30) / footprint)))
        caches = [base] + [base.clone() for _ in range(R - 1)]
        wss = [H.workspace(base.dims, H.HQ_OP_DECODE, L + 8) for _ in range(R)]
        q = torch.randn((B, Hq, d), generator=g, device="cuda").half()
        out = torch.empty_like(q)
        us, p90 = graph_decode_us(H, torch, base.dims, caches, wss, L + 1, q, out, max(2 * R, 32))
        ref_us = None
        if select:
            ref_us = refresh_timing(H, torch, wl, base.dims, caches, [L + 1] * R, qb_keep,
                                    lambda body: capture_graph(torch, body))["us"]
            del qb_keep
        nbytes = U * (q_tok * (n_nw - n_vl) + 512 * (n_vl + W + 1)) + B * Hq * d * 4
        gbs = nbytes / (us * 1e-6) / 1e9
        res = {"B": B, "decode_us": round(us, 2), "p90_us": round(p90, 2), "GBs": round(gbs, 1),
               "frac": round(gbs / PEAK_GBS, 4), "bytes": nbytes, "replicas": R}
        if name != "qwen3_8b" or over:
            res.update({"L": L, "rho": rho})
        if (kb, vb) != (4, 4):
            res["kv_bits"] = f"K{kb}V{vb}"
        if sel_us is not None:
            share = lambda x: round(x / (x + REFRESH * us), 4)
            res.update({"select_us": round(sel_us, 2), "select_share_amortized": share(sel_us),
                        "select_given_lse_us": round(sel1_us, 2), "select_given_lse_share": share(sel1_us),
                        "decode_time_refresh_us": round(ref_us, 2), "decode_time_refresh_share": share(ref_us)})
        del caches, wss, base
        torch.cuda.empty_cache()
    return res


def prefill_timing(H, torch, L=32768, n=3):
    """hq_prefill_attn on the Llama-3.1-8B-shaped layer (B = 1, 32/8 heads,
    d = 128, W = 128) at a 32K prefix: bf16-rounded N(0,1) device inputs,
    the vertical lines chosen by hq_select_vertical from the last 64 queries
    (rho = 5 %), n calls captured in a graph and replayed once between HIP
    events.  Algorithmic work: the causal QK and PV products, 4 d Hq L (L+1)/2
    flop; QK runs on INT8 codes for all but the window and line keys, PV on
    FP16, so the ceiling is between the FP16 peak (2.5 PFLOP/s) and, with
    every QK product at the INT8 rate, 1 / (0.5/5.0 + 0.5/2.5) = 3.33 P/s."""
    B, Hq, Hkv, d, W, rho = 1, 32, 8, 128, 128, 0.05
    g = torch.Generator(device="cuda").manual_seed(2024)
    q = torch.randn((B, Hq, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
    k = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
    v = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
    dims = H.make_dims(B, Hq, Hkv, W, rho)
    n_vl = H.n_vertical(rho, L - W)
    score = torch.zeros((B, Hkv, L), device="cuda")
    idx = torch.zeros((B, Hkv, n_vl), dtype=torch.int32, device="cuda")
    flag = torch.zeros((B, Hkv, L), dtype=torch.uint8, device="cuda")
    qtail = q[:, :, L - 64:].contiguous()
    H.hq_select_vertical(dims, qtail, k, L, score, idx, flag, H.workspace(dims, H.HQ_OP_SELECT, L))
    ws = H.workspace(dims, H.HQ_OP_PREFILL, L)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), device="cuda")
    H.hq_prefill_attn(dims, q, k, v, L, flag, out, ws, lse=lse)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        st = torch.cuda.current_stream()
        for _ in range(n):
            H.hq_prefill_attn(dims, q, k, v, L, flag, out, ws, lse=lse, stream=st)
    graph_upload(gr, torch)
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 4.0 * d * Hq * B * L * (L + 1) / 2
    tf = flops / (ms * 1e-3) / 1e12
    mixed_peak = 1.0 / (0.5 / PEAK_I8_TOPS + 0.5 / PEAK_F16_TFLOPS)
    res = {"workload": "Llama-3.1-8B-shaped layer, B=1", "L": L, "W": W, "rho": rho,
           "n_vertical_per_head": n_vl, "ms": round(ms, 3), "flop": flops, "tflops": round(tf, 1),
           "frac_of_fp16_peak": round(tf / PEAK_F16_TFLOPS, 4),
           "frac_of_int8_qk_fp16_pv_peak": round(tf / mixed_peak, 4),
           "timing": f"{n} calls (INT8 rows of q and k, line lists, attention) in one graph, replayed once"}
    del gr, q, k, v, out, lse, ws, score, idx, flag
    torch.cuda.empty_cache()
    return res


def capacity_run(H, torch, steps=4, L=32768, W=128, rho=0.05, reserve=8 << 30, n_var=4):
    """Attention of a whole Qwen3-8B-shaped model (36 layers, 32/8 heads) at
    the largest batch of 32K-token prefixes whose hybrid caches fit this GPU
    beside the model's 16-bit weights and a reserve.  The weights are not
    allocated (only the attention path runs).  Each layer's cache is built by
    hq_select_vertical + hq_quant_pack one sequence at a time, from n_var
    independent bf16-rounded N(0,1) prefixes.  A token step is
    hq_decode_step (the staging merge and the decode in one launch) in every
    layer for the whole batch; K steps are captured in one graph and replayed
    once between HIP events, and a graph of one step's plain decodes gives
    the decode share."""
    from hybrid_precision_attention_amd.model_cache import QWEN3_8B as shape, ModelCache, plan_capacity
    d, Hq, Hkv = shape.d, shape.Hq, shape.Hkv
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    L_max = L + steps + 1
    plan = plan_capacity(shape, L_max, W, rho, total, reserve_bytes=reserve)
    per_seq = plan["hybrid_bytes_per_seq"]
    B = int(min(plan["max_batch_hybrid"], (free - (6 << 30)) // per_seq))
    res = {"model": f"{shape.name} attention, {shape.layers} layers", "L": L, "W": W, "rho": rho,
           "hbm_bytes": total, "weights_bytes_set_aside": shape.weight_bytes, "reserve_bytes": reserve,
           "hybrid_bytes_per_seq": per_seq, "fp16_bytes_per_seq": plan["fp16_bytes_per_seq"],
           "max_batch_hybrid": plan["max_batch_hybrid"], "max_batch_fp16": plan["max_batch_fp16"]}
    if B < 1:
        res["skipped"] = "no room for one sequence"
        return res
    t0 = time.time()
    g = torch.Generator(device="cuda").manual_seed(77)
    dims1 = H.make_dims(1, Hq, Hkv, W, rho)
    n_nw = L - W
    n_vl = H.n_vertical(rho, n_nw)
    ws_sel = H.workspace(dims1, H.HQ_OP_SELECT, L)
    variants = []
    for _ in range(n_var):
        K = torch.randn((1, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
        V = torch.randn((1, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16).half()
        qb = torch.randn((1, Hq, 64, d), generator=g, device="cuda").half()
        score = torch.zeros((1, Hkv, L), device="cuda")
        idx = torch.zeros((1, Hkv, n_vl), dtype=torch.int32, device="cuda")
        flag = torch.zeros((1, Hkv, L), dtype=torch.uint8, device="cuda")
        H.hq_select_vertical(dims1, qb, K, L, score, idx, flag, ws_sel)
        variants.append((K, V, flag))
    mc = ModelCache(shape, B, L_max, W, rho)
    for l, c in enumerate(mc.layers):
        for b in range(B):
            K, V, flag = variants[(l + b) % n_var]
            v = c.view(b)
            H.hq_quant_pack(v.dims, K, V, L, flag, v)
    torch.cuda.synchronize()
    del variants, ws_sel
    build_s = time.time() - t0

    k_new = [torch.randn((B, Hkv, d), generator=g, device="cuda").half() for _ in range(shape.layers)]
    v_new = [torch.randn((B, Hkv, d), generator=g, device="cuda").half() for _ in range(shape.layers)]
    q = [torch.randn((B, Hq, d), generator=g, device="cuda").half() for _ in range(shape.layers)]
    out = torch.empty((B, Hq, d), dtype=torch.float16, device="cuda")
    ws = H.workspace(mc[0].dims, H.HQ_OP_DECODE, L_max)

    def binds(stream):
        dec = [H.bind_decode(c.dims, c, q[l], out, ws, stream=stream) for l, c in enumerate(mc.layers)]
        stp = [H.bind_step(c.dims, c, q[l], out, ws, stream=stream) for l, c in enumerate(mc.layers)]
        return dec, stp

    dec, _ = binds(torch.cuda.current_stream())
    for f in dec:                   # warm-up: one decode per layer over the packed prefix
        f(L)
    torch.cuda.synchronize()

    def capture(body):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            body(torch.cuda.current_stream())
        graph_upload(gr, torch)
        return gr

    def token_steps(stream):
        _, stp_s = binds(stream)
        for s in range(steps):
            for l in range(shape.layers):
                stp_s[l](L + s, k_new[l].data_ptr(), v_new[l].data_ptr())

    def decode_step(stream):
        dec_s, _ = binds(stream)
        for l in range(shape.layers):
            dec_s[l](L + steps - 1)

    g_steps = capture(token_steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g_steps.replay()
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    g_dec = capture(decode_step)
    g_dec.replay()
    torch.cuda.synchronize()
    e0.record()
    g_dec.replay()
    e1.record()
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1)
    U = B * Hkv
    n_q = n_nw - n_vl + steps
    dec_bytes = shape.layers * (U * (160 * n_q + 512 * (n_vl + W + 1)) + B * Hq * d * 4)
    res.update({"batch": B, "cache_bytes": mc.nbytes(), "build_s": round(build_s, 1), "steps": steps,
                "token_step_ms": round(step_ms, 3), "decode_ms": round(dec_ms, 3),
                "merge_ms": round(step_ms - dec_ms, 3),
                "attn_tokens_per_s": round(B / (step_ms * 1e-3), 1),
                "decode_bytes": dec_bytes,
                "decode_GBs": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
                "decode_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / PEAK_GBS, 4),
                "timing": "K token steps (hq_decode_step in every layer) as one graph, replayed once"})
    del g_steps, g_dec, mc, ws, k_new, v_new, q, out
    torch.cuda.empty_cache()
    return res


def capacity_ragged_run(H, torch, steps=4, L_cap=32768, W=128, rho=0.05, reserve=8 << 30, seed=31):
    """The capacity run's model (Qwen3-8B-shaped attention, 36 layers) with
    paged K4V4 slots and a ragged batch: sequence lengths drawn (seeded) from
    {4096, 8192, ..., 32768}, sequences added while their paged caches fit
    the same HBM budget as the uniform run (each owns K4V4 blocks only for
    its own length).  Caches built by select + pack per sequence; a token
    step is hq_decode_step_ragged in every layer, K steps from one graph."""
    from hybrid_precision_attention_amd.model_cache import (QWEN3_8B as shape, paged_layer_bytes_per_sequence,
                                                            plan_capacity)
    d, Hq, Hkv = shape.d, shape.Hq, shape.Hkv
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    budget = min(total - shape.weight_bytes - reserve, free - (6 << 30))
    L_alloc = L_cap + steps + 1
    choices = list(range(4096, L_cap + 1, 4096))
    rng = np.random.default_rng(seed)
    lens, used = [], 0
    while True:
        Lb = int(rng.choice(choices))
        need = shape.layers * paged_layer_bytes_per_sequence(shape, Lb + steps + 1, L_alloc, W, rho,
                                                             extra_vl=steps + 1)
        if used + need + shape.layers * (1 << 20) > budget:
            break
        lens.append(Lb)
        used += need
    B = len(lens)
    uniform = plan_capacity(shape, L_alloc, W, rho, total, reserve_bytes=reserve)["max_batch_hybrid"]
    res = {"model": f"{shape.name} attention, {shape.layers} layers, paged K4V4 slots",
           "lengths": "uniform over {4096, 8192, ..., 32768} (seeded)", "W": W, "rho": rho,
           "batch": B, "mean_L": round(float(np.mean(lens)), 1) if lens else 0,
           "uniform_32k_batch_same_budget": uniform}
    if B < 1:
        res["skipped"] = "no room for one sequence"
        return res
    t0 = time.time()
    g = torch.Generator(device="cuda").manual_seed(78)
    dims1 = H.make_dims(1, Hq, Hkv, W, rho)
    K = torch.randn((1, Hkv, L_cap, d), generator=g, device="cuda").to(torch.bfloat16).half()
    V = torch.randn((1, Hkv, L_cap, d), generator=g, device="cuda").to(torch.bfloat16).half()
    qb = torch.randn((1, Hq, 64, d), generator=g, device="cuda").half()
    n_vl = H.n_vertical(rho, L_cap - W)
    score = torch.zeros((1, Hkv, L_cap), device="cuda")
    idx = torch.zeros((1, Hkv, n_vl), dtype=torch.int32, device="cuda")
    flag = torch.zeros((1, Hkv, L_cap), dtype=torch.uint8, device="cuda")
    H.hq_select_vertical(dims1, qb, K, L_cap, score, idx, flag, H.workspace(dims1, H.HQ_OP_SELECT, L_cap))
    pre = {}                              # dense prefixes, one contiguous copy per length
    for Lb in sorted(set(lens)):
        f = flag[:, :, :Lb].clone()
        f[:, :, max(0, Lb - W):] = 0
        pre[Lb] = (K[:, :, :Lb].contiguous(), V[:, :, :Lb].contiguous(), f)
    del K, V, score, idx, flag
    seq_max = [Lb + steps + 1 for Lb in lens]
    layers = []
    for l in range(shape.layers):
        c = H.HybridCache.allocate_paged(B, Hq, Hkv, W, rho, L_alloc, extra_vl=steps + 1, seq_L_max=seq_max)
        for b, Lb in enumerate(lens):
            v = c.view(b)
            Kb, Vb, fb = pre[Lb]
            H.hq_quant_pack(v.dims, Kb, Vb, Lb, fb, v)
        layers.append(c)
    torch.cuda.synchronize()
    del pre
    build_s = time.time() - t0
    cache_bytes = sum(c.nbytes() for c in layers)
    k_new = [torch.randn((B, Hkv, d), generator=g, device="cuda").half() for _ in range(shape.layers)]
    v_new = [torch.randn((B, Hkv, d), generator=g, device="cuda").half() for _ in range(shape.layers)]
    q = [torch.randn((B, Hq, d), generator=g, device="cuda").half() for _ in range(shape.layers)]
    out = torch.empty((B, Hq, d), dtype=torch.float16, device="cuda")
    ws = H.workspace(layers[0].dims, H.HQ_OP_DECODE, L_alloc)
    t_dev = [torch.tensor([Lb + s_ for Lb in lens], dtype=torch.int32, device="cuda") for s_ in range(steps)]
    t_max = [max(lens) + s_ for s_ in range(steps)]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        st = torch.cuda.current_stream()
        for s_ in range(steps):
            for l, c in enumerate(layers):
                H.hq_decode_step_ragged(c.dims, c, t_dev[s_], t_max[s_], k_new[l], v_new[l], q[l], out, ws,
                                        stream=st)
    graph_upload(gr, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    gr.replay()
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    # algorithmic decode bytes of a step: each unit's K4V4 and FP16 tokens at its own length
    dec_bytes = 0
    for Lb in lens:
        n_nw = max(0, Lb + steps // 2 - W)
        nv = H.n_vertical(rho, max(0, Lb - W))
        dec_bytes += Hkv * (160 * (n_nw - nv) + 512 * (nv + min(W, Lb) + 1))
    dec_bytes = shape.layers * (dec_bytes + B * Hq * d * 4)
    res.update({"cache_bytes": cache_bytes, "build_s": round(build_s, 1), "steps": steps,
                "token_step_ms": round(step_ms, 3),
                "attn_tokens_per_s": round(B / (step_ms * 1e-3), 1),
                "step_bytes": dec_bytes, "step_GBs": round(dec_bytes / (step_ms * 1e-3) / 1e9, 1),
                "timing": "K token steps (hq_decode_step_ragged in every layer) as one graph, replayed once"})
    del gr, layers, ws, k_new, v_new, q, out
    torch.cuda.empty_cache()
    return res


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "hybrid_precision_attention_amd", "libhq_probe.so"))
    for f in (lib.hq_probe_stream_read, lib.hq_probe_stream_read_nt):
        f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int,
                      ctypes.c_void_p]
    return {"ordinary": lib.hq_probe_stream_read, "nt": lib.hq_probe_stream_read_nt}


def mfma_rate(torch, iters=2048):
    """The matrix-core rate probe (libhq_probe.so): fp16 MFMA chains of the
    16x16x32 and 32x32x16 shapes, alone and with the column-mass exponential
    work interleaved, at two and four waves per SIMD; TFLOP/s of each."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "hybrid_precision_attention_amd", "libhq_probe.so"))
    lib.hq_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    names = {0: "16x16x32", 1: "32x32x16", 2: "16x16x32+exp_mix", 3: "32x32x16+exp_mix"}
    res = {}
    for which, name in names.items():
        flop_per = (8 * 16384) if which in (0, 2) else (4 * 32768)
        best = 0.0
        for wps in (2, 4):                        # waves per SIMD: 256 CUs x wps workgroups of 4 waves
            grid = 256 * wps
            for _ in range(2):
                if lib.hq_probe_mfma_rate(which, grid, iters, sink.data_ptr(), s):
                    raise RuntimeError("mfma probe launch failed")
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lib.hq_probe_mfma_rate(which, grid, iters, sink.data_ptr(), s)
            e1.record()
            torch.cuda.synchronize()
            tflops = grid * 4 * iters * flop_per / (e0.elapsed_time(e1) * 1e-3) / 1e12
            best = max(best, tflops)
        res[name] = round(best, 1)
    res["kernel"] = "mfma_rate_kernel (libhq_probe.so): independent fp16 MFMA chains, best of 2 and 4 waves per SIMD"
    return res


def read_ceiling(torch, nbytes=1 << 30):
    """A plain streaming read of nbytes (libhq_probe.so: 16-byte loads, eight
    in flight per thread, every word consumed) on the same device: the
    achievable-bandwidth reference beside the nominal peak.  Both load
    policies (ordinary, and the non-temporal one the decode uses) at a few
    grid sizes; the best is reported, with each policy's best beside it."""
    fns = _probe_lib()
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    best, per = None, {}
    for pol, fn in fns.items():
        for grid in (2048, 4096, 8192, 16384, 32768):
            def run():
                if fn(x.data_ptr(), nbytes, sink.data_ptr(), 0x9E3779B9, grid, s):
                    raise RuntimeError("stream probe launch failed")
            for _ in range(2):
                run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 10
            e0.record()
            for _ in range(n):
                run()
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes / (e0.elapsed_time(e1) / n * 1e-3) / 1e9
            per[pol] = max(per.get(pol, 0.0), round(gbs, 1))
            if best is None or gbs > best[0]:
                best = (gbs, grid, pol)
    del x
    return {"read_gbs": round(best[0], 1), "bytes": nbytes, "grid": best[1], "policy": best[2],
            "read_gbs_by_policy": per,
            "kernel": "stream_read_kernel (libhq_probe.so): 16-byte loads, 256-thread workgroups"}


def read_ceiling_footprint(torch, footprint):
    """The same streaming read at the decode's footprint: back-to-back
    launches over R = ceil(1 GiB / footprint) buffers (so each launch reads
    from HBM, not the Infinity Cache), replayed from a HIP graph; the best of
    both load policies and a few grid sizes.  What one launch of that size
    can reach, latency included."""
    fns = _probe_lib()
    nbytes = (footprint + 255) // 256 * 256
    R = max(2, math.ceil((1 << 30) / nbytes))
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(R)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = None
    for pol, fn in fns.items():
        for grid in (256, 512, 1024, 2048, 4096):
            n = 2 * R
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                s = torch.cuda.current_stream().cuda_stream
                for i in range(n):
                    if fn(bufs[i % R].data_ptr(), nbytes, sink.data_ptr(), 0x9E3779B9, grid, s):
                        raise RuntimeError("stream probe launch failed")
            graph_upload(g, torch)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            if best is None or us < best[0]:
                best = (us, grid, pol)
            del g
    del bufs
    return {"read_gbs": round(nbytes / (best[0] * 1e-6) / 1e9, 1), "us": round(best[0], 2),
            "bytes": nbytes, "grid": best[1], "policy": best[2], "buffers": R,
            "kernel": "stream_read_kernel (libhq_probe.so), launches of the decode's byte count"}


def cpu_baseline(wl, cache, H, torch):
    """Time the fp64 oracle on whole decode steps of the same cache (every
    unit merges a new token, then decodes) until about 10 s of CPU work, and
    report it in the metric's unit."""
    from oracle import hq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    B, Hkv, G, L, W, d = wl.B, wl.Hkv, wl.G, wl.L, wl.W, wl.d
    rng = np.random.default_rng(0)
    caches = []
    for b in range(B):
        for g in range(Hkv):
            t = {k: (v[b, g].cpu().numpy() if v is not None else None) for k, v in cache.t.items()}
            nq, nvl = int(t["n_q"]), int(t["n_vl"])
            c = O.empty_unit_cache(d, W)
            c["kq"], c["vq"] = t["kq"][:nq], t["vq"][:nq]
            c["kq_meta"], c["vq_meta"], c["q_pos"] = t["kq_meta"][:nq], t["vq_meta"][:nq], t["q_pos"][:nq]
            c["kvl"], c["vvl"], c["vl_pos"] = t["kvl"][:nvl], t["vvl"][:nvl], t["vl_pos"][:nvl]
            if W:
                c["kwin"], c["vwin"] = t["kwin"], t["vwin"]
            caches.append(c)
    steps, nbytes, t_cpu = 0, 0, 0.0
    while t_cpu < 10.0 and steps < 500:
        pos = L + steps
        for c in caches:
            q = rng.standard_normal((G, d)).astype(np.float16)
            kn = rng.standard_normal(d).astype(np.float16)
            t0 = time.perf_counter()
            O.append_merge_unit(c, pos, kn, kn)
            O.decode_fused(c, q, pos)
            t_cpu += time.perf_counter() - t0
            n_win = min(W, pos)
            nbytes += 160 * c["kq"].shape[0] + 512 * (c["kvl"].shape[0] + n_win + 1) + G * d * 4
        steps += 1
    return {"value": round(nbytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle merge + fused decode, {steps} whole decode steps of all "
                      f"{len(caches)} (sequence, KV head) units of the same cache, {t_cpu:.1f} s CPU; "
                      f"GB/s of the same algorithmic bytes"}


if __name__ == "__main__":
    main()
