"""GPU parity of the prefill hybrid-precision attention (hq_quant_int8,
hq_prefill_attn) against the fp64 oracle: INT8 codes and scales bit-exact;
outputs within max-abs 2e-3 / rel-L2 1e-3 and the LSE within the decode
bound, on seeded planted-line inputs over every GQA layout the kernel maps
(G = 1, 2, 3, 4, 8, 16), ragged lengths, W = 0 and W >= L, no / all / planted
vertical lines, more than one 64-entry tile of lines, and the full
Llama-3.1-8B-shaped 32K prefix on sampled query rows."""
import numpy as np
import pytest
import torch

import hybrid_precision_attention_amd as H
from hq_inputs import batch, prefill_queries, workload
from oracle import hq_oracle as O

from gpu_util import check_decode, dev

pytestmark = pytest.mark.gpu


def _flags(wl, x, frac_extra=0.0, seed=0):
    """Vertical-line flags: the planted positions (non-window prefix), plus a
    seeded random fraction of the prefix."""
    B, Hkv, L = wl.B, wl.Hkv, wl.L
    f = np.zeros((B, Hkv, L), np.uint8)
    rng = np.random.default_rng(seed)
    for b in range(B):
        pl = x["plant"][b]
        f[b, :, pl[pl < L]] = 1
        if frac_extra:
            f[b] |= (rng.random((Hkv, L)) < frac_extra).astype(np.uint8)
    return f


def _run(wl, Q, x, flag, lse=True):
    B, Hq, L = wl.B, wl.Hq, wl.L
    dims = H.make_dims(B, Hq, wl.Hkv, wl.W, wl.rho)
    ws = H.workspace(dims, H.HQ_OP_PREFILL, L)
    out = torch.empty((B, Hq, L, 128), dtype=torch.float16, device="cuda")
    lt = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda") if lse else None
    H.hq_prefill_attn(dims, dev(Q), dev(x["K"]), dev(x["V"]), L,
                      dev(flag) if flag is not None else None, out, ws, lse=lt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lt.cpu().numpy() if lse else None)


def _inputs(name, **over):
    wl = workload(name, **over)
    x = batch(wl)
    Q = np.stack([prefill_queries(wl, b) for b in range(wl.B)])
    return wl, x, Q


def test_quant_int8_bit_exact():
    rng = np.random.default_rng(11)
    rows = 1000 + 7                       # not a multiple of the 16 rows a workgroup takes
    x = (rng.standard_normal((rows, 128)) * rng.choice([1e-4, 1.0, 30.0, 2e3], size=(rows, 1)))
    x = np.clip(x, -6e4, 6e4).astype(np.float16)
    x[5] = 0
    x[6] = (np.arange(128) - 64 + 0.5).astype(np.float16)      # exact half-integer quotients
    x[6, 0] = 127
    x[7, :] = np.float16(6.1e-5)                                # subnormal-range scale
    xd = dev(x)
    codes = torch.empty((rows, 128), dtype=torch.int8, device="cuda")
    scales = torch.empty(rows, dtype=torch.float32, device="cuda")
    H.hq_quant_int8(xd, codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = O.int8_quantize_rows(x)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


CASES = [
    # name, overrides, W override, flag mode
    ("tiny", {"L": 300}, None, "planted"),                      # G = 4, ragged tail
    ("tiny", {"L": 300, "B": 2}, 64, "planted+5%"),            # two sequences, W = 64
    ("tiny", {"L": 257, "Hq": 4}, 32, "planted+5%"),           # G = 2 (two position blocks)
    ("tiny", {"L": 130, "Hq": 2}, 0, "planted+5%"),            # G = 1, no window
    ("tiny", {"L": 150, "Hq": 6}, 16, "planted"),              # G = 3 (one head per workgroup)
    ("glm4_9b", {"L": 200, "B": 1}, None, "planted"),          # G = 16
    ("qwen3_32b", {"L": 333, "B": 1}, 128, "planted+5%"),      # G = 8
    ("tiny", {"L": 1000}, 128, "planted+10%"),                 # many far tiles, >64 lines
    ("tiny", {"L": 200}, 0, "none"),                           # INT8 everywhere
    ("tiny", {"L": 200}, 512, "none"),                         # window >= L: FP16 everywhere
    ("tiny", {"L": 200}, 0, "all"),                            # every key a vertical line
    ("tiny", {"L": 1}, None, "planted"),                       # one token
    ("tiny", {"L": 65}, 1, "planted+5%"),                      # window of one (only the diagonal)
]


@pytest.mark.parametrize("name,over,W,mode", CASES)
def test_prefill_parity(name, over, W, mode):
    if W is not None:
        over = dict(over, W=W)
    wl, x, Q = _inputs(name, **over)
    print(f"case {name} {over} {mode}", flush=True)
    if mode == "none":
        flag = None
    elif mode == "all":
        flag = np.ones((wl.B, wl.Hkv, wl.L), np.uint8)
    else:
        extra = {"planted": 0.0, "planted+5%": 0.05, "planted+10%": 0.10}[mode]
        flag = _flags(wl, x, extra)
    o, l = _run(wl, Q, x, flag)
    ref_o, ref_l = O.prefill_hybrid(Q, x["K"], x["V"], flag, wl.W)
    check_decode(o, l, ref_o, ref_l, tag=f"{name} {over} {mode}")


def test_prefill_without_lse_and_repeatable():
    wl, x, Q = _inputs("tiny", L=400)
    flag = _flags(wl, x, 0.05)
    o1, _ = _run(wl, Q, x, flag, lse=False)
    o2, l2 = _run(wl, Q, x, flag)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


def test_prefill_full_size_sampled_rows():
    """The Llama-3.1-8B-shaped 32K prefix (32/8 heads, W = 128, planted lines
    plus the selection's 5 %): every row is computed on the GPU, sampled rows
    (the first, the last 64 buffered positions' ends, and a spread) are
    checked against the oracle's row form."""
    wl = workload("llama31_8b")
    x = batch(wl)
    Q = np.stack([prefill_queries(wl, 0)])
    flag = _flags(wl, x, 0.04, seed=3)
    o, l = _run(wl, Q, x, flag)
    pos = np.array([0, 1, 127, 128, 129, 4095, 16384, 30000, wl.L - 64, wl.L - 1])
    G = wl.G
    for g in range(wl.Hkv):
        ro, rl = O.prefill_rows_unit(Q[0, g * G:(g + 1) * G][:, pos], pos, x["K"][0, g], x["V"][0, g],
                                     flag[0, g], wl.W)
        check_decode(o[0, g * G:(g + 1) * G][:, pos], l[0, g * G:(g + 1) * G][:, pos], ro, rl,
                     tag=f"kv head {g}")


def test_prefill_lse_feeds_the_selection():
    """The prefill's LSE rows of the last 64 positions, given to
    hq_select_vertical as its lse (the first pass skipped) with the prefill's
    tail queries as the buffered ones: scores against the oracle's column
    mass with that LSE (relative 2e-5), flags and indices exactly the
    top-n_vl of the GPU's own scores, and the set equal to the oracle's
    outside the 1e-5 tie band."""
    wl, x, Q = _inputs("tiny", L=1024)
    flag = _flags(wl, x)
    o, lse = _run(wl, Q, x, flag)
    L, W, G, nb = wl.L, wl.W, wl.G, 64
    qbuf = np.ascontiguousarray(Q[:, :, L - nb:])
    lse_rows = np.ascontiguousarray(lse[:, :, L - nb:]).astype(np.float32)
    dims = H.make_dims(wl.B, wl.Hq, wl.Hkv, W, wl.rho)
    n_nw = L - W
    n_vl = O.n_vertical(wl.rho, n_nw)
    score = torch.zeros((wl.B, wl.Hkv, L), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.B, wl.Hkv, n_vl), -1, dtype=torch.int32, device="cuda")
    fl = torch.zeros((wl.B, wl.Hkv, L), dtype=torch.uint8, device="cuda")
    H.hq_select_vertical(dims, dev(qbuf), dev(x["K"]), L, score, idx, fl,
                         H.workspace(dims, H.HQ_OP_SELECT, L), lse=dev(lse_rows))
    torch.cuda.synchronize()
    sg, ig, fg = score.cpu().numpy(), idx.cpu().numpy(), fl.cpu().numpy()
    for b in range(wl.B):
        for g in range(wl.Hkv):
            so = O.column_mass_given_lse_unit(x["K"][b, g], qbuf[b, g * G:(g + 1) * G],
                                              lse_rows[b, g * G:(g + 1) * G].astype(np.float64), L, W)
            err = np.abs(sg[b, g, :n_nw] - so) / np.maximum(so, 1e-30)
            assert err.max() <= 2e-5, f"b{b} g{g} score rel err {err.max():.2e}"
            mine = np.sort(np.lexsort((np.arange(n_nw), -sg[b, g, :n_nw].astype(np.float64)))[:n_vl])
            assert np.array_equal(np.nonzero(fg[b, g])[0], mine) and np.array_equal(ig[b, g], mine)
            theirs = O.top_rho(so, n_vl)
            cut = np.sort(so)[::-1][n_vl - 1]
            bad = [p for p in np.setxor1d(mine, theirs) if abs(so[p] - cut) > 1e-5 * cut]
            assert not bad, f"b{b} g{g}: {len(bad)} set differences outside the tie band"
