"""C-ABI checks that need no GPU: the library loads, exports every function
include/hq.h declares, and rejects bad calls on the host before launching."""
import ctypes
import os
import re

import pytest

import hybrid_precision_attention_amd as H
from hybrid_precision_attention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "hq.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"hq_select_vertical", "hq_quant_pack", "hq_append_merge", "hq_decode_attn",
            "hq_refresh_hybrid", "hq_append_merge_scored", "hq_append_merge_ragged",
            "hq_decode_attn_ragged", "hq_quant_int8", "hq_prefill_attn", "hq_decode_step", "hq_decode_step_ragged",
            "hq_workspace_bytes", "hq_status_string", "hq_abi_version", "hq_n_vertical", "hq_decode_attn_noalloc"} <= set(names)
    for n in names:
        assert hasattr(H.lib, n), n


def test_probe_library_exports_its_header():
    """libhq_probe.so (the benchmark's measurement helpers) exports every
    function include/hq_probe.h declares."""
    with open(os.path.join(ROOT, "include", "hq_probe.h")) as f:
        src = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(hq_probe_[a-z0-9_]+)\s*\(", src)))
    assert {"hq_probe_stream_read", "hq_probe_stream_read_nt", "hq_probe_mfma_rate"} <= set(names)
    probe = ctypes.CDLL(os.path.join(ROOT, "hybrid_precision_attention_amd", "libhq_probe.so"))
    for n in names:
        assert hasattr(probe, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert H.hq_status_string(s) != "unknown status"
    assert H.hq_status_string(7) == "unknown status"
    assert H.lib.hq_abi_version() == 10


def test_n_vertical_is_the_oracles_count():
    """The library's top-rho count (the one every entry point sizes its set
    with) equals the oracle's floor(rho * n + 1e-6) over a grid of rho and
    candidate counts, incl. the tiny workload's 44 of 896 and 0.29 * 100 = 29
    (binary rho); out-of-range rho and empty candidate sets give 0."""
    from oracle import hq_oracle as O
    assert H.n_vertical(0.05, 896) == 44
    assert H.n_vertical(0.29, 100) == 29
    for rho in (0.0, 0.01, 0.05, 0.1, 0.29, 0.3, 1 / 3, 0.5, 0.999999, 1.0):
        for n in (0, 1, 7, 100, 896, 1000, 32640, 65535, 1 << 24):
            assert H.n_vertical(rho, n) == O.n_vertical(rho, n), (rho, n)
    assert H.n_vertical(0.05, -3) == 0
    assert H.n_vertical(-0.1, 100) == 0 and H.n_vertical(1.5, 100) == 0
    assert H.n_vertical(float("nan"), 100) == 0


def _fake_cache(W=128, base=1 << 20):
    """Non-null, 16-byte aligned fake device pointers: calls that fail
    validation never dereference them."""
    c = B.hq_cache()
    for i, (n, _) in enumerate(B.hq_cache._fields_):
        setattr(c, n, base + 4096 * i)
    c.k4_pages = None
    if W == 0:
        c.kwin = None
        c.vwin = None
    return c


P = 1 << 24       # fake aligned pointer


def _dims(**kw):
    d = dict(B=1, Hq=32, Hkv=8, W=128, rho=0.05, cap_q=32640, cap_vl=1632, cap_stg=1)
    d.update(kw)
    return B.make_dims(**d)


def _pack(d, L=32768, cache=None, k=P, v=P, flag=P):
    c = cache or _fake_cache(d.W)
    return H.lib.hq_quant_pack(ctypes.byref(d), k, v, L, flag, ctypes.byref(c), None)


def test_dims_validation():
    assert _pack(_dims(Hq=30, Hkv=8)) == -1            # Hq % Hkv
    assert _pack(_dims(B=0)) == -1
    assert _pack(_dims(W=-1)) == -1
    assert _pack(_dims(rho=1.5)) == -1
    assert _pack(_dims(rho=float("nan"))) == -1
    assert _pack(_dims(d=64)) == -2                    # unsupported head_dim
    assert _pack(_dims(Hq=64, Hkv=2)) == -2            # G = 32 > 16
    assert _pack(_dims(B=8192, Hq=8, Hkv=8)) == -1     # 65536 units: more than a grid dimension holds
    assert H.lib.hq_quant_pack(None, P, P, 10, P, ctypes.byref(_fake_cache()), None) == -1


def test_pack_validation():
    d = _dims()
    assert _pack(d, L=-1) == -1
    assert _pack(d, k=None) == -1
    assert _pack(d, k=P + 4) == -3                      # misaligned
    assert _pack(_dims(cap_q=100)) == -4                # capacity
    c = _fake_cache()
    c.kq = None
    assert _pack(d, cache=c) == -1
    c = _fake_cache()
    c.kq_meta = (1 << 20) + 8
    assert _pack(d, cache=c) == -3
    c = _fake_cache()
    c.q_pos = (1 << 20) + 2                             # positions need 4 bytes
    assert _pack(d, cache=c) == -3
    assert _pack(_dims(W=128), cache=_fake_cache(W=0)) == -1   # W > 0 needs a ring


def test_paged_cache_validation():
    c = _fake_cache()
    c.k4_pages = (1 << 20) + 4096 * 40
    assert _pack(_dims(cap_q=32640 - 16), cache=c) == -1         # paged slots come in 32-slot blocks
    c.k4_pages = (1 << 20) + 4096 * 40 + 2
    assert _pack(_dims(cap_q=32640), cache=c) == -3              # the table needs 4-byte alignment


def test_merge_validation():
    d = _dims()
    c = _fake_cache()
    f = H.lib.hq_append_merge
    assert f(ctypes.byref(d), ctypes.byref(c), -1, P, P, None, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(c), 100, None, P, None, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(c), 100, P + 2, P, None, None) == -3
    assert f(ctypes.byref(d), ctypes.byref(c), 100, P, P, P + 1, None) == -3
    assert f(ctypes.byref(_dims(cap_stg=0)), ctypes.byref(c), 100, P, P, None, None) == -4
    assert f(ctypes.byref(_dims(cap_q=10)), ctypes.byref(c), 1000, P, P, None, None) == -4


def test_decode_validation():
    d = _dims()
    c = _fake_cache()
    need = H.hq_workspace_bytes(d, H.HQ_OP_DECODE, 32768)
    assert need > 0
    f = H.lib.hq_decode_attn
    assert f(ctypes.byref(d), ctypes.byref(c), -1, P, P, None, P, need, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(c), 10, None, P, None, P, need, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(c), 10, P, P + 8, None, P, need, None) == -3
    assert f(ctypes.byref(d), ctypes.byref(c), 10, P, P, None, None, need, None) == -5
    assert f(ctypes.byref(d), ctypes.byref(c), 10, P, P, None, P, need - 1, None) == -5
    assert f(ctypes.byref(d), ctypes.byref(c), 10, P, P, P + 4, P, need, None) == -3


def test_select_validation():
    d = _dims()
    need = H.hq_workspace_bytes(d, H.HQ_OP_SELECT, 32768)
    assert need > 0
    f = H.lib.hq_select_vertical
    args = lambda nb=64, L=32768, ws=P, wsb=need, idx=P: (
        ctypes.byref(d), P, nb, P, L, None, P, idx, P, ws, wsb, None)
    assert f(*args(nb=0)) == -1
    assert f(*args(nb=65)) == -1
    assert f(*args(nb=64, L=32)) == -1                  # nb > L
    assert f(*args(L=0, nb=1)) == -1
    assert f(*args(idx=None)) == -1                     # n_vl > 0 needs vl_idx
    assert f(*args(ws=None)) == -5
    assert f(*args(wsb=need - 1)) == -5


def test_refresh_validation():
    d = _dims()
    c = _fake_cache()
    f = H.lib.hq_refresh_hybrid
    args = lambda t=1000, nb=64, ld=1001, idx=P, cut=P, lse=P, q=P: (
        ctypes.byref(d), ctypes.byref(c), t, q, nb, lse, P, ld, idx, P, cut, None)
    assert f(*args(t=-1)) == -1
    assert f(*args(nb=0)) == -1
    assert f(*args(nb=65)) == -1
    assert f(*args(t=10, nb=12, ld=11)) == -1           # nb > t + 1
    assert f(*args(ld=1000)) == -1                       # score row shorter than t + 1
    assert f(*args(idx=None)) == -1                      # n_vl > 0 needs vl_idx
    assert f(*args(cut=None)) == -1
    assert f(*args(lse=None)) == -1
    assert f(*args(q=P + 8)) == -3
    assert f(*args(cut=P + 4)) == -3
    bad = _fake_cache()
    bad.q_pos = None
    assert f(ctypes.byref(d), ctypes.byref(bad), 1000, P, 64, P, P, 1001, P, P, P, None) == -1


def test_scored_merge_validation():
    d = _dims()
    c = _fake_cache()
    f = H.lib.hq_append_merge_scored
    args = lambda t=100, ld=100, score=P, cut=P, k=P: (
        ctypes.byref(d), ctypes.byref(c), t, k, P, score, ld, cut, None)
    assert f(*args(t=-1)) == -1
    assert f(*args(score=None)) == -1
    assert f(*args(cut=None)) == -1
    assert f(*args(ld=99)) == -1                         # the leaving position may be t - 1
    assert f(*args(k=P + 2)) == -3
    assert f(ctypes.byref(_dims(cap_stg=0)), ctypes.byref(c), 100, P, P, P, 100, P, None) == -4


def test_step_validation():
    d = _dims()
    c = _fake_cache()
    need = H.hq_workspace_bytes(d, H.HQ_OP_DECODE, 32768)
    f = H.lib.hq_decode_step
    args = lambda t=1000, k=P, q=P, ev=None, lse=None, ws=P, wsb=need, dd=d: (
        ctypes.byref(dd), ctypes.byref(c), t, k, P, ev, q, P, lse, ws, wsb, None)
    assert f(*args(t=-1)) == -1
    assert f(*args(k=None)) == -1
    assert f(*args(q=None)) == -1
    assert f(*args(k=P + 2)) == -3
    assert f(*args(ev=P + 1)) == -3
    assert f(*args(lse=P + 4)) == -3
    assert f(*args(ws=None)) == -5
    assert f(*args(wsb=need - 1)) == -5
    assert f(*args(t=32640 + 128, dd=_dims(cap_q=32640))) == -4       # the K4V4 region would overflow
    assert f(ctypes.byref(d), None, 10, P, P, None, P, P, None, P, need, None) == -1
    g = H.lib.hq_decode_step_ragged
    rargs = lambda ts=P, tmax=1000, k=P, wsb=need, dd=d: (
        ctypes.byref(dd), ctypes.byref(c), ts, tmax, k, P, None, P, P, None, P, wsb, None)
    assert g(*rargs(ts=None)) == -1
    assert g(*rargs(tmax=-1)) == -1
    assert g(*rargs(ts=P + 4)) == -3
    assert g(*rargs(k=P + 2)) == -3
    assert g(*rargs(wsb=need - 1)) == -5
    assert g(*rargs(tmax=32640 + 128, dd=_dims(cap_q=32640))) == -4


def test_prefill_validation():
    d = _dims()
    L = 4096
    need = H.hq_workspace_bytes(d, H.HQ_OP_PREFILL, L)
    assert need > 0
    f = H.lib.hq_prefill_attn
    args = lambda L=L, q=P, k=P, flag=None, out=P, lse=None, ws=P, wsb=need: (
        ctypes.byref(d), q, k, P, L, flag, out, lse, ws, wsb, None)
    assert f(*args(L=-1)) == -1
    assert f(*args(L=0, q=None)) == 0                   # nothing to do
    assert f(*args(q=None)) == -1
    assert f(*args(k=P + 2)) == -3
    assert f(*args(flag=P + 1)) == -3
    assert f(*args(lse=P + 4)) == -3
    assert f(*args(ws=None)) == -5
    assert f(*args(wsb=need - 1)) == -5
    assert f(ctypes.byref(_dims(d=64)), P, P, P, L, None, P, None, P, need, None) == -2
    assert H.hq_workspace_bytes(d, H.HQ_OP_PREFILL, 8192) > need
    assert f(*args(L=65535 * 32 + 1)) == -2             # more query blocks than a grid dimension holds
    g = H.lib.hq_quant_int8
    assert g(P, -1, P, P, None) == -1
    assert g(None, 4, P, P, None) == -1
    assert g(P, 4, P + 8, P, None) == -3
    assert g(None, 0, None, None, None) == 0            # no rows


def test_workspace_bytes():
    d = _dims()
    assert H.hq_workspace_bytes(d, 99, 100) == 0
    assert H.hq_workspace_bytes(d, H.HQ_OP_DECODE, -1) == 0
    assert H.hq_workspace_bytes(_dims(d=64), H.HQ_OP_DECODE, 100) == 0
    small = H.hq_workspace_bytes(d, H.HQ_OP_SELECT, 1024)
    big = H.hq_workspace_bytes(d, H.HQ_OP_SELECT, 32768)
    assert 0 < small <= big


def test_noalloc_decode_rejects_requests_beyond_its_scratch():
    """hq_decode_attn_noalloc checks on the host, before any HIP call, that
    the request fits its static scratch: at most 4096 units, and the records
    of the call's split plan within the area after the counters."""
    q, out = P, P + (1 << 22)
    for kw, L in ((dict(B=8190, Hkv=8, Hq=64), 4096),               # 65520 units
                  (dict(B=512, Hkv=8, Hq=128, cap_q=32768), 32768)):  # 4096 units, 16 heads each
        d = _dims(**kw)
        st = H.lib.hq_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(_fake_cache()), L, q, out, None, None)
        assert st == -7, (kw, st)
    # argument errors come first, as in hq_decode_attn
    d = _dims()
    assert H.lib.hq_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(_fake_cache()), -1, q, out, None, None) == -1
    assert H.lib.hq_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(_fake_cache()), 10, q + 8, out, None,
                                        None) == -3

