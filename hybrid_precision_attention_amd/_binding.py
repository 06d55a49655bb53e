"""ctypes binding of libhq.so: argument marshalling only.

Every operation runs in the library's HIP kernels; this module only turns
torch tensors (device memory) and the current torch stream into the plain
pointers and sizes of the C ABI, and raises ``HQError`` on a nonzero status.
There is no fallback: without the built library, importing fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhq.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                      "or python hybrid_precision_attention_amd/build.py")
lib = ctypes.CDLL(_LIB_PATH)

HQ_OK = 0
HQ_OP_SELECT = 1
HQ_OP_DECODE = 2
HQ_OP_PREFILL = 3
PAGE = 32           # K4V4 slots per block of a paged cache
D = 128


class hq_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("W", ctypes.c_int32), ("rho", ctypes.c_double),
                ("cap_q", ctypes.c_int32), ("cap_vl", ctypes.c_int32),
                ("cap_stg", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32)]


class hq_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "kq", "vq", "kq_meta", "vq_meta", "q_pos", "kvl", "vvl", "vl_pos",
        "kwin", "vwin", "kstg", "vstg", "n_q", "n_vl", "n_stg", "k4_pages")]


_p = ctypes.c_void_p
lib.hq_select_vertical.argtypes = [ctypes.POINTER(hq_dims), _p, ctypes.c_int32, _p, ctypes.c_int32,
                                   _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.hq_quant_pack.argtypes = [ctypes.POINTER(hq_dims), _p, _p, ctypes.c_int32, _p,
                              ctypes.POINTER(hq_cache), _p]
lib.hq_append_merge.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), ctypes.c_int32,
                                _p, _p, _p, _p]
lib.hq_decode_attn.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), ctypes.c_int32,
                               _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.hq_decode_attn_noalloc.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), ctypes.c_int32,
                                       _p, _p, _p, _p]
lib.hq_refresh_hybrid.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), ctypes.c_int32,
                                  _p, ctypes.c_int32, _p, _p, ctypes.c_int32, _p, _p, _p, _p]
lib.hq_append_merge_scored.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache),
                                       ctypes.c_int32, _p, _p, _p, ctypes.c_int32, _p, _p]
lib.hq_append_merge_ragged.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), _p,
                                       ctypes.c_int32, _p, _p, _p, _p]
lib.hq_decode_attn_ragged.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), _p,
                                      ctypes.c_int32, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.hq_decode_step.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), ctypes.c_int32, _p, _p,
                               _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.hq_decode_step_ragged.argtypes = [ctypes.POINTER(hq_dims), ctypes.POINTER(hq_cache), _p, ctypes.c_int32,
                                      _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.hq_quant_int8.argtypes = [_p, ctypes.c_int64, _p, _p, _p]
lib.hq_prefill_attn.argtypes = [ctypes.POINTER(hq_dims), _p, _p, _p, ctypes.c_int32, _p, _p, _p, _p,
                                ctypes.c_size_t, _p]
lib.hq_workspace_bytes.argtypes = [ctypes.POINTER(hq_dims), ctypes.c_int, ctypes.c_int32]
lib.hq_workspace_bytes.restype = ctypes.c_size_t
lib.hq_status_string.argtypes = [ctypes.c_int]
lib.hq_status_string.restype = ctypes.c_char_p
lib.hq_abi_version.restype = ctypes.c_int
lib.hq_n_vertical.argtypes = [ctypes.c_double, ctypes.c_int32]
lib.hq_n_vertical.restype = ctypes.c_int32
for _f in ("hq_select_vertical", "hq_quant_pack", "hq_append_merge", "hq_decode_attn",
           "hq_refresh_hybrid", "hq_append_merge_scored", "hq_append_merge_ragged",
           "hq_decode_attn_ragged", "hq_quant_int8", "hq_prefill_attn", "hq_decode_step",
           "hq_decode_step_ragged", "hq_decode_attn_noalloc"):
    getattr(lib, _f).restype = ctypes.c_int


class HQError(RuntimeError):
    def __init__(self, status: int, op: str):
        super().__init__(f"{op}: {hq_status_string(status)} (status {status})")
        self.status = status


def hq_status_string(status: int) -> str:
    return lib.hq_status_string(status).decode()


def n_vertical(rho: float, n_nw: int) -> int:
    """The vertical-line count the library uses for n_nw candidates
    (hq_n_vertical: floor(rho * n_nw + 1e-6))."""
    return int(lib.hq_n_vertical(float(rho), int(n_nw)))


def make_dims(B, Hq, Hkv, W, rho, cap_q=0, cap_vl=0, cap_stg=1, d=D, k_bits=4, v_bits=4) -> hq_dims:
    return hq_dims(B, Hq, Hkv, d, W, float(rho), cap_q, cap_vl, cap_stg, k_bits, v_bits)


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() or None


def _need(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """The C ABI takes plain pointers and cannot see sizes: raise before the
    call unless t (when given) holds the n elements the call reads or writes."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements; the call reads or writes {n}")


def _rows4(t: torch.Tensor, B: int, H: int, name: str) -> int:
    """Rows per head of a [B][H][rows][128] tensor (shape checked)."""
    if t.dim() != 4 or tuple(t.shape[:2]) != (B, H) or t.shape[3] != D:
        raise ValueError(f"{name} must be [{B}][{H}][rows][{D}], got {list(t.shape)}")
    return int(t.shape[2])


def _bits(b: int) -> int:
    return 4 if b == 0 else b


def _same_cache(dims: hq_dims, cache: "HybridCache") -> None:
    """The dims of a cache call must describe the buffers the cache holds."""
    c = cache.dims
    for f in ("B", "Hkv", "d", "W", "cap_q", "cap_vl", "cap_stg"):
        if getattr(dims, f) != getattr(c, f):
            raise ValueError(f"dims.{f} = {getattr(dims, f)} differs from the cache's {getattr(c, f)}")
    for f in ("k_bits", "v_bits"):
        if _bits(getattr(dims, f)) != _bits(getattr(c, f)):
            raise ValueError(f"dims.{f} = {getattr(dims, f)} differs from the cache's {getattr(c, f)}")


def _check_token(dims, cache, k_new, v_new, evict_is_vl) -> None:
    """A new token's K and V rows [B][Hkv][128] and its eviction flags [B][Hkv]."""
    _same_cache(dims, cache)
    U = dims.B * dims.Hkv
    _need(k_new, U * D, "k_new")
    _need(v_new, U * D, "v_new")
    _need(evict_is_vl, U, "evict_is_vl")


def _check_query(dims, cache, q, out, lse) -> None:
    """Decode queries and outputs [B][Hq][128], LSE [B][Hq]."""
    _same_cache(dims, cache)
    R = dims.B * dims.Hq
    _need(q, R * D, "q")
    _need(out, R * D, "out")
    _need(lse, R, "lse")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, op: str):
    if status != HQ_OK:
        raise HQError(status, op)


@dataclass
class HybridCache:
    """Device buffers of one layer's hybrid cache (layout of ``hq_cache``)."""
    dims: hq_dims
    t: dict

    @staticmethod
    def allocate(B, Hq, Hkv, W, rho, L_max, extra_vl=0, cap_stg=1, device="cuda", k_bits=4, v_bits=4):
        """Capacities for prefixes up to L_max tokens: every non-window
        position may be quantised; the vertical-line region holds the top-rho
        set of L_max plus ``extra_vl`` promotions.  Quantised keys and values
        use k_bits / v_bits codes (2, 4 or 8)."""
        n_nw = max(0, L_max - W)
        cap_q = max(1, n_nw)
        cap_vl = max(1, n_vertical(rho, n_nw) + extra_vl)
        dims = make_dims(B, Hq, Hkv, W, rho, cap_q, cap_vl, max(1, cap_stg), k_bits=k_bits, v_bits=v_bits)
        dev = torch.device(device)
        u8, f16, i32 = torch.uint8, torch.float16, torch.int32
        t = {
            "kq": torch.zeros((B, Hkv, cap_q, D * k_bits // 8), dtype=u8, device=dev),
            "vq": torch.zeros((B, Hkv, cap_q, D * v_bits // 8), dtype=u8, device=dev),
            "kq_meta": torch.zeros((B, Hkv, cap_q, D // 32, 2), dtype=f16, device=dev),
            "vq_meta": torch.zeros((B, Hkv, cap_q, D // 32, 2), dtype=f16, device=dev),
            "q_pos": torch.zeros((B, Hkv, cap_q), dtype=i32, device=dev),
            "kvl": torch.zeros((B, Hkv, cap_vl, D), dtype=f16, device=dev),
            "vvl": torch.zeros((B, Hkv, cap_vl, D), dtype=f16, device=dev),
            "vl_pos": torch.zeros((B, Hkv, cap_vl), dtype=i32, device=dev),
            "kwin": torch.zeros((B, Hkv, W, D), dtype=f16, device=dev) if W else None,
            "vwin": torch.zeros((B, Hkv, W, D), dtype=f16, device=dev) if W else None,
            "kstg": torch.zeros((B, Hkv, dims.cap_stg, D), dtype=f16, device=dev),
            "vstg": torch.zeros((B, Hkv, dims.cap_stg, D), dtype=f16, device=dev),
            "n_q": torch.zeros((B, Hkv), dtype=i32, device=dev),
            "n_vl": torch.zeros((B, Hkv), dtype=i32, device=dev),
            "n_stg": torch.zeros((B, Hkv), dtype=i32, device=dev),
            "k4_pages": None,
        }
        return HybridCache(dims, t)

    @staticmethod
    def allocate_paged(B, Hq, Hkv, W, rho, L_max, extra_vl=0, cap_stg=1, device="cuda", k_bits=4, v_bits=4,
                       seq_L_max=None, shuffle_seed=None):
        """Paged K4V4 slots: a pool of 32-slot blocks shared by all units and
        a page table per unit.  Sequence b's units get blocks only for the
        slots their own maximum length seq_L_max[b] (default L_max) can
        reach; the other table entries point at one spare block at the end
        of the pool, so that a stray write stays in bounds.  With
        shuffle_seed the blocks are handed out in a seeded random order (the
        layout is then far from contiguous; results are unchanged)."""
        n_nw = max(0, L_max - W)
        npb = max(1, -(-n_nw // PAGE))
        cap_q = npb * PAGE
        cap_vl = max(1, n_vertical(rho, n_nw) + extra_vl)
        dims = make_dims(B, Hq, Hkv, W, rho, cap_q, cap_vl, max(1, cap_stg), k_bits=k_bits, v_bits=v_bits)
        import numpy as np
        lens = list(seq_L_max) if seq_L_max is not None else [L_max] * B
        need = np.array([min(npb, -(-max(0, Lb - W) // PAGE)) for Lb in lens], dtype=np.int64)
        unit_need = np.repeat(need, Hkv)                 # blocks of each unit, in unit order
        total = int(unit_need.sum())
        order = np.arange(total, dtype=np.int32)
        if shuffle_seed is not None:
            np.random.default_rng(shuffle_seed).shuffle(order)
        spare = total                                  # the overflow block
        table = np.full((B * Hkv, npb), spare, dtype=np.int32)
        table[np.arange(npb)[None, :] < unit_need[:, None]] = order     # row by row: each unit's blocks
        pages = torch.from_numpy(table.reshape(B, Hkv, npb))
        P = total + 1
        dev = torch.device(device)
        u8, f16, i32 = torch.uint8, torch.float16, torch.int32
        t = {
            "kq": torch.zeros((P * PAGE, D * k_bits // 8), dtype=u8, device=dev),
            "vq": torch.zeros((P * PAGE, D * v_bits // 8), dtype=u8, device=dev),
            "kq_meta": torch.zeros((P * PAGE, D // 32, 2), dtype=f16, device=dev),
            "vq_meta": torch.zeros((P * PAGE, D // 32, 2), dtype=f16, device=dev),
            "q_pos": torch.zeros((P * PAGE,), dtype=i32, device=dev),
            "kvl": torch.zeros((B, Hkv, cap_vl, D), dtype=f16, device=dev),
            "vvl": torch.zeros((B, Hkv, cap_vl, D), dtype=f16, device=dev),
            "vl_pos": torch.zeros((B, Hkv, cap_vl), dtype=i32, device=dev),
            "kwin": torch.zeros((B, Hkv, W, D), dtype=f16, device=dev) if W else None,
            "vwin": torch.zeros((B, Hkv, W, D), dtype=f16, device=dev) if W else None,
            "kstg": torch.zeros((B, Hkv, dims.cap_stg, D), dtype=f16, device=dev),
            "vstg": torch.zeros((B, Hkv, dims.cap_stg, D), dtype=f16, device=dev),
            "n_q": torch.zeros((B, Hkv), dtype=i32, device=dev),
            "n_vl": torch.zeros((B, Hkv), dtype=i32, device=dev),
            "n_stg": torch.zeros((B, Hkv), dtype=i32, device=dev),
            "k4_pages": pages.to(dev),
        }
        return HybridCache(dims, t)

    @property
    def paged(self) -> bool:
        return self.t.get("k4_pages") is not None

    def k4_unit(self, b: int, g: int):
        """The K4V4 slots of unit (b, g) in slot order (through the page
        table when paged): kq, vq, kq_meta, vq_meta, q_pos."""
        names = ("kq", "vq", "kq_meta", "vq_meta", "q_pos")
        if not self.paged:
            return tuple(self.t[n][b, g] for n in names)
        pages = self.t["k4_pages"][b, g].long()
        rows = (pages[:, None] * PAGE + torch.arange(PAGE, device=pages.device)[None, :]).reshape(-1)
        return tuple(self.t[n][rows] for n in names)

    def struct(self) -> hq_cache:
        """The ``hq_cache`` of these buffers (built once: tensors never move)."""
        cs = getattr(self, "_struct", None)
        if cs is None:
            cs = hq_cache(*[(self.t[n].data_ptr() if self.t[n] is not None else None)
                            for n, _ in hq_cache._fields_])
            self._struct = cs
        return cs

    def view(self, b: int) -> "HybridCache":
        """Sequence b alone, as a B = 1 cache over the same memory (for
        building the caches of a ragged batch one sequence at a time)."""
        d = hq_dims.from_buffer_copy(self.dims)
        d.B = 1
        pools = {"kq", "vq", "kq_meta", "vq_meta", "q_pos"} if self.paged else set()
        return HybridCache(d, {k: (v if k in pools else v[b:b + 1]) if v is not None else None
                               for k, v in self.t.items()})

    def nbytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.t.values() if v is not None)

    def clone(self) -> "HybridCache":
        return HybridCache(hq_dims.from_buffer_copy(self.dims),
                           {k: (v.clone() if v is not None else None) for k, v in self.t.items()})


def hq_workspace_bytes(dims: hq_dims, op: int, L_max: int) -> int:
    return int(lib.hq_workspace_bytes(ctypes.byref(dims), op, L_max))


def workspace(dims: hq_dims, op: int, L_max: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the decode arrival counters must start at 0)."""
    n = hq_workspace_bytes(dims, op, L_max)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def hq_select_vertical(dims, qbuf, k, L, score, vl_idx, vl_flag, ws, lse=None, stream=None):
    """qbuf [B][Hq][nb][128] fp16, k [B][Hkv][L][128] fp16, lse [B][Hq][nb]
    fp32 or None; score and vl_flag [B][Hkv][L], vl_idx [B][Hkv][n_vl]."""
    nb = _rows4(qbuf, dims.B, dims.Hq, "qbuf")
    U = dims.B * dims.Hkv
    _need(k, U * L * D, "k")
    _need(lse, dims.B * dims.Hq * nb, "lse")
    _need(score, U * L, "score")
    _need(vl_idx, U * n_vertical(dims.rho, max(0, L - dims.W)), "vl_idx")
    _need(vl_flag, U * L, "vl_flag")
    st = lib.hq_select_vertical(ctypes.byref(dims), _ptr(qbuf, torch.float16, "qbuf"), nb,
                                _ptr(k, torch.float16, "k"), L, _ptr(lse, torch.float32, "lse"),
                                _ptr(score, torch.float32, "score"),
                                _ptr(vl_idx, torch.int32, "vl_idx"),
                                _ptr(vl_flag, torch.uint8, "vl_flag"), _ptr(ws, None, "ws"),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "hq_select_vertical")


def hq_quant_pack(dims, k, v, L, vl_flag, cache: HybridCache, stream=None):
    _same_cache(dims, cache)
    U = dims.B * dims.Hkv
    _need(k, U * L * D, "k")
    _need(v, U * L * D, "v")
    _need(vl_flag, U * L, "vl_flag")
    cs = cache.struct()
    st = lib.hq_quant_pack(ctypes.byref(dims), _ptr(k, torch.float16, "k"),
                           _ptr(v, torch.float16, "v"), L, _ptr(vl_flag, torch.uint8, "vl_flag"),
                           ctypes.byref(cs), _stream(stream))
    _check(st, "hq_quant_pack")


def hq_append_merge(dims, cache: HybridCache, t, k_new, v_new, evict_is_vl=None, stream=None):
    _check_token(dims, cache, k_new, v_new, evict_is_vl)
    cs = cache.struct()
    st = lib.hq_append_merge(ctypes.byref(dims), ctypes.byref(cs), t,
                             _ptr(k_new, torch.float16, "k_new"), _ptr(v_new, torch.float16, "v_new"),
                             _ptr(evict_is_vl, torch.uint8, "evict_is_vl"), _stream(stream))
    _check(st, "hq_append_merge")


def hq_decode_attn(dims, cache: HybridCache, L, q, out, ws, lse=None, stream=None):
    _check_query(dims, cache, q, out, lse)
    cs = cache.struct()
    st = lib.hq_decode_attn(ctypes.byref(dims), ctypes.byref(cs), L, _ptr(q, torch.float16, "q"),
                            _ptr(out, torch.float16, "out"), _ptr(lse, torch.float32, "lse"),
                            _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "hq_decode_attn")


def hq_decode_attn_noalloc(dims, cache: HybridCache, L, q, out, lse=None, stream=None):
    """hq_decode_attn without a workspace: the library's static per-GPU
    scratch holds the arrival counters and partial records (calls that
    overlap on one GPU race)."""
    _check_query(dims, cache, q, out, lse)
    cs = cache.struct()
    st = lib.hq_decode_attn_noalloc(ctypes.byref(dims), ctypes.byref(cs), L, _ptr(q, torch.float16, "q"),
                                    _ptr(out, torch.float16, "out"), _ptr(lse, torch.float32, "lse"),
                                    _stream(stream))
    _check(st, "hq_decode_attn_noalloc")


def hq_refresh_hybrid(dims, cache: HybridCache, t, qbuf, lse, score, vl_idx, vl_flag, cut,
                      stream=None):
    """score [B][Hkv][score_ld] (score_ld = its last dimension)."""
    _same_cache(dims, cache)
    nb = _rows4(qbuf, dims.B, dims.Hq, "qbuf")
    U, ld = dims.B * dims.Hkv, score.shape[-1]
    _need(lse, dims.B * dims.Hq * nb, "lse")
    _need(score, U * ld, "score")
    _need(vl_idx, U * n_vertical(dims.rho, max(0, t - dims.W)), "vl_idx")
    _need(vl_flag, U * ld, "vl_flag")
    _need(cut, U, "cut")
    cs = cache.struct()
    st = lib.hq_refresh_hybrid(ctypes.byref(dims), ctypes.byref(cs), t,
                               _ptr(qbuf, torch.float16, "qbuf"), qbuf.shape[2],
                               _ptr(lse, torch.float32, "lse"), _ptr(score, torch.float32, "score"),
                               score.shape[-1], _ptr(vl_idx, torch.int32, "vl_idx"),
                               _ptr(vl_flag, torch.uint8, "vl_flag"),
                               _ptr(cut, torch.float32, "cut"), _stream(stream))
    _check(st, "hq_refresh_hybrid")


def hq_append_merge_scored(dims, cache: HybridCache, t, k_new, v_new, score, cut, stream=None):
    _check_token(dims, cache, k_new, v_new, None)
    _need(score, dims.B * dims.Hkv * score.shape[-1], "score")
    _need(cut, dims.B * dims.Hkv, "cut")
    cs = cache.struct()
    st = lib.hq_append_merge_scored(ctypes.byref(dims), ctypes.byref(cs), t,
                                    _ptr(k_new, torch.float16, "k_new"),
                                    _ptr(v_new, torch.float16, "v_new"),
                                    _ptr(score, torch.float32, "score"), score.shape[-1],
                                    _ptr(cut, torch.float32, "cut"), _stream(stream))
    _check(st, "hq_append_merge_scored")


def hq_append_merge_ragged(dims, cache: HybridCache, t_seq, t_max, k_new, v_new, evict_is_vl=None,
                           stream=None):
    """t_seq: [B] int32 device tensor of per-sequence positions (<= t_max)."""
    _check_token(dims, cache, k_new, v_new, evict_is_vl)
    _need(t_seq, dims.B, "t_seq")
    cs = cache.struct()
    st = lib.hq_append_merge_ragged(ctypes.byref(dims), ctypes.byref(cs), _ptr(t_seq, torch.int32, "t_seq"),
                                    t_max, _ptr(k_new, torch.float16, "k_new"),
                                    _ptr(v_new, torch.float16, "v_new"),
                                    _ptr(evict_is_vl, torch.uint8, "evict_is_vl"), _stream(stream))
    _check(st, "hq_append_merge_ragged")


def hq_decode_attn_ragged(dims, cache: HybridCache, L_seq, L_max, q, out, ws, lse=None, stream=None):
    """L_seq: [B] int32 device tensor of per-sequence query positions (<= L_max)."""
    _check_query(dims, cache, q, out, lse)
    _need(L_seq, dims.B, "L_seq")
    cs = cache.struct()
    st = lib.hq_decode_attn_ragged(ctypes.byref(dims), ctypes.byref(cs), _ptr(L_seq, torch.int32, "L_seq"),
                                   L_max, _ptr(q, torch.float16, "q"), _ptr(out, torch.float16, "out"),
                                   _ptr(lse, torch.float32, "lse"), _ptr(ws, None, "ws"),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "hq_decode_attn_ragged")


def hq_decode_step(dims, cache: HybridCache, t, k_new, v_new, q, out, ws, lse=None, evict_is_vl=None,
                   stream=None):
    """hq_append_merge(t) + hq_decode_attn(t) in one launch (nothing may be staged)."""
    _check_token(dims, cache, k_new, v_new, evict_is_vl)
    _check_query(dims, cache, q, out, lse)
    cs = cache.struct()
    st = lib.hq_decode_step(ctypes.byref(dims), ctypes.byref(cs), t, _ptr(k_new, torch.float16, "k_new"),
                            _ptr(v_new, torch.float16, "v_new"), _ptr(evict_is_vl, torch.uint8, "evict_is_vl"),
                            _ptr(q, torch.float16, "q"), _ptr(out, torch.float16, "out"),
                            _ptr(lse, torch.float32, "lse"), _ptr(ws, None, "ws"),
                            ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "hq_decode_step")


def hq_decode_step_ragged(dims, cache: HybridCache, t_seq, t_max, k_new, v_new, q, out, ws, lse=None,
                          evict_is_vl=None, stream=None):
    """t_seq: [B] int32 device tensor of per-sequence positions (<= t_max)."""
    _check_token(dims, cache, k_new, v_new, evict_is_vl)
    _check_query(dims, cache, q, out, lse)
    _need(t_seq, dims.B, "t_seq")
    cs = cache.struct()
    st = lib.hq_decode_step_ragged(ctypes.byref(dims), ctypes.byref(cs), _ptr(t_seq, torch.int32, "t_seq"), t_max,
                                   _ptr(k_new, torch.float16, "k_new"), _ptr(v_new, torch.float16, "v_new"),
                                   _ptr(evict_is_vl, torch.uint8, "evict_is_vl"), _ptr(q, torch.float16, "q"),
                                   _ptr(out, torch.float16, "out"), _ptr(lse, torch.float32, "lse"),
                                   _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "hq_decode_step_ragged")


def bind_step(dims, cache: HybridCache, q, out, ws, lse=None, stream=None):
    """Returns f(t, k_ptr, v_ptr, q_ptr=None): hq_decode_step on fixed buffers.
    The bound tensors are checked here; the raw addresses passed per call are
    not (each must hold a [B][Hkv][128] or [B][Hq][128] fp16 row set)."""
    _check_query(dims, cache, q, out, lse)
    cs = cache.struct()
    d_ref, c_ref = ctypes.byref(dims), ctypes.byref(cs)
    qp = _ptr(q, torch.float16, "q")
    op, lp = _ptr(out, torch.float16, "out"), _ptr(lse, torch.float32, "lse")
    wp, wb, sp = _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)
    fn = lib.hq_decode_step

    def call(t, k_ptr, v_ptr, q_ptr=None):
        st = fn(d_ref, c_ref, t, k_ptr, v_ptr, None, q_ptr or qp, op, lp, wp, wb, sp)
        if st:
            raise HQError(st, "hq_decode_step")
    call.keep = (dims, cs, q, out, ws, lse)
    return call


def hq_quant_int8(x, codes, scales, stream=None):
    """x [..][128] fp16 rows -> codes [..][128] int8, scales [..] fp32."""
    rows = x.numel() // 128
    if x.shape[-1] != 128 or codes.numel() != rows * 128 or scales.numel() != rows:
        raise ValueError("hq_quant_int8: x [..][128], codes of x's shape, scales [rows]")
    st = lib.hq_quant_int8(_ptr(x, torch.float16, "x"), rows, _ptr(codes, torch.int8, "codes"),
                           _ptr(scales, torch.float32, "scales"), _stream(stream))
    _check(st, "hq_quant_int8")


def hq_prefill_attn(dims, q, k, v, L, vl_flag, out, ws, lse=None, stream=None):
    """q [B][Hq][L][128], k, v [B][Hkv][L][128] fp16; vl_flag [B][Hkv][L] uint8
    or None; out like q; lse [B][Hq][L] fp32 or None; ws from
    workspace(dims, HQ_OP_PREFILL, L)."""
    U, R = dims.B * dims.Hkv, dims.B * dims.Hq
    _need(q, R * L * D, "q")
    _need(out, R * L * D, "out")
    _need(lse, R * L, "lse")
    _need(k, U * L * D, "k")
    _need(v, U * L * D, "v")
    _need(vl_flag, U * L, "vl_flag")
    st = lib.hq_prefill_attn(ctypes.byref(dims), _ptr(q, torch.float16, "q"), _ptr(k, torch.float16, "k"),
                             _ptr(v, torch.float16, "v"), L, _ptr(vl_flag, torch.uint8, "vl_flag"),
                             _ptr(out, torch.float16, "out"), _ptr(lse, torch.float32, "lse"),
                             _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "hq_prefill_attn")


# --------------------------------------------------------------------------
# Pre-bound calls: the pointer arguments are marshalled once, so a decode
# loop pays one ctypes call per launch and nothing else.
# --------------------------------------------------------------------------
def bind_decode(dims, cache: HybridCache, q, out, ws, lse=None, stream=None):
    """Returns f(L, q_ptr=None): hq_decode_attn on fixed buffers; q_ptr
    optionally points at another query tensor of the same shape (not
    checked)."""
    _check_query(dims, cache, q, out, lse)
    cs = cache.struct()
    d_ref, c_ref = ctypes.byref(dims), ctypes.byref(cs)
    qp = _ptr(q, torch.float16, "q")
    op, lp = _ptr(out, torch.float16, "out"), _ptr(lse, torch.float32, "lse")
    wp, wb, sp = _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)
    fn = lib.hq_decode_attn

    def call(L, q_ptr=None):
        st = fn(d_ref, c_ref, L, q_ptr or qp, op, lp, wp, wb, sp)
        if st:
            raise HQError(st, "hq_decode_attn")
    call.keep = (dims, cs, q, out, ws, lse)
    return call


def bind_merge(dims, cache: HybridCache, evict_is_vl=None, stream=None):
    """Returns f(t, k_ptr, v_ptr): hq_append_merge of the token at t whose
    [B][Hkv][d] fp16 rows start at the given device addresses (not checked)."""
    _check_token(dims, cache, None, None, evict_is_vl)
    cs = cache.struct()
    d_ref, c_ref = ctypes.byref(dims), ctypes.byref(cs)
    ep, sp = _ptr(evict_is_vl, torch.uint8, "evict_is_vl"), _stream(stream)
    fn = lib.hq_append_merge

    def call(t, k_ptr, v_ptr):
        st = fn(d_ref, c_ref, t, k_ptr, v_ptr, ep, sp)
        if st:
            raise HQError(st, "hq_append_merge")
    call.keep = (dims, cs, evict_is_vl)
    return call
