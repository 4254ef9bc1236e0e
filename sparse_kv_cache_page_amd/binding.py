"""Thin Python binding of libentmaxkv.so (the C ABI in include/entmaxkv.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, turned into raw pointers, and handed to the C entry point together
with torch's current HIP stream.  Every step of the computation runs in the
library's HIP kernels; there is no other execution path.  If the library is
not built, or there is no GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libentmaxkv.so")

EKV_OK = 0
EKV_BF16, EKV_F32 = 0, 1
EKV_SELECT_TOPK, EKV_SELECT_GAUSS, EKV_SELECT_GAUSS_EST, EKV_SELECT_GAUSS_MASS = 0, 1, 2, 3

EXPORTED = (
    "ekv_build_page_meta",
    "ekv_score_pages",
    "ekv_select_pages",
    "ekv_entmax_decode",
    "ekv_decode_workspace_bytes",
    "ekv_entmax_decode_fused",
    "ekv_decode_fused_workspace_bytes",
    "ekv_score_select_pages",
    "ekv_append_token",
    "ekv_validate_cache",
    "ekv_softmax_decode",
    "ekv_softmax_workspace_bytes",
    "ekv_score_select_workspace_bytes",
    "ekv_decode_step",
    "ekv_step_workspace_bytes",
    "ekv_decode_step_noalloc",
    "ekv_topk_decode",
    "ekv_topk_decode_workspace_bytes",
    "ekv_score_box_pages",
    "ekv_score_hint_bytes",
    "ekv_gauss_expected_max",
    "ekv_status_string",
)


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("compact_moments", ctypes.c_int32),
    ]


class EkvError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m sparse_kv_cache_page_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(CacheDesc)
    lib.ekv_build_page_meta.argtypes = [dp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.ekv_score_pages.argtypes = [dp, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ekv_select_pages.argtypes = [dp, vp, i32, i32, f32, f32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ekv_entmax_decode.argtypes = [dp, vp, f32, f32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                      vp, vp, vp, sz, vp]
    lib.ekv_decode_step.argtypes = [dp, vp, f32, f32, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp,
                                    vp, vp, vp, vp, sz, vp]
    lib.ekv_topk_decode.argtypes = [dp, vp, f32, f32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, sz, vp]
    lib.ekv_score_box_pages.argtypes = [dp, vp, f32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.ekv_score_hint_bytes.argtypes = [dp]
    lib.ekv_score_hint_bytes.restype = sz
    lib.ekv_topk_decode_workspace_bytes.argtypes = [dp, i32]
    lib.ekv_topk_decode_workspace_bytes.restype = sz
    lib.ekv_decode_step_noalloc.argtypes = [dp, vp, f32, f32, vp, vp, vp, vp, i32, i32, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp]
    lib.ekv_score_select_pages.argtypes = [dp, vp, f32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp,
                                           vp, vp, sz, vp]
    lib.ekv_score_select_workspace_bytes.argtypes = [dp]
    lib.ekv_append_token.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ekv_validate_cache.argtypes = [dp, vp, vp, vp, vp]
    lib.ekv_score_select_workspace_bytes.restype = sz
    lib.ekv_step_workspace_bytes.argtypes = [dp, i32]
    lib.ekv_step_workspace_bytes.restype = sz
    lib.ekv_entmax_decode_fused.argtypes = [dp, vp, f32, f32, vp, vp, vp, vp, vp, vp, i32, vp,
                                            vp, vp, vp, vp, vp, sz, vp]
    lib.ekv_decode_fused_workspace_bytes.argtypes = [dp, i32]
    lib.ekv_decode_fused_workspace_bytes.restype = sz
    lib.ekv_decode_workspace_bytes.argtypes = [dp, i32]
    lib.ekv_decode_workspace_bytes.restype = sz
    lib.ekv_softmax_decode.argtypes = [dp, vp, f32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz,
                                       vp]
    lib.ekv_softmax_workspace_bytes.argtypes = [dp, i32]
    lib.ekv_softmax_workspace_bytes.restype = sz
    lib.ekv_gauss_expected_max.argtypes = [i32]
    lib.ekv_gauss_expected_max.restype = ctypes.c_double
    lib.ekv_status_string.argtypes = [ctypes.c_int]
    lib.ekv_status_string.restype = ctypes.c_char_p
    for name in ("ekv_build_page_meta", "ekv_score_pages", "ekv_select_pages",
                 "ekv_entmax_decode", "ekv_decode_step", "ekv_decode_step_noalloc",
                 "ekv_topk_decode", "ekv_score_box_pages",
                 "ekv_score_select_pages",
                 "ekv_entmax_decode_fused", "ekv_append_token", "ekv_validate_cache",
                 "ekv_softmax_decode"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def gauss_expected_max(n: int) -> float:
    """ekv_gauss_expected_max: the library's e_n = E[max of n iid N(0,1)] (host-only)."""
    return float(load_library().ekv_gauss_expected_max(int(n)))


def status_string(status: int) -> str:
    return load_library().ekv_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != EKV_OK:
        raise EkvError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@dataclass(frozen=True)
class CacheShape:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_pages_per_seq: int
    num_phys_pages: int
    kv_dtype: torch.dtype = torch.bfloat16
    moments_dtype: torch.dtype = torch.float32   # page mean/var: float32 or bfloat16

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def desc(self) -> CacheDesc:
        if self.kv_dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("K/V must be bfloat16 or float32")
        if self.moments_dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("page moments must be float32 or bfloat16")
        return CacheDesc(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                         self.page_size, self.max_pages_per_seq, self.num_phys_pages,
                         EKV_BF16 if self.kv_dtype == torch.bfloat16 else EKV_F32,
                         1 if self.moments_dtype == torch.bfloat16 else 0)


def _need(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _kv_shape(s: CacheShape):
    return (s.num_phys_pages, s.num_kv_heads, s.page_size, s.head_dim)


def build_page_meta(s: CacheShape, K, block_table, seq_lens, kmin, kmax, mean=None, var=None,
                    first_page=None, span: int = 0):
    """ekv_build_page_meta: per-page bounding box and key moments."""
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq))
    _need(seq_lens, "seq_lens", torch.int32, (s.batch,))
    mshape = (s.num_phys_pages, s.num_kv_heads, s.head_dim)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    if mean is not None or var is not None:
        _need(mean, "mean", s.moments_dtype, mshape)
        _need(var, "var", s.moments_dtype, mshape)
    if first_page is not None:
        _need(first_page, "first_page", torch.int32, (s.batch,))
    d = s.desc()
    _check("ekv_build_page_meta", load_library().ekv_build_page_meta(
        ctypes.byref(d), _ptr(K), _ptr(block_table), _ptr(seq_lens), _ptr(first_page),
        int(span), _ptr(kmin), _ptr(kmax), _ptr(mean), _ptr(var), _stream()))


def validate_cache(s: CacheShape, block_table, seq_lens):
    """ekv_validate_cache: (#rows with an invalid length, #invalid block-table entries),
    counted on the device; synchronises to read the two counts."""
    _need(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq))
    _need(seq_lens, "seq_lens", torch.int32, (s.batch,))
    bad = torch.empty(2, dtype=torch.int32, device=seq_lens.device)
    d = s.desc()
    _check("ekv_validate_cache", load_library().ekv_validate_cache(
        ctypes.byref(d), _ptr(block_table), _ptr(seq_lens), _ptr(bad), _stream()))
    b = bad.cpu()
    return int(b[0]), int(b[1])


def append_token(s: CacheShape, k_new, v_new, block_table, seq_lens, K, V, kmin, kmax,
                 mean=None, var=None):
    """ekv_append_token: write each row's token at position seq_lens[b] - 1 into the
    paged cache and bring its page's metadata up to date (one launch)."""
    kv_new = (s.batch, s.num_kv_heads, s.head_dim)
    _need(k_new, "k_new", s.kv_dtype, kv_new)
    _need(v_new, "v_new", s.kv_dtype, kv_new)
    _need(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq))
    _need(seq_lens, "seq_lens", torch.int32, (s.batch,))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(V, "V", s.kv_dtype, _kv_shape(s))
    mshape = (s.num_phys_pages, s.num_kv_heads, s.head_dim)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    if mean is not None or var is not None:
        _need(mean, "mean", s.moments_dtype, mshape)
        _need(var, "var", s.moments_dtype, mshape)
    d = s.desc()
    _check("ekv_append_token", load_library().ekv_append_token(
        ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(seq_lens), _ptr(K),
        _ptr(V), _ptr(kmin), _ptr(kmax), _ptr(mean), _ptr(var), _stream()))


def score_pages(s: CacheShape, q, scale: float, kmin, kmax, block_table, seq_lens, ubg,
                ub=None, mean=None, var=None, gm=None, gv=None):
    """ekv_score_pages: box upper bounds (and Gaussian moments when gm/gv given)."""
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    mshape = (s.num_phys_pages, Hkv, d)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    if ub is not None:
        _need(ub, "ub", torch.float32, (B, Hkv, mp, Hq // Hkv))
    if gm is not None or gv is not None:
        _need(gm, "gm", torch.float64, (B, Hq, mp))
        _need(gv, "gv", torch.float64, (B, Hq, mp))
        _need(mean, "mean", s.moments_dtype, mshape)
        _need(var, "var", s.moments_dtype, mshape)
    d_ = s.desc()
    _check("ekv_score_pages", load_library().ekv_score_pages(
        ctypes.byref(d_), _ptr(q), float(scale), _ptr(kmin), _ptr(kmax), _ptr(mean), _ptr(var),
        _ptr(block_table), _ptr(seq_lens), _ptr(ub), _ptr(ubg), _ptr(gm), _ptr(gv), _stream()))


def select_pages(s: CacheShape, seq_lens, policy: int, top_k: int, alpha: float, delta: float,
                 ubg, sel, n_sel, ub=None, gm=None, gv=None, tau_hat=None):
    """ekv_select_pages: top-k (policy 0) or Gaussian-aware selection with the box
    bound (policy 1) or the expected maximum (policy 2) as a page's estimated maximum, or
    the page's expected entmax mass against delta (policy 3)."""
    B, Hq, Hkv, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.max_pages_per_seq
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    _need(sel, "sel", torch.int32, (B, Hkv, mp))
    _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    if policy == EKV_SELECT_GAUSS:
        _need(ub, "ub", torch.float32, (B, Hkv, mp, Hq // Hkv))
    if policy in (EKV_SELECT_GAUSS, EKV_SELECT_GAUSS_EST, EKV_SELECT_GAUSS_MASS):
        _need(gm, "gm", torch.float64, (B, Hq, mp))
        _need(gv, "gv", torch.float64, (B, Hq, mp))
        _need(tau_hat, "tau_hat", torch.float64, (B, Hq))
    d = s.desc()
    _check("ekv_select_pages", load_library().ekv_select_pages(
        ctypes.byref(d), _ptr(seq_lens), int(policy), int(top_k), float(alpha), float(delta),
        _ptr(ub), _ptr(ubg), _ptr(gm), _ptr(gv), _ptr(sel), _ptr(n_sel), _ptr(tau_hat),
        _stream()))


def decode_workspace_bytes(s: CacheShape, max_sel: int = 0) -> int:
    d = s.desc()
    return int(load_library().ekv_decode_workspace_bytes(ctypes.byref(d), int(max_sel)))


def decode_fused_workspace_bytes(s: CacheShape, max_sel: int = 0) -> int:
    d = s.desc()
    return int(load_library().ekv_decode_fused_workspace_bytes(ctypes.byref(d), int(max_sel)))


def entmax_decode(s: CacheShape, q, scale: float, alpha: float, K, V, block_table, seq_lens,
                  out, ws, sel=None, n_sel=None, max_sel: int = 0, tau=None, n_support=None,
                  fused: bool = False, ub=None, zlb=None):
    """ekv_entmax_decode (or, with fused=True, ekv_entmax_decode_fused, whose
    workspace must be zero-filled before first use): alpha-entmax attention
    over the selected pages (all if sel is None).  With ub (per-head page
    bounds [B, Hkv, maxP, G]) and zlb ([B, Hq], written), selected pages that
    cannot hold any head's support are not read."""
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(V, "V", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(out, "out", torch.float32, (B, Hq, d))
    if sel is not None or n_sel is not None:
        _need(sel, "sel", torch.int32, (B, Hkv, mp))
        _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    if tau is not None:
        _need(tau, "tau", torch.float32, (B, Hq))
    if n_support is not None:
        _need(n_support, "n_support", torch.int32, (B, Hq))
    if ub is not None or zlb is not None:
        _need(ub, "ub", torch.float32, (B, Hkv, mp, Hq // Hkv))
        _need(zlb, "zlb", torch.float32, (B, Hq))
    if not (isinstance(ws, torch.Tensor) and ws.is_cuda and ws.dtype == torch.uint8
            and ws.is_contiguous()):
        raise TypeError("ws must be a contiguous uint8 GPU tensor")
    d_ = s.desc()
    name = "ekv_entmax_decode_fused" if fused else "ekv_entmax_decode"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(d_), _ptr(q), float(scale), float(alpha), _ptr(K), _ptr(V),
        _ptr(block_table), _ptr(seq_lens), _ptr(sel), _ptr(n_sel), int(max_sel), _ptr(ub),
        _ptr(zlb), _ptr(out), _ptr(tau), _ptr(n_support), _ptr(ws),
        ctypes.c_size_t(ws.numel()), _stream()))


def softmax_workspace_bytes(s: CacheShape, max_sel: int = 0) -> int:
    d = s.desc()
    return int(load_library().ekv_softmax_workspace_bytes(ctypes.byref(d), int(max_sel)))


def softmax_decode(s: CacheShape, q, scale: float, K, V, block_table, seq_lens, out, ws,
                   sel=None, n_sel=None, max_sel: int = 0, lse=None):
    """ekv_softmax_decode: softmax attention over the selected pages (every page
    of each row if sel is None); lse [B, Hq] receives ln sum exp(scores)."""
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(V, "V", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(out, "out", torch.float32, (B, Hq, d))
    if sel is not None or n_sel is not None:
        _need(sel, "sel", torch.int32, (B, Hkv, mp))
        _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq))
    if not (isinstance(ws, torch.Tensor) and ws.is_cuda and ws.dtype == torch.uint8
            and ws.is_contiguous()):
        raise TypeError("ws must be a contiguous uint8 GPU tensor")
    d_ = s.desc()
    _check("ekv_softmax_decode", load_library().ekv_softmax_decode(
        ctypes.byref(d_), _ptr(q), float(scale), _ptr(K), _ptr(V), _ptr(block_table),
        _ptr(seq_lens), _ptr(sel), _ptr(n_sel), int(max_sel), _ptr(out), _ptr(lse), _ptr(ws),
        ctypes.c_size_t(ws.numel()), _stream()))


def step_workspace_bytes(s: CacheShape, top_k: int) -> int:
    d = s.desc()
    return int(load_library().ekv_step_workspace_bytes(ctypes.byref(d), int(top_k)))


def decode_step(s: CacheShape, q, scale: float, alpha: float, K, V, block_table, seq_lens,
                top_k: int, kmin, kmax, ubg, sel, n_sel, out, ws, refresh_last_page: bool = False,
                tau=None, n_support=None):
    """ekv_decode_step: [last-page refresh] + score + top-k + entmax decode, two launches.

    `ws` must be a uint8 GPU tensor of step_workspace_bytes() bytes, zero-filled
    before its first use (torch.zeros); every call leaves it reusable.
    """
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(V, "V", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    mshape = (s.num_phys_pages, Hkv, d)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    _need(sel, "sel", torch.int32, (B, Hkv, mp))
    _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    _need(out, "out", torch.float32, (B, Hq, d))
    if tau is not None:
        _need(tau, "tau", torch.float32, (B, Hq))
    if n_support is not None:
        _need(n_support, "n_support", torch.int32, (B, Hq))
    if not (isinstance(ws, torch.Tensor) and ws.is_cuda and ws.dtype == torch.uint8
            and ws.is_contiguous()):
        raise TypeError("ws must be a contiguous uint8 GPU tensor")
    d_ = s.desc()
    _check("ekv_decode_step", load_library().ekv_decode_step(
        ctypes.byref(d_), _ptr(q), float(scale), float(alpha), _ptr(K), _ptr(V),
        _ptr(block_table), _ptr(seq_lens), int(bool(refresh_last_page)), int(top_k), _ptr(kmin),
        _ptr(kmax), _ptr(ubg), _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(tau), _ptr(n_support),
        _ptr(ws), ctypes.c_size_t(ws.numel()), _stream()))


def topk_decode_workspace_bytes(s: CacheShape, top_k: int) -> int:
    d = s.desc()
    return int(load_library().ekv_topk_decode_workspace_bytes(ctypes.byref(d), int(top_k)))


def score_hint_bytes(s: CacheShape) -> int:
    d = s.desc()
    return int(load_library().ekv_score_hint_bytes(ctypes.byref(d)))


def score_box_pages(s: CacheShape, q, scale: float, block_table, seq_lens, kmin, kmax, ubg,
                    ub=None, hint=None, K=None, refresh_last_page: bool = False):
    """ekv_score_box_pages: box bounds (ub, ubg) and, into `hint` (uint8 GPU tensor of
    score_hint_bytes()), each page slice's best page per head for ekv_topk_decode."""
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    mshape = (s.num_phys_pages, Hkv, d)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    if ub is not None:
        _need(ub, "ub", torch.float32, (B, Hkv, mp, Hq // Hkv))
    if hint is not None and not (isinstance(hint, torch.Tensor) and hint.is_cuda and
                                 hint.dtype == torch.uint8 and hint.is_contiguous() and
                                 hint.numel() >= score_hint_bytes(s)):
        raise TypeError("hint must be a contiguous uint8 GPU tensor of score_hint_bytes() bytes")
    if refresh_last_page:
        _need(K, "K", s.kv_dtype, _kv_shape(s))
    d_ = s.desc()
    _check("ekv_score_box_pages", load_library().ekv_score_box_pages(
        ctypes.byref(d_), _ptr(q), float(scale), _ptr(K), _ptr(block_table), _ptr(seq_lens),
        int(bool(refresh_last_page)), _ptr(kmin), _ptr(kmax), _ptr(ub), _ptr(ubg), _ptr(hint),
        _stream()))


def topk_decode(s: CacheShape, q, scale: float, alpha: float, K, V, block_table, seq_lens,
                top_k: int, ubg, sel, n_sel, out, ws, ub=None, tau=None, n_support=None,
                hint=None):
    """ekv_topk_decode: top-k selection from ubg and the sparse entmax decode over it
    (with page pruning when the per-head bounds ub [B, Hkv, maxP, G] are given, and
    the scorer's hints when `hint` is)."""
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(V, "V", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    _need(sel, "sel", torch.int32, (B, Hkv, mp))
    _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    _need(out, "out", torch.float32, (B, Hq, d))
    if ub is not None:
        _need(ub, "ub", torch.float32, (B, Hkv, mp, Hq // Hkv))
    if tau is not None:
        _need(tau, "tau", torch.float32, (B, Hq))
    if n_support is not None:
        _need(n_support, "n_support", torch.int32, (B, Hq))
    if not (isinstance(ws, torch.Tensor) and ws.is_cuda and ws.dtype == torch.uint8
            and ws.is_contiguous()):
        raise TypeError("ws must be a contiguous uint8 GPU tensor")
    d_ = s.desc()
    _check("ekv_topk_decode", load_library().ekv_topk_decode(
        ctypes.byref(d_), _ptr(q), float(scale), float(alpha), _ptr(K), _ptr(V),
        _ptr(block_table), _ptr(seq_lens), int(top_k), _ptr(ub), _ptr(ubg), _ptr(hint),
        _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(tau), _ptr(n_support), _ptr(ws),
        ctypes.c_size_t(ws.numel()), _stream()))


NOALLOC_SCRATCH_BYTES = 64 << 20   # EKV_NOALLOC_SCRATCH_BYTES
NOALLOC_COUNTER_BYTES = 64 << 10   # EKV_NOALLOC_COUNTER_BYTES


def decode_step_noalloc(s: CacheShape, q, scale: float, alpha: float, K, V, block_table,
                        seq_lens, top_k: int, kmin, kmax, ubg, sel, n_sel, out,
                        refresh_last_page: bool = False, tau=None, n_support=None):
    """ekv_decode_step_noalloc: decode_step with the library's own per-device
    scratch instead of a workspace (no device allocation anywhere); shapes whose
    scratch exceeds NOALLOC_SCRATCH_BYTES are refused.  Calls on one GPU must
    not overlap in time."""
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(V, "V", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    mshape = (s.num_phys_pages, Hkv, d)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    _need(sel, "sel", torch.int32, (B, Hkv, mp))
    _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    _need(out, "out", torch.float32, (B, Hq, d))
    if tau is not None:
        _need(tau, "tau", torch.float32, (B, Hq))
    if n_support is not None:
        _need(n_support, "n_support", torch.int32, (B, Hq))
    d_ = s.desc()
    _check("ekv_decode_step_noalloc", load_library().ekv_decode_step_noalloc(
        ctypes.byref(d_), _ptr(q), float(scale), float(alpha), _ptr(K), _ptr(V),
        _ptr(block_table), _ptr(seq_lens), int(bool(refresh_last_page)), int(top_k), _ptr(kmin),
        _ptr(kmax), _ptr(ubg), _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(tau), _ptr(n_support),
        _stream()))


def score_select_workspace_bytes(s: CacheShape) -> int:
    d = s.desc()
    return int(load_library().ekv_score_select_workspace_bytes(ctypes.byref(d)))


def score_select_pages(s: CacheShape, q, scale: float, K, block_table, seq_lens, top_k: int,
                       kmin, kmax, ubg, sel, n_sel, ws, refresh_last_page: bool = False, ub=None):
    """ekv_score_select_pages: [last-page refresh] + scores + top-k in one launch
    (per-head bounds also written to ub [B, Hkv, maxP, G] when given).

    `ws`: uint8 GPU tensor of score_select_workspace_bytes() bytes, zero-filled
    before first use (torch.zeros); every call leaves it reusable.
    """
    B, Hq, Hkv, d, mp = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.max_pages_per_seq
    _need(q, "q", torch.float32, (B, Hq, d))
    _need(K, "K", s.kv_dtype, _kv_shape(s))
    _need(block_table, "block_table", torch.int32, (B, mp))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    mshape = (s.num_phys_pages, Hkv, d)
    _need(kmin, "kmin", s.kv_dtype, mshape)
    _need(kmax, "kmax", s.kv_dtype, mshape)
    _need(ubg, "ubg", torch.float32, (B, Hkv, mp))
    _need(sel, "sel", torch.int32, (B, Hkv, mp))
    _need(n_sel, "n_sel", torch.int32, (B, Hkv))
    if not (isinstance(ws, torch.Tensor) and ws.is_cuda and ws.dtype == torch.uint8
            and ws.is_contiguous()):
        raise TypeError("ws must be a contiguous uint8 GPU tensor")
    d_ = s.desc()
    if ub is not None:
        _need(ub, "ub", torch.float32, (B, Hkv, mp, Hq // Hkv))
    _check("ekv_score_select_pages", load_library().ekv_score_select_pages(
        ctypes.byref(d_), _ptr(q), float(scale), _ptr(K), _ptr(block_table), _ptr(seq_lens),
        int(bool(refresh_last_page)), int(top_k), _ptr(kmin), _ptr(kmax), _ptr(ub), _ptr(ubg),
        _ptr(sel), _ptr(n_sel), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream()))
