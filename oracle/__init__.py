"""ctypes front end of the fp64 CPU oracle (``oracle/sfi_oracle.c``).

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg import this package.  It builds ``liboracle.so`` with gcc (no fast-math)
and wraps the reference functions.  Inputs are torch tensors (any device: they are
copied to host memory) holding exactly the bytes the GPU reads; results are float64
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sfi_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt oracle library to load instead (the sanitizer test points this at a build with
# AddressSanitizer and UndefinedBehaviorSanitizer); never built here.
_LIB_OVERRIDE = os.environ.get("SFI_ORACLE_LIB")
_lib = None

SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(force: bool = True) -> str:
    """Compile the oracle (plain gcc, -O2, OpenMP, IEEE double semantics)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile the oracle with AddressSanitizer and UndefinedBehaviorSanitizer into `path`
    (CPU only; the library must be loaded with the sanitizer runtimes preloaded)."""
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-fno-fast-math"] + SANITIZE_FLAGS + ["-o", path, _SRC, "-lm"])
    return path


class _Refine(ctypes.Structure):
    _fields_ = [("lambda_", ctypes.c_double), ("alpha_soft", ctypes.c_double),
                ("alpha_cross", ctypes.c_double), ("prior_decay", ctypes.c_double),
                ("tail_frac", ctypes.c_double), ("tail_brake", ctypes.c_double)]


class _Cache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("is_bf16", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_cap", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("len", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.orc_dense.argtypes = [ctypes.POINTER(_Cache), P, P, P, P, ctypes.c_int64]
        L.orc_select.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                                 ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 P, ctypes.c_int32, P, P]
        L.orc_sparse.argtypes = [ctypes.POINTER(_Cache), P, P, ctypes.c_int32, P,
                                 ctypes.c_int32, P, P, P]
        L.orc_sink_mask.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_double, P]
        L.orc_sparse_routed.argtypes = [ctypes.POINTER(_Cache), P, P, ctypes.c_int32, P,
                                        ctypes.c_int32, P, P, ctypes.c_double, P, P, P, P]
        L.orc_reorg.argtypes = [ctypes.POINTER(_Cache), P, ctypes.c_int32, P, P, P, P]
        L.orc_sparse_compact.argtypes = [ctypes.POINTER(_Cache), P, P, P, P, ctypes.c_int32, P,
                                         ctypes.c_int32, P, P, P]
        L.orc_select_refined.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                                         ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Refine),
                                         P, ctypes.c_int32, P, P, P]
        L.orc_threads.argtypes = []
        for f in (L.orc_dense, L.orc_select, L.orc_sparse, L.orc_sink_mask, L.orc_threads,
                  L.orc_sparse_routed, L.orc_reorg, L.orc_sparse_compact, L.orc_select_refined):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _host_bytes(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's raw bytes (bf16 kept as uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Cache:
    """Host copy of a KV cache in the library's layout (contiguous or paged)."""

    def __init__(self, k, v, lens, Hq, block_table=None, block_size=0, max_blocks=0):
        self.k = _host_bytes(k)
        self.v = _host_bytes(v)
        self.is_bf16 = int(k.dtype == torch.bfloat16)
        self.lens = np.ascontiguousarray(np.asarray(
            lens.cpu() if torch.is_tensor(lens) else lens, dtype=np.int32))
        self.B = int(self.lens.shape[0])
        self.Hq = int(Hq)
        if block_table is None:
            assert k.dim() == 4
            self.Hkv, self.n_cap, self.d = int(k.shape[1]), int(k.shape[2]), int(k.shape[3])
            self.bt = None
            self.block_size = 0
            self.max_blocks = 0
        else:
            self.Hkv, self.d = int(k.shape[1]), int(k.shape[3])
            self.n_cap = 0
            self.bt = _host_bytes(block_table.to(torch.int32))
            self.block_size = int(block_size)
            self.max_blocks = int(max_blocks)

    def with_lens(self, lens):
        c = object.__new__(Cache)
        c.__dict__.update(self.__dict__)
        c.lens = np.ascontiguousarray(np.asarray(
            lens.cpu() if torch.is_tensor(lens) else lens, dtype=np.int32))
        return c

    def _struct(self):
        return _Cache(self.B, self.Hq, self.Hkv, self.d, self.is_bf16,
                      self.k.ctypes.data, self.v.ctypes.data, self.n_cap,
                      self.bt.ctypes.data if self.bt is not None else None,
                      self.block_size, self.max_blocks, self.lens.ctypes.data)


def dense(cache: Cache, q, logit_stride: int | None = None, want_logits: bool = True):
    """Returns (out [B][Hq][d], lse [B][Hq], logits [B][Hq][stride] or None), float64."""
    qh = _host_bytes(q)
    stride = int(logit_stride or max(int(cache.lens.max()), 1))
    out = np.zeros((cache.B, cache.Hq, cache.d), np.float64)
    lse = np.zeros((cache.B, cache.Hq), np.float64)
    logits = np.full((cache.B, cache.Hq, stride), np.nan, np.float64) if want_logits else None
    s = cache._struct()
    rc = lib().orc_dense(ctypes.byref(s), _ptr(qh), _ptr(out), _ptr(lse),
                         _ptr(logits) if logits is not None else None, stride)
    assert rc == 0
    return out, lse, logits


def select(lens, Hq: int, Hkv: int, logits, n_sink: int, n_recent: int, k_sel: int,
           idx_stride: int | None = None, want_f: bool = False):
    """logits: array-like [B][Hq][stride] (fp32 values are widened exactly).
    Returns (idx int32 [B][Hkv][idx_stride], n_idx int32 [B][Hkv], f or None)."""
    z = np.ascontiguousarray(np.asarray(logits.cpu() if torch.is_tensor(logits) else logits,
                                        dtype=np.float64))
    B, _, stride = z.shape
    lens = np.ascontiguousarray(np.asarray(lens.cpu() if torch.is_tensor(lens) else lens,
                                           dtype=np.int32))
    idx_stride = int(idx_stride or (n_sink + k_sel))
    idx = np.zeros((B, Hkv, idx_stride), np.int32)
    n_idx = np.zeros((B, Hkv), np.int32)
    f = np.zeros((B, Hkv, stride), np.float64) if want_f else None
    rc = lib().orc_select(B, Hq, Hkv, _ptr(lens), _ptr(z), stride, n_sink, n_recent, k_sel,
                          _ptr(idx), idx_stride, _ptr(n_idx), _ptr(f) if f is not None else None)
    if rc != 0:
        raise ValueError("idx_stride too small for sink + selected")
    return idx, n_idx, f


REFINE_DEFAULTS = dict(lambda_=0.02, alpha_soft=0.5, alpha_cross=0.35, prior_decay=1.0,
                       tail_frac=1.0 / 16, tail_brake=1.0)


def select_refined(lens, Hq: int, Hkv: int, logits, n_sink: int, n_recent: int, k_sel: int,
                   key_norm=None, params: dict | None = None, idx_stride: int | None = None,
                   want_scores: bool = False):
    """The full Selector (prior, reverse-KL fusion, Soft-NMS, cross-head exclusivity, Top-K).
    logits [B][Hq][stride]; key_norm [B][Hkv][>= max len] or None; params override
    REFINE_DEFAULTS.  Returns (idx, n_idx, fused, refined): the log-scores before and after the
    refinements ([B][Hkv][stride], -inf outside J) when want_scores, else None."""
    z = np.ascontiguousarray(np.asarray(logits.cpu() if torch.is_tensor(logits) else logits,
                                        dtype=np.float64))
    B, _, stride = z.shape
    lens = _i32(lens)
    kn = None
    if key_norm is not None:
        kn = np.ascontiguousarray(np.asarray(
            key_norm.cpu() if torch.is_tensor(key_norm) else key_norm, dtype=np.float64))
    pr = dict(REFINE_DEFAULTS)
    pr.update(params or {})
    rp = _Refine(pr["lambda_"], pr["alpha_soft"], pr["alpha_cross"], pr["prior_decay"],
                 pr["tail_frac"], pr["tail_brake"])
    idx_stride = int(idx_stride or (n_sink + k_sel))
    idx = np.zeros((B, Hkv, idx_stride), np.int32)
    n_idx = np.zeros((B, Hkv), np.int32)
    fused = np.zeros((B, Hkv, stride), np.float64) if want_scores else None
    refined = np.zeros((B, Hkv, stride), np.float64) if want_scores else None
    rc = lib().orc_select_refined(B, Hq, Hkv, _ptr(lens), _ptr(z), stride,
                                  _ptr(kn) if kn is not None else None,
                                  kn.shape[-1] if kn is not None else 0, n_sink, n_recent, k_sel,
                                  ctypes.byref(rp), _ptr(idx), idx_stride, _ptr(n_idx),
                                  _ptr(fused) if fused is not None else None,
                                  _ptr(refined) if refined is not None else None)
    if rc != 0:
        raise ValueError("idx_stride too small for sink + selected")
    return idx, n_idx, fused, refined


def sparse(cache: Cache, q, idx, n_idx, n_recent: int, head_mask=None):
    """Returns (out [B][Hq][d], lse [B][Hq]) over sink+selected+recent, float64."""
    qh = _host_bytes(q)
    idx = np.ascontiguousarray(np.asarray(idx.cpu() if torch.is_tensor(idx) else idx,
                                          dtype=np.int32))
    n_idx = np.ascontiguousarray(np.asarray(n_idx.cpu() if torch.is_tensor(n_idx) else n_idx,
                                            dtype=np.int32))
    hm = None
    if head_mask is not None:
        hm = np.ascontiguousarray(np.asarray(
            head_mask.cpu() if torch.is_tensor(head_mask) else head_mask, dtype=np.uint8))
    out = np.zeros((cache.B, cache.Hq, cache.d), np.float64)
    lse = np.zeros((cache.B, cache.Hq), np.float64)
    s = cache._struct()
    rc = lib().orc_sparse(ctypes.byref(s), _ptr(qh), _ptr(idx), idx.shape[-1], _ptr(n_idx),
                          n_recent, _ptr(hm) if hm is not None else None, _ptr(out), _ptr(lse))
    assert rc == 0
    return out, lse


def _i32(a):
    return np.ascontiguousarray(np.asarray(a.cpu() if torch.is_tensor(a) else a, dtype=np.int32))


def reorg(cache: Cache, idx, n_idx):
    """Compact segment of the two-segment layout.  Returns (ck, cv, cpos): ck, cv hold
    [B][Hkv][idx_stride][d] rows in the cache's element format (uint16 bf16 bits or float32),
    cpos int32 [B][Hkv][idx_stride]."""
    idx = _i32(idx)
    n_idx = _i32(n_idx)
    B, Hkv, stride = idx.shape
    ck = np.empty((B, Hkv, stride, cache.d), cache.k.dtype)
    cv = np.empty_like(ck)
    cpos = np.empty((B, Hkv, stride), np.int32)
    s = cache._struct()
    rc = lib().orc_reorg(ctypes.byref(s), _ptr(idx), stride, _ptr(n_idx), _ptr(ck), _ptr(cv),
                         _ptr(cpos))
    assert rc == 0
    return ck, cv, cpos


def sparse_compact(cache: Cache, q, ck, cv, cpos, n_idx, n_recent: int, head_mask=None):
    """Fast step on the two-segment layout.  Returns (out [B][Hq][d], lse [B][Hq]), float64."""
    qh = _host_bytes(q)
    ck = np.ascontiguousarray(ck)
    cv = np.ascontiguousarray(cv)
    assert ck.dtype == cache.k.dtype and cv.dtype == cache.k.dtype
    cpos = _i32(cpos)
    n_idx = _i32(n_idx)
    hm = None
    if head_mask is not None:
        hm = np.ascontiguousarray(np.asarray(
            head_mask.cpu() if torch.is_tensor(head_mask) else head_mask, dtype=np.uint8))
    out = np.zeros((cache.B, cache.Hq, cache.d), np.float64)
    lse = np.zeros((cache.B, cache.Hq), np.float64)
    s = cache._struct()
    rc = lib().orc_sparse_compact(ctypes.byref(s), _ptr(qh), _ptr(ck), _ptr(cv), _ptr(cpos),
                                  cpos.shape[-1], _ptr(n_idx), n_recent,
                                  _ptr(hm) if hm is not None else None, _ptr(out), _ptr(lse))
    assert rc == 0
    return out, lse


def sparse_routed(cache: Cache, q, idx, n_idx, n_recent: int, route_lse, gamma: float,
                  head_mask=None):
    """Fast step with group routing.  Returns (out [B][Hq][d], lse [B][Hq], routed uint8
    [B][Hkv], margin [B][Hkv]) in float64; margin is the group's smallest
    z0 - route_lse - log(gamma) (routed exactly when it is >= 0)."""
    import math
    qh = _host_bytes(q)
    idx = np.ascontiguousarray(np.asarray(idx.cpu() if torch.is_tensor(idx) else idx,
                                          dtype=np.int32))
    n_idx = np.ascontiguousarray(np.asarray(n_idx.cpu() if torch.is_tensor(n_idx) else n_idx,
                                            dtype=np.int32))
    rl = np.ascontiguousarray(np.asarray(route_lse.cpu() if torch.is_tensor(route_lse)
                                         else route_lse, dtype=np.float64))
    hm = None
    if head_mask is not None:
        hm = np.ascontiguousarray(np.asarray(
            head_mask.cpu() if torch.is_tensor(head_mask) else head_mask, dtype=np.uint8))
    out = np.zeros((cache.B, cache.Hq, cache.d), np.float64)
    lse = np.zeros((cache.B, cache.Hq), np.float64)
    routed = np.zeros((cache.B, cache.Hkv), np.uint8)
    margin = np.zeros((cache.B, cache.Hkv), np.float64)
    s = cache._struct()
    rc = lib().orc_sparse_routed(ctypes.byref(s), _ptr(qh), _ptr(idx), idx.shape[-1], _ptr(n_idx),
                                 n_recent, _ptr(hm) if hm is not None else None, _ptr(rl),
                                 math.log(gamma), _ptr(margin), _ptr(routed), _ptr(out), _ptr(lse))
    assert rc == 0
    return out, lse, routed, margin


def sink_mask(z0, lse, frac: float):
    """z0, lse: [B][Hq].  Returns uint8 mask [B][Hq]."""
    z0 = np.ascontiguousarray(np.asarray(z0.cpu() if torch.is_tensor(z0) else z0, np.float64))
    lse = np.ascontiguousarray(np.asarray(lse.cpu() if torch.is_tensor(lse) else lse,
                                          np.float64))
    B, Hq = z0.shape
    m = np.zeros((B, Hq), np.uint8)
    rc = lib().orc_sink_mask(B, Hq, _ptr(z0), _ptr(lse), float(frac), _ptr(m))
    if rc != 0:
        raise ValueError("frac outside [0, 1]")
    return m


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(lib().orc_threads())
