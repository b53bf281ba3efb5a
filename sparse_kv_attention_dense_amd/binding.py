"""Thin ctypes binding of libsfi.so (include/sfi.h), with the same names as the C ABI.

Argument marshalling only: tensors are passed as device pointers, the stream is torch's
current HIP stream unless one is given, and a non-zero status raises ``SfiError``.  Every
computation happens in the library's HIP kernels; there is no fallback of any kind, and
importing this module fails loudly when libsfi.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsfi.so")

SFI_OK, SFI_E_INVALID, SFI_E_UNSUPPORTED, SFI_E_WORKSPACE, SFI_E_HIP = 0, -1, -2, -3, -4
SFI_E_SCRATCH = -5
SFI_NOALLOC_SCRATCH_BYTES = 8 << 20
SFI_F32, SFI_BF16 = 0, 1
SFI_OP_DENSE, SFI_OP_SELECT, SFI_OP_SPARSE, SFI_OP_SELECT_REFINED, SFI_OP_SLOW = 0, 1, 2, 3, 4

EXPORTED = ("sfi_dense_decode", "sfi_select", "sfi_slow_step", "sfi_select_refined", "sfi_sink_bypass_mask",
            "sfi_sparse_decode", "sfi_sparse_decode_noalloc", "sfi_sparse_decode_step",
            "sfi_sparse_decode_routed", "sfi_reorg", "sfi_sparse_decode_compact",
            "sfi_slow_step_layers", "sfi_workspace_bytes", "sfi_stream_read", "sfi_gather_read",
            "sfi_group_dot", "sfi_status_string")


class SfiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sfi_status_string(status)}")


class sfi_refine(ctypes.Structure):
    _fields_ = [("lambda_", ctypes.c_float), ("alpha_soft", ctypes.c_float),
                ("alpha_cross", ctypes.c_float), ("prior_decay", ctypes.c_float),
                ("tail_frac", ctypes.c_float), ("tail_brake", ctypes.c_float)]


REFINE_DEFAULTS = dict(lambda_=0.02, alpha_soft=0.5, alpha_cross=0.35, prior_decay=1.0,
                       tail_frac=1.0 / 16, tail_brake=1.0)


class sfi_step(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("q", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("n_idx", ctypes.c_void_p), ("head_mask", ctypes.c_void_p),
                ("seg_k", ctypes.c_void_p), ("seg_v", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("n_recent", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class sfi_kv_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n_cap", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("len", ctypes.c_void_p), ("max_len", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing; build it with "
                              "`python -m sparse_kv_attention_dense_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        D = ctypes.POINTER(sfi_kv_desc)
        L.sfi_dense_decode.argtypes = [D, P, P, P, P, i64, P, ctypes.c_size_t, P]
        L.sfi_select.argtypes = [D, P, i64, i32, i32, i32, P, i32, P, P, ctypes.c_size_t, P]
        L.sfi_slow_step.argtypes = [D, P, P, P, P, i64, i32, i32, i32, P, i32, P, ctypes.c_float,
                                    P, P, ctypes.c_size_t, P, P, P]
        L.sfi_sink_bypass_mask.argtypes = [D, P, i64, P, ctypes.c_float, P, P]
        L.sfi_sparse_decode.argtypes = [D, P, P, i32, P, i32, P, P, P, P, ctypes.c_size_t, P]
        L.sfi_sparse_decode_noalloc.argtypes = [D, P, P, i32, P, i32, P, P, P, P]
        L.sfi_sparse_decode_step.argtypes = [D, P, i32, i32, P, ctypes.c_size_t, P]
        L.sfi_sparse_decode_routed.argtypes = [D, P, P, i32, P, i32, P, P, ctypes.c_float, P,
                                               P, P, P, ctypes.c_size_t, P]
        L.sfi_slow_step_layers.argtypes = [i32, D, P, P, P, i32, P, i64, P, ctypes.c_size_t, P,
                                           ctypes.c_size_t, i32, i32, i32, P, i32, P,
                                           ctypes.c_float, P, P, P, P, P, P, P, P, P]
        L.sfi_gather_read.argtypes = [D, P, i32, P, i32, i32, P, P]
        L.sfi_workspace_bytes.argtypes = [D, i32, i32, i32]
        L.sfi_workspace_bytes.restype = ctypes.c_size_t
        L.sfi_reorg.argtypes = [D, P, i32, P, P, P, P, P]
        L.sfi_select_refined.argtypes = [D, P, i64, P, i64, i32, i32, i32,
                                         ctypes.POINTER(sfi_refine), P, i32, P, P,
                                         ctypes.c_size_t, P]
        L.sfi_sparse_decode_compact.argtypes = [D, P, P, P, P, i32, P, i32, P, P, P, P,
                                                ctypes.c_size_t, P]
        L.sfi_stream_read.argtypes = [P, ctypes.c_uint64, i32, P, P]
        L.sfi_group_dot.argtypes = [P, i64, P, i32, i32, i32, P, P, P]
        L.sfi_status_string.argtypes = [ctypes.c_int]
        L.sfi_status_string.restype = ctypes.c_char_p
        for f in ("sfi_dense_decode", "sfi_select", "sfi_sink_bypass_mask", "sfi_sparse_decode",
                  "sfi_sparse_decode_routed", "sfi_slow_step_layers", "sfi_stream_read",
                  "sfi_reorg", "sfi_sparse_decode_compact", "sfi_select_refined",
                  "sfi_group_dot"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    # a plain int: the argtypes turn it into a void* without a ctypes object per argument
    return None if t is None else t.data_ptr()


def _current_raw_stream():
    """torch's current HIP stream on the current device, as an address.  torch's raw-stream
    query avoids building a torch.cuda.Stream object on every call; the public path is the
    fallback."""
    try:
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    except AttributeError:
        return torch.cuda.current_stream().cuda_stream


def _stream(stream):
    if stream is not None:
        return int(stream)
    if torch.cuda.is_available():
        return _current_raw_stream()
    return None


def _check(status: int, where: str):
    if status != SFI_OK:
        raise SfiError(status, where)


_F32, _I32, _U8 = torch.float32, torch.int32, torch.uint8
_CACHE_DTYPES = {torch.float32: SFI_F32, torch.bfloat16: SFI_BF16}


def _buf(t, name: str, dtype=None, numel: int = 0, optional: bool = False,
         device: bool = True):
    """Checks a tensor before its pointer crosses the C ABI.  The library sees only the
    address, so a buffer of another dtype, a strided view or one smaller than the call's
    sizes would be read or written past its end by a kernel; such calls raise here instead.
    The common case is one combined test; a failure is then diagnosed in this order: type,
    dtype, contiguity, size, GPU residence."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: a tensor is required")
    try:
        if ((dtype is None or t.dtype is dtype) and t.is_contiguous() and t.numel() >= numel
                and (t.is_cuda or not device)):
            return
    except AttributeError:
        pass
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: holds {t.numel()} elements, the call needs {numel}")
    raise ValueError(f"{name}: must be in GPU memory, is on {t.device}")


class KVDesc:
    """Builds an ``sfi_kv_desc`` from tensors and keeps them alive while it is in use.

    k, v: contiguous [B][Hkv][n_cap][d] or paged [num_blocks][Hkv][block_size][d], fp32 or
    bf16.  lens: int32 [B] on the device.  max_len: host bound of lens.  block_table: int32
    [B][max_blocks] on the device for the paged layout.
    """

    def __init__(self, k, v, lens, max_len: int, num_q_heads: int, block_table=None,
                 block_size: int = 0, batch: Optional[int] = None):
        self._keep = (k, v, lens, block_table)
        n_batch = int(batch if batch is not None else lens.shape[0])
        _buf(lens, "lens", _I32, n_batch, device=False)
        if k is not None:
            if k.dtype not in _CACHE_DTYPES:
                raise TypeError(f"k: dtype {k.dtype}, expected torch.float32 or torch.bfloat16")
            if k.dim() != 4:
                raise ValueError("k: expected [B][Hkv][n_cap][d] or [num_blocks][Hkv][block_size][d]")
            _buf(k, "k", k.dtype, device=False)
            _buf(v, "v", k.dtype, device=False)
            if tuple(v.shape) != tuple(k.shape):
                raise ValueError(f"v: shape {tuple(v.shape)} differs from k {tuple(k.shape)}")
            if block_table is None and int(k.shape[0]) < n_batch:
                raise ValueError(f"k: {int(k.shape[0])} sequences, the batch has {n_batch}")
            if block_table is not None:
                if block_table.dim() != 2:
                    raise ValueError("block_table: expected [B][max_blocks]")
                _buf(block_table, "block_table", _I32, n_batch * int(block_table.shape[1]),
                     device=False)
                if int(k.shape[2]) != int(block_size):
                    raise ValueError(f"k: pages of {int(k.shape[2])} positions, block_size "
                                     f"says {block_size}")
            dtype = _CACHE_DTYPES[k.dtype]
            hkv, d = int(k.shape[1]), int(k.shape[-1])
        else:
            dtype, hkv, d = SFI_F32, 0, 0
        for name, t in (("lens", lens), ("k", k), ("v", v), ("block_table", block_table)):
            _buf(t, name, optional=True)                     # GPU residence, checked last
        self.cache_dtype = k.dtype if k is not None else None
        self.c = sfi_kv_desc()
        self.c.batch = n_batch
        self.c.num_q_heads = int(num_q_heads)
        self.c.num_kv_heads = hkv
        self.c.head_dim = d
        self.c.dtype = dtype
        self.c.k = k.data_ptr() if k is not None else None
        self.c.v = v.data_ptr() if v is not None else None
        self.c.n_cap = int(k.shape[2]) if (k is not None and block_table is None) else 0
        self.c.block_table = block_table.data_ptr() if block_table is not None else None
        self.c.block_size = int(block_size)
        self.c.max_blocks = int(block_table.shape[1]) if block_table is not None else 0
        self.c.len = lens.data_ptr() if lens is not None else None
        self.c.max_len = int(max_len)

    @classmethod
    def for_logits(cls, lens, max_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int = 128):
        """Descriptor for calls that read no cache (sfi_select, sfi_sink_bypass_mask)."""
        d = cls(None, None, lens, max_len, num_q_heads)
        d.c.num_kv_heads = int(num_kv_heads)
        if int(num_kv_heads) < 1:
            raise ValueError("num_kv_heads must be at least 1")
        d.c.head_dim = int(head_dim)
        d.c.dtype = SFI_BF16
        return d

    def with_lens(self, lens, max_len: int) -> "KVDesc":
        """Same cache, other lengths (a later decode step)."""
        _buf(lens, "lens", _I32, self.c.batch)
        d = object.__new__(KVDesc)
        d._keep = self._keep + (lens,)
        d.cache_dtype = self.cache_dtype
        d.c = sfi_kv_desc.from_buffer_copy(self.c)
        d.c.len = lens.data_ptr()
        d.c.max_len = int(max_len)
        return d

    @property
    def ref(self):
        return ctypes.byref(self.c)

    # sizes that the calls' buffers must cover (elements)
    @property
    def heads(self) -> int:                 # query heads over the batch
        return self.c.batch * self.c.num_q_heads

    @property
    def units(self) -> int:                 # (sequence, KV head) units over the batch
        return self.c.batch * self.c.num_kv_heads

    def need_cache(self, what: str):
        if self.cache_dtype is None:
            raise ValueError(f"{what}: the descriptor has no cache (KVDesc.for_logits)")


def sfi_status_string(status: int) -> str:
    return lib().sfi_status_string(int(status)).decode()


def sfi_workspace_bytes(desc: KVDesc, op: int, idx_stride: int = 0, n_recent: int = 0) -> int:
    return int(lib().sfi_workspace_bytes(desc.ref, int(op), int(idx_stride), int(n_recent)))


def sfi_stream_read(buf, n_workgroups: int, sink, stream=None):
    """Sequential read of the whole of `buf` (a measurement yardstick); sink: >= 64 int32."""
    _buf(buf, "buf")
    _buf(sink, "sink", _I32, 64)
    _check(lib().sfi_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(n_workgroups),
                                 _ptr(sink), _stream(stream)), "sfi_stream_read")


GROUP_DOT_UNITS = {"read": 0, "valu": 1, "mfma": 2}


def sfi_group_dot(rows, q, unit: str, n_workgroups: int, part, sink, stream=None):
    """The GQA group's dot products with bf16 key rows of 128 elements (a measurement
    yardstick): rows [n_rows][128] and q [G][128] bf16, unit "read", "valu" or "mfma"; part
    float32 [n_workgroups] takes per-workgroup sums (not written by "read"); sink >= 64 int32."""
    _buf(rows, "rows", torch.bfloat16)
    _buf(q, "q", torch.bfloat16)
    if rows.numel() % 128 or q.numel() % 128:
        raise ValueError("sfi_group_dot: rows and q hold rows of 128 elements")
    _buf(part, "part", _F32, int(n_workgroups))
    _buf(sink, "sink", _I32, 64)
    _check(lib().sfi_group_dot(_ptr(rows), rows.numel() // 128, _ptr(q), q.numel() // 128,
                               GROUP_DOT_UNITS[unit], int(n_workgroups), _ptr(part), _ptr(sink),
                               _stream(stream)), "sfi_group_dot")


def sfi_gather_read(desc: KVDesc, idx, idx_stride: int, n_idx, n_recent: int,
                    n_workgroups: int, sink, stream=None):
    desc.need_cache("sfi_gather_read")
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    _buf(n_idx, "n_idx", _I32, desc.units)
    _buf(sink, "sink", _I32, 64)
    _check(lib().sfi_gather_read(desc.ref, _ptr(idx), int(idx_stride), _ptr(n_idx),
                                 int(n_recent), int(n_workgroups), _ptr(sink), _stream(stream)),
           "sfi_gather_read")


def sfi_dense_decode(desc: KVDesc, q, out, lse, logits, logit_stride: int, ws, stream=None):
    desc.need_cache("sfi_dense_decode")
    _buf(q, "q", desc.cache_dtype, desc.heads * desc.c.head_dim)
    _buf(out, "out", _F32, desc.heads * desc.c.head_dim)
    _buf(lse, "lse", _F32, desc.heads, optional=True)
    _buf(logits, "logits", _F32, desc.heads * int(logit_stride), optional=True)
    _buf(ws, "ws")
    _check(lib().sfi_dense_decode(desc.ref, _ptr(q), _ptr(out), _ptr(lse), _ptr(logits),
                                  int(logit_stride), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "sfi_dense_decode")


def sfi_slow_step(desc: KVDesc, q, out, lse, logits, logit_stride: int, n_sink: int,
                  n_recent: int, k_sel: int, idx, idx_stride: int, n_idx, mask_frac: float,
                  head_mask, ws, dense_done=None, stream=None, dense_begin=None):
    """dense_begin, dense_done: torch.cuda.Events (recorded right before and after the dense
    kernels, after the library's own checks) or None."""
    desc.need_cache("sfi_slow_step")
    _buf(q, "q", desc.cache_dtype, desc.heads * desc.c.head_dim)
    _buf(out, "out", _F32, desc.heads * desc.c.head_dim)
    _buf(lse, "lse", _F32, desc.heads)
    _selector_bufs(desc, logits, logit_stride, idx, idx_stride, n_idx, ws)
    _buf(head_mask, "head_mask", _U8, desc.heads, optional=True)
    st = _stream(stream)
    ev = _event_handle(dense_done, stream) if dense_done is not None else None
    eb = _event_handle(dense_begin, stream) if dense_begin is not None else None
    _check(lib().sfi_slow_step(desc.ref, _ptr(q), _ptr(out), _ptr(lse), _ptr(logits),
                               int(logit_stride), int(n_sink), int(n_recent), int(k_sel),
                               _ptr(idx), int(idx_stride), _ptr(n_idx), float(mask_frac),
                               _ptr(head_mask), _ptr(ws), ws.numel() * ws.element_size(),
                               eb, ev, st), "sfi_slow_step")


def _selector_bufs(desc: KVDesc, logits, logit_stride: int, idx, idx_stride: int, n_idx, ws):
    _buf(logits, "logits", _F32, desc.heads * int(logit_stride))
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    _buf(n_idx, "n_idx", _I32, desc.units)
    _buf(ws, "ws")


def sfi_select(desc: KVDesc, logits, logit_stride: int, n_sink: int, n_recent: int, k_sel: int,
               idx, idx_stride: int, n_idx, ws, stream=None):
    _selector_bufs(desc, logits, logit_stride, idx, idx_stride, n_idx, ws)
    _check(lib().sfi_select(desc.ref, _ptr(logits), int(logit_stride), int(n_sink),
                            int(n_recent), int(k_sel), _ptr(idx), int(idx_stride), _ptr(n_idx),
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "sfi_select")


def sfi_select_refined(desc: KVDesc, logits, logit_stride: int, key_norm, norm_stride: int,
                       n_sink: int, n_recent: int, k_sel: int, params: dict, idx,
                       idx_stride: int, n_idx, ws, stream=None):
    _selector_bufs(desc, logits, logit_stride, idx, idx_stride, n_idx, ws)
    _buf(key_norm, "key_norm", _F32, desc.units * int(norm_stride), optional=True)
    pr = dict(REFINE_DEFAULTS)
    pr.update(params or {})
    p = sfi_refine(pr["lambda_"], pr["alpha_soft"], pr["alpha_cross"], pr["prior_decay"],
                   pr["tail_frac"], pr["tail_brake"])
    _check(lib().sfi_select_refined(desc.ref, _ptr(logits), int(logit_stride), _ptr(key_norm),
                                    int(norm_stride), int(n_sink), int(n_recent), int(k_sel),
                                    ctypes.byref(p), _ptr(idx), int(idx_stride), _ptr(n_idx),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "sfi_select_refined")


def sfi_sink_bypass_mask(desc: KVDesc, logits, logit_stride: int, lse, frac: float, head_mask,
                         stream=None):
    _buf(logits, "logits", _F32, (desc.heads - 1) * int(logit_stride) + 1)
    _buf(lse, "lse", _F32, desc.heads)
    _buf(head_mask, "head_mask", _U8, desc.heads)
    _check(lib().sfi_sink_bypass_mask(desc.ref, _ptr(logits), int(logit_stride), _ptr(lse),
                                      float(frac), _ptr(head_mask), _stream(stream)),
           "sfi_sink_bypass_mask")


def _fast_bufs(desc: KVDesc, what: str, q, n_idx, head_mask, out, lse, ws):
    desc.need_cache(what)
    _buf(q, "q", desc.cache_dtype, desc.heads * desc.c.head_dim)
    _buf(n_idx, "n_idx", _I32, desc.units)
    _buf(head_mask, "head_mask", _U8, desc.heads, optional=True)
    _buf(out, "out", _F32, desc.heads * desc.c.head_dim)
    _buf(lse, "lse", _F32, desc.heads, optional=True)
    _buf(ws, "ws")


def sfi_sparse_decode(desc: KVDesc, q, idx, idx_stride: int, n_idx, n_recent: int, head_mask,
                      out, lse, ws, stream=None):
    _fast_bufs(desc, "sfi_sparse_decode", q, n_idx, head_mask, out, lse, ws)
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    _check(lib().sfi_sparse_decode(desc.ref, _ptr(q), _ptr(idx), int(idx_stride), _ptr(n_idx),
                                   int(n_recent), _ptr(head_mask), _ptr(out), _ptr(lse),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "sfi_sparse_decode")


def sfi_sparse_decode_noalloc(desc: KVDesc, q, idx, idx_stride: int, n_idx, n_recent: int,
                              head_mask, out, lse, stream=None):
    desc.need_cache("sfi_sparse_decode_noalloc")
    _buf(q, "q", desc.cache_dtype, desc.heads * desc.c.head_dim)
    _buf(n_idx, "n_idx", _I32, desc.units)
    _buf(head_mask, "head_mask", _U8, desc.heads, optional=True)
    _buf(out, "out", _F32, desc.heads * desc.c.head_dim)
    _buf(lse, "lse", _F32, desc.heads, optional=True)
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    _check(lib().sfi_sparse_decode_noalloc(desc.ref, _ptr(q), _ptr(idx), int(idx_stride),
                                           _ptr(n_idx), int(n_recent), _ptr(head_mask), _ptr(out),
                                           _ptr(lse), _stream(stream)),
           "sfi_sparse_decode_noalloc")


def step_descriptor(device="cuda") -> torch.Tensor:
    """Device memory for one sfi_step (plumbing: torch allocates it once)."""
    return torch.zeros(256, dtype=torch.uint8, device=device)


def write_step(step_buf, desc: KVDesc, q, idx, idx_stride: int, n_idx, n_recent: int,
               head_mask, out, lse, segment=None, stream=None):
    """Checks this step's buffers as sfi_sparse_decode does (desc gives the cache, the lengths
    and, when paged, the block table of the step), packs an sfi_step on the host and copies it
    into step_buf on the stream.  segment: (ck, cv) of the two-segment layout, with idx its
    cpos, or None."""
    desc.need_cache("write_step")
    _fast_bufs(desc, "write_step", q, n_idx, head_mask, out, lse, step_buf)
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    ck = cv = None
    if segment is not None:
        ck, cv = segment
        rows = desc.units * int(idx_stride) * desc.c.head_dim
        _buf(ck, "seg_k", desc.cache_dtype, rows)
        _buf(cv, "seg_v", desc.cache_dtype, rows)
    c = desc.c
    st = sfi_step(c.k, c.v, c.block_table, c.len, _ptr(q), _ptr(idx), _ptr(n_idx),
                  _ptr(head_mask), _ptr(ck), _ptr(cv), _ptr(out), _ptr(lse), int(n_recent), 0)
    raw = torch.frombuffer(bytearray(bytes(st)), dtype=torch.uint8)
    s = torch.cuda.current_stream() if stream is None else stream
    with torch.cuda.stream(s):
        step_buf[:raw.numel()].copy_(raw)


def sfi_sparse_decode_step(desc: KVDesc, step_buf, idx_stride: int, max_recent: int, ws,
                           stream=None):
    """desc gives the shapes and the cache's capacity; the step's pointers come from
    step_buf (written by write_step)."""
    desc.need_cache("sfi_sparse_decode_step")
    _buf(step_buf, "step", _U8, ctypes.sizeof(sfi_step))
    _buf(ws, "ws")
    _check(lib().sfi_sparse_decode_step(desc.ref, _ptr(step_buf), int(idx_stride),
                                        int(max_recent), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)), "sfi_sparse_decode_step")


def sfi_sparse_decode_routed(desc: KVDesc, q, idx, idx_stride: int, n_idx, n_recent: int,
                             head_mask, route_lse, gamma: float, routed, out, lse, ws,
                             stream=None):
    _fast_bufs(desc, "sfi_sparse_decode_routed", q, n_idx, head_mask, out, lse, ws)
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    _buf(route_lse, "route_lse", _F32, desc.heads)
    _buf(routed, "routed", _U8, desc.units, optional=True)
    _check(lib().sfi_sparse_decode_routed(desc.ref, _ptr(q), _ptr(idx), int(idx_stride),
                                          _ptr(n_idx), int(n_recent), _ptr(head_mask),
                                          _ptr(route_lse), float(gamma), _ptr(routed), _ptr(out),
                                          _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)),
           "sfi_sparse_decode_routed")


def _segment_bufs(desc: KVDesc, idx_stride: int, ck, cv, cpos):
    rows = desc.units * int(idx_stride)
    _buf(ck, "seg_k", desc.cache_dtype, rows * desc.c.head_dim)
    _buf(cv, "seg_v", desc.cache_dtype, rows * desc.c.head_dim)
    _buf(cpos, "seg_pos", _I32, rows)


def sfi_reorg(desc: KVDesc, idx, idx_stride: int, n_idx, ck, cv, cpos, stream=None):
    desc.need_cache("sfi_reorg")
    _buf(idx, "idx", _I32, desc.units * int(idx_stride))
    _buf(n_idx, "n_idx", _I32, desc.units)
    _segment_bufs(desc, idx_stride, ck, cv, cpos)
    _check(lib().sfi_reorg(desc.ref, _ptr(idx), int(idx_stride), _ptr(n_idx), _ptr(ck), _ptr(cv),
                           _ptr(cpos), _stream(stream)), "sfi_reorg")


def sfi_sparse_decode_compact(desc: KVDesc, q, ck, cv, cpos, idx_stride: int, n_idx,
                              n_recent: int, head_mask, out, lse, ws, stream=None):
    _fast_bufs(desc, "sfi_sparse_decode_compact", q, n_idx, head_mask, out, lse, ws)
    _segment_bufs(desc, idx_stride, ck, cv, cpos)
    _check(lib().sfi_sparse_decode_compact(desc.ref, _ptr(q), _ptr(ck), _ptr(cv), _ptr(cpos),
                                           int(idx_stride), _ptr(n_idx), int(n_recent),
                                           _ptr(head_mask), _ptr(out), _ptr(lse), _ptr(ws),
                                           ws.numel() * ws.element_size(), _stream(stream)),
           "sfi_sparse_decode_compact")


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def _event_handle(ev, stream):
    """Raw HIP event of a torch.cuda.Event (torch creates it on the first record)."""
    if not ev.cuda_event:
        ev.record(stream)
    return ev.cuda_event


def sfi_slow_step_layers(descs, qs, outs, lses, logits_slots, logit_stride: int, sel_ws_slots,
                         dense_ws, n_sink: int, n_recent: int, k_sel: int, idxs, idx_stride: int,
                         n_idxs, mask_frac: float, head_masks, stream, side_stream, slot_events,
                         attn_event, done_event, segments=None):
    """Layer-wise slow step (see include/sfi.h).  descs, qs, outs, lses, idxs, n_idxs,
    head_masks: one per layer (head_masks may be None); logits_slots, sel_ws_slots and
    slot_events: one per ring slot; streams are torch.cuda.Stream, events torch.cuda.Event.
    segments: None, or one (seg_k, seg_v, seg_pos) per layer for a Reorg after each Selector."""
    n, r = len(descs), len(logits_slots)
    for name, xs, want in (("qs", qs, n), ("outs", outs, n), ("lses", lses, n), ("idxs", idxs, n),
                           ("n_idxs", n_idxs, n), ("sel_ws_slots", sel_ws_slots, r),
                           ("slot_events", slot_events, r)):
        if len(xs) != want:
            raise ValueError(f"{name}: {len(xs)} entries, expected {want}")
    for li, d in enumerate(descs):
        d.need_cache("sfi_slow_step_layers")
        _buf(qs[li], f"qs[{li}]", d.cache_dtype, d.heads * d.c.head_dim)
        _buf(outs[li], f"outs[{li}]", _F32, d.heads * d.c.head_dim)
        _buf(lses[li], f"lses[{li}]", _F32, d.heads)
        _buf(idxs[li], f"idxs[{li}]", _I32, d.units * int(idx_stride))
        _buf(n_idxs[li], f"n_idxs[{li}]", _I32, d.units)
        if head_masks is not None:
            _buf(head_masks[li], f"head_masks[{li}]", _U8, d.heads, optional=True)
        if segments is not None:
            _segment_bufs(d, idx_stride, *segments[li])
        for si, lg in enumerate(logits_slots):
            _buf(lg, f"logits_slots[{si}]", _F32, d.heads * int(logit_stride))
    for si, w in enumerate(sel_ws_slots):
        _buf(w, f"sel_ws_slots[{si}]")
    _buf(dense_ws, "dense_ws")
    darr = (sfi_kv_desc * n)(*[d.c for d in descs])
    evs = (ctypes.c_void_p * r)(*[_event_handle(e, side_stream) for e in slot_events])
    sel_bytes = min(w.numel() * w.element_size() for w in sel_ws_slots)
    _check(lib().sfi_slow_step_layers(
        n, darr, _ptr_array(qs), _ptr_array(outs), _ptr_array(lses), r, _ptr_array(logits_slots),
        int(logit_stride), _ptr_array(sel_ws_slots), sel_bytes, _ptr(dense_ws),
        dense_ws.numel() * dense_ws.element_size(), int(n_sink), int(n_recent), int(k_sel),
        _ptr_array(idxs), int(idx_stride), _ptr_array(n_idxs), float(mask_frac),
        None if head_masks is None else _ptr_array(head_masks),
        None if segments is None else _ptr_array([t[0] for t in segments]),
        None if segments is None else _ptr_array([t[1] for t in segments]),
        None if segments is None else _ptr_array([t[2] for t in segments]),
        ctypes.c_void_p(stream.cuda_stream), ctypes.c_void_p(side_stream.cuda_stream), evs,
        ctypes.c_void_p(_event_handle(attn_event, stream)),
        ctypes.c_void_p(_event_handle(done_event, side_stream))), "sfi_slow_step_layers")


def workspace(desc: KVDesc, idx_stride: int = 1, n_recent: int = 0, device="cuda",
              refined: bool = False):
    """A workspace large enough for every op on this descriptor (plumbing:
    torch allocates it once; the library itself never allocates).  refined: also for
    sfi_select_refined."""
    ops = (SFI_OP_DENSE, SFI_OP_SELECT, SFI_OP_SPARSE, SFI_OP_SLOW) + (
        (SFI_OP_SELECT_REFINED,) if refined else ())
    n = max(sfi_workspace_bytes(desc, op, idx_stride, n_recent) for op in ops)
    if n == 0:
        raise SfiError(SFI_E_INVALID, "workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)
