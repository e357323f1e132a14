"""Thin ctypes binding of libyoco_xattn.so.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no fallback: if the library is missing, loading raises. Before each
call the binding checks what the C ABI cannot see (dtype, device, shape and
contiguity of every tensor) and raises YocoError(INVALID_ARG) on a mismatch.

The functions mirror the C ABI (include/yoco_xattn.h) one to one:
``kv_append``, ``kv_append_ring``, ``xattn_prefill``, ``xattn_prefill_window``,
``xattn_decode``, ``xattn_decode_noalloc``, ``xattn_decode_window``, ``workspace_size``, ``decode_splits``,
``kv_project_pack``, ``kv_project_append``, ``gret_workspace_size``, ``gret_prefill``,
``gret_decode``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libyoco_xattn.so")

YOCO_OK = 0
YOCO_ERR_INVALID_ARG = 1
NOALLOC_SCRATCH_BYTES = 8 << 20   # YOCO_NOALLOC_SCRATCH_BYTES of the C header
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip launch failed"}
DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1}

EXPORTS = ("yoco_kv_append", "yoco_kv_append_ring", "yoco_xattn_prefill", "yoco_xattn_prefill_window",
           "yoco_xattn_decode", "yoco_xattn_decode_noalloc", "yoco_xattn_decode_window", "yoco_xattn_workspace_size",
           "yoco_xattn_decode_splits", "yoco_kv_project_pack", "yoco_kv_project_append", "yoco_gret_workspace_size",
           "yoco_gret_prefill", "yoco_gret_decode", "yoco_status_string")


class YocoError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class KvCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pool_rows", ctypes.c_int64),
                ("seq_start", ctypes.c_void_p), ("seq_len", ctypes.c_void_p), ("seq_cap", ctypes.c_void_p)]


class GretDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Residual(ctypes.Structure):
    _fields_ = [("k1", ctypes.c_void_p), ("v1", ctypes.c_void_p), ("lam", ctypes.c_float),
                ("a_k", ctypes.c_float * 2), ("a_v", ctypes.c_float * 2)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the library. Raises OSError when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run decoder_shared_kv_amd.build.build() first")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    dims_p = ctypes.POINTER(Dims)
    cache_p = ctypes.POINTER(KvCache)
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.yoco_kv_append.argtypes = [dims_p, cache_p, P, P, P, P]
    lib.yoco_kv_append_ring.argtypes = [dims_p, cache_p, P, P, P, P]
    sz = ctypes.c_size_t
    lib.yoco_xattn_prefill.argtypes = [dims_p, cache_p, P, P, i32, i64, P, P, P, sz, P]
    lib.yoco_xattn_prefill_window.argtypes = [dims_p, cache_p, P, P, i32, i64, i32, P, P, P, sz, P]
    lib.yoco_xattn_decode.argtypes = [dims_p, cache_p, P, i32, i64, P, P, P, ctypes.c_size_t, P]
    lib.yoco_xattn_decode_noalloc.argtypes = [dims_p, cache_p, P, i32, i64, P, P, P]
    lib.yoco_xattn_decode_window.argtypes = [dims_p, cache_p, P, i32, i64, i32, P, P, P, ctypes.c_size_t, P]
    lib.yoco_kv_project_pack.argtypes = [dims_p, i32, P, P, P, P, P]
    lib.yoco_kv_project_append.argtypes = [dims_p, cache_p, P, P, i64, i32, P, ctypes.c_float,
                                           ctypes.POINTER(Residual), P, P]
    gdims_p = ctypes.POINTER(GretDims)
    lib.yoco_gret_workspace_size.argtypes = [gdims_p, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.yoco_gret_prefill.argtypes = [gdims_p, P, P, P, P, P, i64, P, P, P, P, ctypes.c_size_t, P]
    lib.yoco_gret_decode.argtypes = [gdims_p, P, P, P, P, P, P, P]
    lib.yoco_xattn_workspace_size.argtypes = [dims_p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.yoco_xattn_decode_splits.argtypes = [dims_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_int32)]
    lib.yoco_status_string.argtypes = [ctypes.c_int]
    lib.yoco_status_string.restype = ctypes.c_char_p
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _need(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None, optional: bool = False) -> None:
    """Raise YocoError(INVALID_ARG) unless t is a contiguous tensor of this dtype, shape and device."""
    if t is None:
        if optional:
            return
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} is missing")
    if not isinstance(t, torch.Tensor):
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} is not a tensor")
    if dtype is not None and t.dtype != dtype:
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} is not contiguous")


@dataclass
class SharedKV:
    """The one shared K^,V^ pool and its per-sequence metadata (all device tensors)."""
    k: torch.Tensor          # [pool_rows, Hkv, d]
    v: torch.Tensor
    seq_start: torch.Tensor  # int64 [B]
    seq_len: torch.Tensor    # int32 [B]
    seq_cap: torch.Tensor    # int32 [B]

    def validate(self) -> None:
        """The pool and its metadata: one dtype, one device, dense, int64 starts, int32 lengths."""
        if self.k.dim() != 3:
            raise YocoError(YOCO_ERR_INVALID_ARG, f"k must be [rows, Hkv, d], got {tuple(self.k.shape)}")
        if self.k.dtype not in DTYPE_CODE:
            raise YocoError(2, f"cache dtype {self.k.dtype}")
        dev = self.k.device
        _need(self.k, "k", device=dev)
        _need(self.v, "v", self.k.dtype, self.k.shape, dev)
        b = int(self.seq_len.shape[0]) if self.seq_len.dim() == 1 else -1
        _need(self.seq_start, "seq_start", torch.int64, (b,), dev)
        _need(self.seq_len, "seq_len", torch.int32, (b,), dev)
        _need(self.seq_cap, "seq_cap", torch.int32, (b,), dev)

    def descriptor(self) -> KvCache:
        self.validate()
        return KvCache(self.k.data_ptr(), self.v.data_ptr(), int(self.k.shape[0]), self.seq_start.data_ptr(),
                       self.seq_len.data_ptr(), self.seq_cap.data_ptr())


def make_dims(batch: int, q_heads: int, kv_heads: int, head_dim: int, dtype: torch.dtype, scale: float) -> Dims:
    if dtype not in DTYPE_CODE:
        raise YocoError(2, f"dtype {dtype}")
    return Dims(batch, q_heads, kv_heads, head_dim, DTYPE_CODE[dtype], float(scale))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, what: str) -> None:
    if status != YOCO_OK:
        raise YocoError(status, what)


def _dims_for(cache: SharedKV, q_heads: int, scale: float, batch: int) -> Dims:
    return make_dims(batch, q_heads, cache.k.shape[1], cache.k.shape[2], cache.k.dtype, scale)


def _rows(cache: SharedKV, t: torch.Tensor, name: str) -> None:
    """t is [B, Hkv, d] in the cache's dtype and device (appended rows)."""
    b = int(cache.seq_len.shape[0])
    _need(t, name, cache.k.dtype, (b, cache.k.shape[1], cache.k.shape[2]), cache.k.device)


def _flag(t: Optional[torch.Tensor], cache: SharedKV, name: str) -> None:
    if t is not None:
        _need(t, name, torch.int32, device=cache.k.device)
        if t.numel() < 1:
            raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} is empty")


def _queries(cache: SharedKV, q: torch.Tensor, name: str = "q") -> None:
    if q is None or q.dim() != 3:
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} must be [rows, Hq, d]")
    _need(q, name, cache.k.dtype, device=cache.k.device)
    if int(q.shape[2]) != int(cache.k.shape[2]) or int(q.shape[1]) % int(cache.k.shape[1]) != 0:
        raise YocoError(YOCO_ERR_INVALID_ARG, f"{name} shape {tuple(q.shape)} does not fit the cache's heads")


def _out_lse(q: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor], lse_shape) -> None:
    _need(out, "out", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, lse_shape, q.device, optional=True)


def kv_append(cache: SharedKV, k_new: torch.Tensor, v_new: torch.Tensor, overflow: Optional[torch.Tensor] = None,
              q_heads: Optional[int] = None, stream=None) -> None:
    """Append one row per sequence (k_new, v_new: [B, Hkv, d]); see yoco_kv_append."""
    lib = load_library()
    batch = int(cache.seq_len.shape[0])
    dims = _dims_for(cache, q_heads or cache.k.shape[1], 1.0, batch)
    desc = cache.descriptor()
    _rows(cache, k_new, "k_new")
    _rows(cache, v_new, "v_new")
    _flag(overflow, cache, "overflow")
    _check(lib.yoco_kv_append(ctypes.byref(dims), ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(overflow),
                              _stream(stream)), "yoco_kv_append")


def kv_append_ring(cache: SharedKV, k_new: torch.Tensor, v_new: torch.Tensor, flag: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Append one row per sequence to ring window caches (slot seq_len mod seq_cap); see yoco_kv_append_ring."""
    lib = load_library()
    batch = int(cache.seq_len.shape[0])
    dims = _dims_for(cache, cache.k.shape[1], 1.0, batch)
    desc = cache.descriptor()
    _rows(cache, k_new, "k_new")
    _rows(cache, v_new, "v_new")
    _flag(flag, cache, "flag")
    _check(lib.yoco_kv_append_ring(ctypes.byref(dims), ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(flag),
                                   _stream(stream)), "yoco_kv_append_ring")


def _prefill_args(cache: SharedKV, q: torch.Tensor, cu_seqlens: torch.Tensor, out, lse, workspace):
    desc = cache.descriptor()
    _need(workspace, "workspace", torch.uint8, device=cache.k.device, optional=True)
    _queries(cache, q)
    total_q, hq, _ = q.shape
    if cu_seqlens is None or cu_seqlens.dim() != 1 or int(cu_seqlens.shape[0]) != int(cache.seq_len.shape[0]) + 1:
        raise YocoError(YOCO_ERR_INVALID_ARG, "cu_seqlens must be [B + 1] with B the cache's sequences")
    _need(cu_seqlens, "cu_seqlens", torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _out_lse(q, out, lse, (hq, total_q))
    return desc, out


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else int(t.numel() * t.element_size())


def xattn_prefill(cache: SharedKV, q: torch.Tensor, cu_seqlens: torch.Tensor, max_q_len: int, scale: float,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None,
                  workspace: Optional[torch.Tensor] = None):
    """Causal prefill over packed queries q [total_q, Hq, d]; returns out (and fills lse [Hq, total_q]).

    workspace: the work queue (alloc_prefill_workspace: zeroed once, left zero by
    every call), or None for the static grid."""
    lib = load_library()
    desc, out = _prefill_args(cache, q, cu_seqlens, out, lse, workspace)
    total_q, hq, _ = q.shape
    dims = _dims_for(cache, hq, scale, int(cu_seqlens.shape[0]) - 1)
    _check(lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), _ptr(cu_seqlens), int(max_q_len),
                                  int(total_q), _ptr(out), _ptr(lse), _ptr(workspace), _nbytes(workspace),
                                  _stream(stream)), "yoco_xattn_prefill")
    return out


def xattn_prefill_window(cache: SharedKV, q: torch.Tensor, cu_seqlens: torch.Tensor, max_q_len: int, window: int,
                         scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         stream=None, workspace: Optional[torch.Tensor] = None):
    """Sliding-window prefill: row at position p attends rows max(0, p - window + 1) .. p."""
    lib = load_library()
    desc, out = _prefill_args(cache, q, cu_seqlens, out, lse, workspace)
    total_q, hq, _ = q.shape
    dims = _dims_for(cache, hq, scale, int(cu_seqlens.shape[0]) - 1)
    _check(lib.yoco_xattn_prefill_window(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), _ptr(cu_seqlens),
                                         int(max_q_len), int(total_q), int(window), _ptr(out), _ptr(lse),
                                         _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "yoco_xattn_prefill_window")
    return out


def workspace_size(batch: int, q_heads: int, kv_heads: int, head_dim: int, dtype: torch.dtype,
                   max_len: int, is_decode: bool = True) -> int:
    """Workspace bytes of a decode call (is_decode) or of a prefill call (its work queue)."""
    lib = load_library()
    dims = make_dims(batch, q_heads, kv_heads, head_dim, dtype, 1.0)
    n = ctypes.c_size_t(0)
    _check(lib.yoco_xattn_workspace_size(ctypes.byref(dims), int(max_len), int(bool(is_decode)), ctypes.byref(n)),
           "yoco_xattn_workspace_size")
    return int(n.value)


def alloc_prefill_workspace(device, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """A zeroed prefill work-queue workspace (reused as is: every call leaves it zero)."""
    n = workspace_size(1, 1, 1, 128, dtype, 1, is_decode=False)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def decode_splits(batch: int, q_heads: int, kv_heads: int, head_dim: int, dtype: torch.dtype, max_kv_len: int,
                  total_kv_len: int = 0):
    """(shares, rows per share) of the decode plan for these hints: every KV head
    (bf16; query head for fp32) cuts the 128-row blocks of all sequences into
    `shares` equal shares, one workgroup each."""
    lib = load_library()
    dims = make_dims(batch, q_heads, kv_heads, head_dim, dtype, 1.0)
    s, r = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.yoco_xattn_decode_splits(ctypes.byref(dims), int(max_kv_len), int(total_kv_len), ctypes.byref(s),
                                        ctypes.byref(r)),
           "yoco_xattn_decode_splits")
    return int(s.value), int(r.value)


def alloc_workspace(cache: SharedKV, q_heads: int, max_kv_len: int) -> torch.Tensor:
    n = workspace_size(int(cache.seq_len.shape[0]), q_heads, cache.k.shape[1], cache.k.shape[2], cache.k.dtype,
                       max_kv_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=cache.k.device)


def _decode_args(cache: SharedKV, q: torch.Tensor, out, lse, workspace=None, need_workspace=True):
    desc = cache.descriptor()
    _queries(cache, q)
    if int(q.shape[0]) != int(cache.seq_len.shape[0]):
        raise YocoError(YOCO_ERR_INVALID_ARG, f"q has {q.shape[0]} rows for {cache.seq_len.shape[0]} sequences")
    if need_workspace:
        _need(workspace, "workspace", torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _out_lse(q, out, lse, tuple(q.shape[:2]))
    return desc, out


def xattn_decode(cache: SharedKV, q: torch.Tensor, max_kv_len: int, scale: float, workspace: torch.Tensor,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None,
                 total_kv_len: int = 0):
    """One query per sequence (q [B, Hq, d]) against the whole shared cache; returns out.

    max_kv_len / total_kv_len are the host-side sizing hints of the split plan
    (the longest sequence's rows, all sequences' rows; 0 = B * max_kv_len); the
    kernels count the rows on the device, so wrong hints cost speed, not rows."""
    lib = load_library()
    desc, out = _decode_args(cache, q, out, lse, workspace)
    batch, hq, _ = q.shape
    dims = _dims_for(cache, hq, scale, batch)
    _check(lib.yoco_xattn_decode(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), int(max_kv_len), int(total_kv_len),
                                 _ptr(out),
                                 _ptr(lse), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                 _stream(stream)), "yoco_xattn_decode")
    return out


def xattn_decode_noalloc(cache: SharedKV, q: torch.Tensor, max_kv_len: int, scale: float,
                         out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None,
                         total_kv_len: int = 0):
    """xattn_decode whose partials live in the library's device-resident scratch
    (NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace: the call allocates
    nothing, so the caller passes `out`. Calls that may overlap on one GPU race."""
    lib = load_library()
    if out is None:
        raise YocoError(YOCO_ERR_INVALID_ARG, "out is missing (the no-allocation call allocates nothing)")
    desc, out = _decode_args(cache, q, out, lse, need_workspace=False)
    batch, hq, _ = q.shape
    dims = _dims_for(cache, hq, scale, batch)
    _check(lib.yoco_xattn_decode_noalloc(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), int(max_kv_len),
                                         int(total_kv_len), _ptr(out), _ptr(lse), _stream(stream)),
           "yoco_xattn_decode_noalloc")
    return out


def xattn_decode_window(cache: SharedKV, q: torch.Tensor, max_kv_len: int, window: int, scale: float,
                        workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None, total_kv_len: int = 0):
    """Decode over a full cache with a sliding window: the last min(seq_len, window) rows only."""
    lib = load_library()
    desc, out = _decode_args(cache, q, out, lse, workspace)
    batch, hq, _ = q.shape
    dims = _dims_for(cache, hq, scale, batch)
    _check(lib.yoco_xattn_decode_window(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), int(max_kv_len),
                                        int(total_kv_len), int(window), _ptr(out), _ptr(lse), _ptr(workspace),
                                        int(workspace.numel() * workspace.element_size()), _stream(stream)),
           "yoco_xattn_decode_window")
    return out


def kv_project_pack(gain: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, kv_heads: int, head_dim: int,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Packed projection weights (gain folded, [W_K | W_V] transposed): [2 * Hkv * d, d_model] bf16."""
    lib = load_library()
    if w_k is None or w_k.dim() != 2:
        raise YocoError(YOCO_ERR_INVALID_ARG, "w_k must be [d_model, Hkv * d]")
    d_model = int(w_k.shape[0])
    hd = kv_heads * head_dim
    dev = w_k.device
    _need(w_k, "w_k", torch.bfloat16, (d_model, hd), dev)
    _need(w_v, "w_v", torch.bfloat16, (d_model, hd), dev)
    _need(gain, "gain", torch.bfloat16, (d_model,), dev)
    if out is None:
        out = torch.empty(2 * hd, d_model, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (2 * hd, d_model), dev)
    dims = make_dims(1, kv_heads, kv_heads, head_dim, w_k.dtype, 1.0)
    _check(lib.yoco_kv_project_pack(ctypes.byref(dims), d_model, _ptr(gain), _ptr(w_k), _ptr(w_v), _ptr(out),
                                    _stream(stream)), "yoco_kv_project_pack")
    return out


def kv_project_append(cache: SharedKV, x: torch.Tensor, cu_seqlens: torch.Tensor, w_packed: torch.Tensor, eps: float,
                      residual: Optional[dict] = None, overflow: Optional[torch.Tensor] = None, stream=None) -> None:
    """RMSNorm(x) [W_K | W_V] appended to each sequence's rows (x [T, d_model], packed by cu_seqlens).

    residual (optional): {"k1", "v1" (device [T, Hkv*d]), "lam", "a_k": (a1, a2), "a_v": (a1, a2)}."""
    lib = load_library()
    batch = int(cu_seqlens.shape[0]) - 1
    dims = _dims_for(cache, cache.k.shape[1], 1.0, batch)
    desc = cache.descriptor()
    dev = cache.k.device
    if x is None or x.dim() != 2:
        raise YocoError(YOCO_ERR_INVALID_ARG, "x must be [T, d_model]")
    if batch != int(cache.seq_len.shape[0]):
        raise YocoError(YOCO_ERR_INVALID_ARG, "cu_seqlens must be [B + 1] with B the cache's sequences")
    t_rows, d_model = int(x.shape[0]), int(x.shape[1])
    hd = int(cache.k.shape[1]) * int(cache.k.shape[2])
    _need(x, "x", torch.bfloat16, device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
    _need(w_packed, "w_packed", torch.bfloat16, (2 * hd, d_model), dev)
    _flag(overflow, cache, "overflow")
    res = None
    if residual is not None:
        _need(residual["k1"], "residual k1", torch.bfloat16, (t_rows, hd), dev)
        _need(residual["v1"], "residual v1", torch.bfloat16, (t_rows, hd), dev)
        res = Residual(_ptr(residual["k1"]), _ptr(residual["v1"]), float(residual["lam"]),
                       (ctypes.c_float * 2)(*residual["a_k"]), (ctypes.c_float * 2)(*residual["a_v"]))
    _check(lib.yoco_kv_project_append(ctypes.byref(dims), ctypes.byref(desc), _ptr(x), _ptr(cu_seqlens),
                                      t_rows, d_model, _ptr(w_packed), float(eps),
                                      ctypes.byref(res) if res is not None else None, _ptr(overflow),
                                      _stream(stream)), "yoco_kv_project_append")


def gret_dims(batch: int, heads: int, head_dim: int, dtype: torch.dtype = torch.bfloat16) -> GretDims:
    if dtype not in DTYPE_CODE:
        raise YocoError(2, f"dtype {dtype}")
    return GretDims(batch, heads, head_dim, DTYPE_CODE[dtype])


def gret_workspace_size(batch: int, heads: int, head_dim: int, total_rows: int) -> int:
    """Workspace bytes of gret_prefill over total_rows packed rows of up to `batch` sequences."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.yoco_gret_workspace_size(ctypes.byref(gret_dims(batch, heads, head_dim)), int(total_rows),
                                        ctypes.byref(n)), "yoco_gret_workspace_size")
    return int(n.value)


def _gret_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor):
    if q is None or q.dim() != 3:
        raise YocoError(YOCO_ERR_INVALID_ARG, "q must be [T, H, d]")
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k, "k", torch.bfloat16, q.shape, dev)
    _need(v, "v", torch.bfloat16, q.shape, dev)
    _need(gamma, "gamma", torch.float32, tuple(q.shape[:2]), dev)
    return dev


def gret_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, cu_seqlens: torch.Tensor,
                 workspace: torch.Tensor, state_in: Optional[torch.Tensor] = None,
                 state_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None):
    """Gated retention over packed sequences (q, k, v [T, H, d] bf16, gamma [T, H] fp32); returns out."""
    lib = load_library()
    dev = _gret_qkv(q, k, v, gamma)
    total, heads, d = q.shape
    batch = int(cu_seqlens.shape[0]) - 1
    _need(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    st_shape = (batch, heads, d, d)
    _need(state_in, "state_in", torch.float32, st_shape, dev, optional=True)
    _need(state_out, "state_out", torch.float32, st_shape, dev, optional=True)
    if out is None:
        out = torch.empty_like(v)
    _need(out, "out", torch.bfloat16, q.shape, dev)
    dims = gret_dims(batch, heads, d, q.dtype)
    _check(lib.yoco_gret_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(cu_seqlens),
                                 int(total), _ptr(state_in), _ptr(state_out), _ptr(out),
                                 _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                 _stream(stream)), "yoco_gret_prefill")
    return out


def gret_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, state: torch.Tensor,
                out: Optional[torch.Tensor] = None, stream=None):
    """One recurrent gRet step (q, k, v [B, H, d], gamma [B, H]); updates state [B, H, d, d] in place."""
    lib = load_library()
    dev = _gret_qkv(q, k, v, gamma)
    batch, heads, d = q.shape
    _need(state, "state", torch.float32, (batch, heads, d, d), dev)
    if out is None:
        out = torch.empty_like(v)
    _need(out, "out", torch.bfloat16, q.shape, dev)
    dims = gret_dims(batch, heads, d, q.dtype)
    _check(lib.yoco_gret_decode(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(state), _ptr(out),
                                _stream(stream)), "yoco_gret_decode")
    return out
