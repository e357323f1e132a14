"""Thin ctypes binding of libyoco_xattn.so.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no fallback: if the library is missing, loading raises.

The functions mirror the C ABI (include/yoco_xattn.h) one to one:
``kv_append``, ``kv_append_ring``, ``xattn_prefill``, ``xattn_prefill_window``,
``xattn_decode``, ``xattn_decode_window``, ``workspace_size``, ``decode_splits``,
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
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip launch failed"}
DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1}

EXPORTS = ("yoco_kv_append", "yoco_kv_append_ring", "yoco_xattn_prefill", "yoco_xattn_prefill_window",
           "yoco_xattn_decode", "yoco_xattn_decode_window", "yoco_xattn_workspace_size",
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
    lib.yoco_xattn_prefill.argtypes = [dims_p, cache_p, P, P, i32, i64, P, P, P]
    lib.yoco_xattn_prefill_window.argtypes = [dims_p, cache_p, P, P, i32, i64, i32, P, P, P]
    lib.yoco_xattn_decode.argtypes = [dims_p, cache_p, P, i32, i64, P, P, P, ctypes.c_size_t, P]
    lib.yoco_xattn_decode_window.argtypes = [dims_p, cache_p, P, i32, i64, i32, P, P, P, ctypes.c_size_t, P]
    lib.yoco_kv_project_pack.argtypes = [dims_p, i32, P, P, P, P, P]
    lib.yoco_kv_project_append.argtypes = [dims_p, cache_p, P, P, i64, i32, P, ctypes.c_float,
                                           ctypes.POINTER(Residual), P, P]
    gdims_p = ctypes.POINTER(GretDims)
    lib.yoco_gret_workspace_size.argtypes = [gdims_p, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.yoco_gret_prefill.argtypes = [gdims_p, P, P, P, P, P, i64, i32, P, P, P, P, ctypes.c_size_t, P]
    lib.yoco_gret_decode.argtypes = [gdims_p, P, P, P, P, P, P, P]
    lib.yoco_xattn_workspace_size.argtypes = [dims_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.yoco_xattn_decode_splits.argtypes = [dims_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_int32)]
    lib.yoco_status_string.argtypes = [ctypes.c_int]
    lib.yoco_status_string.restype = ctypes.c_char_p
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


@dataclass
class SharedKV:
    """The one shared K^,V^ pool and its per-sequence metadata (all device tensors)."""
    k: torch.Tensor          # [pool_rows, Hkv, d]
    v: torch.Tensor
    seq_start: torch.Tensor  # int64 [B]
    seq_len: torch.Tensor    # int32 [B]
    seq_cap: torch.Tensor    # int32 [B]

    def descriptor(self) -> KvCache:
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


def kv_append(cache: SharedKV, k_new: torch.Tensor, v_new: torch.Tensor, overflow: Optional[torch.Tensor] = None,
              q_heads: Optional[int] = None, stream=None) -> None:
    """Append one row per sequence (k_new, v_new: [B, Hkv, d]); see yoco_kv_append."""
    lib = load_library()
    batch = int(cache.seq_len.shape[0])
    dims = _dims_for(cache, q_heads or cache.k.shape[1], 1.0, batch)
    desc = cache.descriptor()
    _check(lib.yoco_kv_append(ctypes.byref(dims), ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(overflow),
                              _stream(stream)), "yoco_kv_append")


def kv_append_ring(cache: SharedKV, k_new: torch.Tensor, v_new: torch.Tensor, flag: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Append one row per sequence to ring window caches (slot seq_len mod seq_cap); see yoco_kv_append_ring."""
    lib = load_library()
    batch = int(cache.seq_len.shape[0])
    dims = _dims_for(cache, cache.k.shape[1], 1.0, batch)
    desc = cache.descriptor()
    _check(lib.yoco_kv_append_ring(ctypes.byref(dims), ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(flag),
                                   _stream(stream)), "yoco_kv_append_ring")


def xattn_prefill(cache: SharedKV, q: torch.Tensor, cu_seqlens: torch.Tensor, max_q_len: int, scale: float,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """Causal prefill over packed queries q [total_q, Hq, d]; returns out (and fills lse [Hq, total_q])."""
    lib = load_library()
    total_q, hq, _ = q.shape
    batch = int(cu_seqlens.shape[0]) - 1
    if out is None:
        out = torch.empty_like(q)
    dims = _dims_for(cache, hq, scale, batch)
    desc = cache.descriptor()
    _check(lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), _ptr(cu_seqlens), int(max_q_len),
                                  int(total_q), _ptr(out), _ptr(lse), _stream(stream)), "yoco_xattn_prefill")
    return out


def xattn_prefill_window(cache: SharedKV, q: torch.Tensor, cu_seqlens: torch.Tensor, max_q_len: int, window: int,
                         scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         stream=None):
    """Sliding-window prefill: row at position p attends rows max(0, p - window + 1) .. p."""
    lib = load_library()
    total_q, hq, _ = q.shape
    batch = int(cu_seqlens.shape[0]) - 1
    if out is None:
        out = torch.empty_like(q)
    dims = _dims_for(cache, hq, scale, batch)
    desc = cache.descriptor()
    _check(lib.yoco_xattn_prefill_window(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), _ptr(cu_seqlens),
                                         int(max_q_len), int(total_q), int(window), _ptr(out), _ptr(lse),
                                         _stream(stream)), "yoco_xattn_prefill_window")
    return out


def workspace_size(batch: int, q_heads: int, kv_heads: int, head_dim: int, dtype: torch.dtype,
                   max_kv_len: int) -> int:
    lib = load_library()
    dims = make_dims(batch, q_heads, kv_heads, head_dim, dtype, 1.0)
    n = ctypes.c_size_t(0)
    _check(lib.yoco_xattn_workspace_size(ctypes.byref(dims), int(max_kv_len), ctypes.byref(n)),
           "yoco_xattn_workspace_size")
    return int(n.value)


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


def xattn_decode(cache: SharedKV, q: torch.Tensor, max_kv_len: int, scale: float, workspace: torch.Tensor,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None,
                 total_kv_len: int = 0):
    """One query per sequence (q [B, Hq, d]) against the whole shared cache; returns out.

    max_kv_len / total_kv_len are the host-side sizing hints of the split plan
    (the longest sequence's rows, all sequences' rows; 0 = B * max_kv_len); the
    kernels count the rows on the device, so wrong hints cost speed, not rows."""
    lib = load_library()
    batch, hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    dims = _dims_for(cache, hq, scale, batch)
    desc = cache.descriptor()
    _check(lib.yoco_xattn_decode(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), int(max_kv_len), int(total_kv_len),
                                 _ptr(out),
                                 _ptr(lse), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                 _stream(stream)), "yoco_xattn_decode")
    return out


def xattn_decode_window(cache: SharedKV, q: torch.Tensor, max_kv_len: int, window: int, scale: float,
                        workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None, total_kv_len: int = 0):
    """Decode over a full cache with a sliding window: the last min(seq_len, window) rows only."""
    lib = load_library()
    batch, hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    dims = _dims_for(cache, hq, scale, batch)
    desc = cache.descriptor()
    _check(lib.yoco_xattn_decode_window(ctypes.byref(dims), ctypes.byref(desc), _ptr(q), int(max_kv_len),
                                        int(total_kv_len), int(window), _ptr(out), _ptr(lse), _ptr(workspace),
                                        int(workspace.numel() * workspace.element_size()), _stream(stream)),
           "yoco_xattn_decode_window")
    return out


def kv_project_pack(gain: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, kv_heads: int, head_dim: int,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Packed projection weights (gain folded, [W_K | W_V] transposed): [2 * Hkv * d, d_model] bf16."""
    lib = load_library()
    d_model = int(w_k.shape[0])
    if out is None:
        out = torch.empty(2 * kv_heads * head_dim, d_model, dtype=torch.bfloat16, device=w_k.device)
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
    res = None
    if residual is not None:
        res = Residual(_ptr(residual["k1"]), _ptr(residual["v1"]), float(residual["lam"]),
                       (ctypes.c_float * 2)(*residual["a_k"]), (ctypes.c_float * 2)(*residual["a_v"]))
    _check(lib.yoco_kv_project_append(ctypes.byref(dims), ctypes.byref(desc), _ptr(x), _ptr(cu_seqlens),
                                      int(x.shape[0]), int(x.shape[1]), _ptr(w_packed), float(eps),
                                      ctypes.byref(res) if res is not None else None, _ptr(overflow),
                                      _stream(stream)), "yoco_kv_project_append")


def gret_dims(batch: int, heads: int, head_dim: int, dtype: torch.dtype = torch.bfloat16) -> GretDims:
    if dtype not in DTYPE_CODE:
        raise YocoError(2, f"dtype {dtype}")
    return GretDims(batch, heads, head_dim, DTYPE_CODE[dtype])


def gret_workspace_size(batch: int, heads: int, head_dim: int, max_len: int) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.yoco_gret_workspace_size(ctypes.byref(gret_dims(batch, heads, head_dim)), int(max_len),
                                        ctypes.byref(n)), "yoco_gret_workspace_size")
    return int(n.value)


def gret_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, cu_seqlens: torch.Tensor,
                 max_len: int, workspace: torch.Tensor, state_in: Optional[torch.Tensor] = None,
                 state_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None):
    """Gated retention over packed sequences (q, k, v [T, H, d] bf16, gamma [T, H] fp32); returns out."""
    lib = load_library()
    total, heads, d = q.shape
    batch = int(cu_seqlens.shape[0]) - 1
    if out is None:
        out = torch.empty_like(v)
    dims = gret_dims(batch, heads, d, q.dtype)
    _check(lib.yoco_gret_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(cu_seqlens),
                                 int(total), int(max_len), _ptr(state_in), _ptr(state_out), _ptr(out),
                                 _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                 _stream(stream)), "yoco_gret_prefill")
    return out


def gret_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, state: torch.Tensor,
                out: Optional[torch.Tensor] = None, stream=None):
    """One recurrent gRet step (q, k, v [B, H, d], gamma [B, H]); updates state [B, H, d, d] in place."""
    lib = load_library()
    batch, heads, d = q.shape
    if out is None:
        out = torch.empty_like(v)
    dims = gret_dims(batch, heads, d, q.dtype)
    _check(lib.yoco_gret_decode(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(state), _ptr(out),
                                _stream(stream)), "yoco_gret_decode")
    return out
