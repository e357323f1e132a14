"""Seeded tensors in the shared-cache pool layout.

Layout (shared by every consumer):

* ``k_pool``, ``v_pool``: ``[rows, Hkv, d]``, ``d`` contiguous; sequence ``b`` owns
  rows ``seq_start[b] .. seq_start[b] + seq_cap[b] - 1`` of the pool, of which the
  first ``seq_len[b]`` are valid. Capacity rows past ``seq_len`` hold finite junk
  drawn from the same distribution, so that a reader that strays past the valid
  rows changes the result.
* ``q`` (prefill): one ``[sum(L_b), Hq, d]`` tensor per layer, sequences packed
  back to back, ``cu_seqlens[b]`` = first packed row of sequence ``b``.
* decode queries: ``[steps, layers, B, Hq, d]``; appended rows ``[steps, B, Hkv, d]``.

Random streams: ``SeedSequence(seed).spawn(8)``; stream 0 draws K, 1 V, 2 the
prefill queries (layer after layer), 3 the appended K rows, 4 the appended V rows,
5 the decode queries, 7 the ragged lengths. Entries are ``standard_normal``
float32 times ``std`` (in float32), rounded once to the storage dtype by torch's
round-to-nearest-even conversion. Tensors are returned on the CPU.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(8)]


def _draw(rng, shape, std: float, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(_TORCH_DTYPE[dtype])


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of an fp32/bf16 CPU tensor to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16 (or fp32) CPU tensor to a float32 NumPy array."""
    return t.detach().to("cpu").to(torch.float32).numpy()


@dataclass
class PrefillCase:
    q: List[torch.Tensor]          # per layer [total_q, Hq, d]
    k_pool: torch.Tensor           # [rows, Hkv, d]
    v_pool: torch.Tensor
    seq_start: torch.Tensor        # int64 [B]
    seq_len: torch.Tensor          # int32 [B]
    seq_cap: torch.Tensor          # int32 [B]
    cu_seqlens: torch.Tensor       # int32 [B+1]
    scale: float
    dtype: str

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens[-1])


@dataclass
class DecodeCase:
    k_pool: torch.Tensor           # [rows, Hkv, d]; rows seq_len[b].. of each sequence are free capacity
    v_pool: torch.Tensor
    seq_start: torch.Tensor        # int64 [B]
    seq_len: torch.Tensor          # int32 [B], rows valid before the first append
    seq_cap: torch.Tensor          # int32 [B]
    k_new: torch.Tensor            # [steps, B, Hkv, d]
    v_new: torch.Tensor
    q: torch.Tensor                # [steps, layers, B, Hq, d]
    scale: float
    dtype: str


def _pool(rngs, lens: Sequence[int], caps: Sequence[int], kv_heads, head_dim, std, dtype, k_std=None, v_std=None):
    starts = np.zeros(len(lens), dtype=np.int64)
    if len(lens) > 1:
        starts[1:] = np.cumsum(np.asarray(caps[:-1], dtype=np.int64))
    rows = int(sum(caps))
    k = _draw(rngs[0], (rows, kv_heads, head_dim), std if k_std is None else k_std, dtype)
    v = _draw(rngs[1], (rows, kv_heads, head_dim), std if v_std is None else v_std, dtype)
    return (k, v, torch.from_numpy(starts), torch.tensor(list(lens), dtype=torch.int32),
            torch.tensor(list(caps), dtype=torch.int32))


def make_prefill_case(lens: Sequence[int], q_heads: int, kv_heads: int, head_dim: int, layers: int,
                      dtype: str, seed: int, std: float, scale: Optional[float] = None,
                      cap_extra: int = 0, q_std: Optional[float] = None, k_std: Optional[float] = None,
                      v_std: Optional[float] = None) -> PrefillCase:
    rngs = _streams(seed)
    caps = [int(n) + cap_extra for n in lens]
    k, v, start, seq_len, cap = _pool(rngs, lens, caps, kv_heads, head_dim, std, dtype, k_std, v_std)
    total_q = int(sum(lens))
    qs = [_draw(rngs[2], (total_q, q_heads, head_dim), std if q_std is None else q_std, dtype)
          for _ in range(layers)]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return PrefillCase(qs, k, v, start, seq_len, cap, torch.from_numpy(cu),
                       float(scale if scale is not None else head_dim ** -0.5), dtype)


def make_chunk_case(kv_lens: Sequence[int], q_lens: Sequence[int], q_heads: int, kv_heads: int, head_dim: int,
                    dtype: str, seed: int, std: float, scale: Optional[float] = None,
                    cap_extra: int = 0) -> PrefillCase:
    """Cache rows kv_lens[b] per sequence and q_lens[b] query rows (a chunk of new
    tokens after the cached ones), packed like a prefill."""
    rngs = _streams(seed)
    caps = [int(n) + cap_extra for n in kv_lens]
    k, v, start, seq_len, cap = _pool(rngs, kv_lens, caps, kv_heads, head_dim, std, dtype)
    total_q = int(sum(q_lens))
    q = _draw(rngs[2], (total_q, q_heads, head_dim), std, dtype)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    return PrefillCase([q], k, v, start, seq_len, cap, torch.from_numpy(cu),
                       float(scale if scale is not None else head_dim ** -0.5), dtype)


def make_decode_case(lens: Sequence[int], q_heads: int, kv_heads: int, head_dim: int, layers: int,
                     steps: int, dtype: str, seed: int, std: float, scale: Optional[float] = None,
                     cap_extra: int = 0, q_std: Optional[float] = None, k_std: Optional[float] = None,
                     v_std: Optional[float] = None) -> DecodeCase:
    rngs = _streams(seed)
    caps = [int(n) + steps + cap_extra for n in lens]
    k, v, start, seq_len, cap = _pool(rngs, lens, caps, kv_heads, head_dim, std, dtype, k_std, v_std)
    b = len(lens)
    k_new = _draw(rngs[3], (steps, b, kv_heads, head_dim), std if k_std is None else k_std, dtype)
    v_new = _draw(rngs[4], (steps, b, kv_heads, head_dim), std if v_std is None else v_std, dtype)
    q = _draw(rngs[5], (steps, layers, b, q_heads, head_dim), std if q_std is None else q_std, dtype)
    return DecodeCase(k, v, start, seq_len, cap, k_new, v_new, q,
                      float(scale if scale is not None else head_dim ** -0.5), dtype)
