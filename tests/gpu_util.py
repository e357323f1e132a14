"""Helpers for the GPU parity tests: move seeded cases to the device, run the
library through its binding, bring results back as float64 NumPy arrays."""
from __future__ import annotations

import numpy as np
import torch

import decoder_shared_kv_amd as dk
import synth

DEV = torch.device("cuda:0")


def device_cache(k_pool, v_pool, seq_start, seq_len, seq_cap) -> dk.SharedKV:
    return dk.SharedKV(k_pool.to(DEV).contiguous(), v_pool.to(DEV).contiguous(), seq_start.to(DEV),
                       seq_len.to(DEV).clone(), seq_cap.to(DEV))


_QUEUE = {}


def prefill_workspace() -> torch.Tensor:
    """One zeroed work-queue workspace per process, reused by every prefill call
    (each completed call leaves it zero); tests check that it stays zero."""
    if "ws" not in _QUEUE:
        _QUEUE["ws"] = dk.alloc_prefill_workspace(DEV)
    return _QUEUE["ws"]


def run_prefill(case: synth.PrefillCase, layer: int = 0, cache: dk.SharedKV = None, with_lse: bool = True,
                queue: bool = True, max_q: int = None):
    """Prefill through the library: with the work queue (the launch configuration
    the benchmark times) unless queue=False (the static grid)."""
    if cache is None:
        cache = device_cache(case.k_pool, case.v_pool, case.seq_start, case.seq_len, case.seq_cap)
    q = case.q[layer].to(DEV)
    hq = q.shape[1]
    lse = torch.full((hq, case.total_q), float("nan"), device=DEV) if with_lse else None
    if max_q is None:
        max_q = int((case.cu_seqlens[1:] - case.cu_seqlens[:-1]).max()) if case.cu_seqlens.numel() > 1 else 0
    ws = prefill_workspace() if queue else None
    out = dk.xattn_prefill(cache, q, case.cu_seqlens.to(DEV), max_q, case.scale, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return f64(out), (lse.cpu().numpy().astype(np.float64) if with_lse else None)


def run_decode(cache: dk.SharedKV, q: torch.Tensor, scale: float, max_kv_len: int = None, with_lse: bool = True,
               total_kv_len: int = None):
    """Decode through the library; the split-plan hints default to the true
    longest and total row counts (pass total_kv_len=0 for the B x max plan)."""
    q = q.to(DEV).contiguous()
    if max_kv_len is None:
        max_kv_len = int(cache.seq_len.max().item())
    if total_kv_len is None:
        total_kv_len = int(cache.seq_len.sum().item())
    ws = dk.alloc_workspace(cache, q.shape[1], max_kv_len)
    lse = torch.full(q.shape[:2], float("nan"), device=DEV) if with_lse else None
    out = dk.xattn_decode(cache, q, max_kv_len, scale, ws, lse=lse, total_kv_len=total_kv_len)
    torch.cuda.synchronize()
    return f64(out), (lse.cpu().numpy().astype(np.float64) if with_lse else None)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def say(msg: str) -> None:
    print(msg, flush=True)
