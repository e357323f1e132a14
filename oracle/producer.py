"""fp64 CPU oracle of the shared-cache producer: K̂, V̂ rows from the last
Self-Decoder output, written into the one shared cache.

TEST INFRASTRUCTURE ONLY (see oracle/xattn.py): only the tests, the smoke check
and the benchmark's CPU leg use it; it shares no code with the HIP kernels.

The definition, written out:

* The Self-Decoder output X^{L/2} is normalised and projected once into the
  global pair K̂ = LN(X^{L/2}) W_K, V̂ = LN(X^{L/2}) W_V ("YOCO",
  zdszero.github.io, section "架构总览", the K̂, V̂ equations).
* LN is RMSNorm (xingfushuangcheng.com explainer of YOCO, section "自解码器",
  the sentence after the Self-Decoder equations).
* YOCO++ caches, instead of the middle layer's K, V alone, a weighted sum with
  the bottom layer's: K' = λ(α₁ K₁ + α₂ K), V' = λ(α₁ᵛ V₁ + α₂ᵛ V), λ = 35,
  initialised to α₁ = 0, α₂ = 1/λ so that the start equals YOCO; the sum is
  formed at prefill and cached, so decode reads no more than YOCO
  (gist.science explainer of YOCO++ (2604.13556), sections 2.1 and 2.2).
* The rows join each sequence's part of the shared cache after its valid rows,
  like the per-token append ("YOCO", section "Decode：新 token 仍需经过两部分").

Readings where the pages are silent (listed in the design notes): RMSNorm is
x / sqrt(mean(x²) + eps) times a per-feature gain γ, eps passed explicitly; W_K
and W_V are [d_model, Hkv·d] (K̂ rows are [Hkv, d], the cache layout); a chunk
of T_b rows that does not fit into sequence b's capacity is not written at all
and raises the overflow flag.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["rmsnorm_ref", "kv_project_ref", "kv_combine_ref", "project_append_ref", "YOCOPP_LAMBDA"]

YOCOPP_LAMBDA = 35.0   # the pages' fixed scaling factor


def rmsnorm_ref(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma (float64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def kv_combine_ref(k_mid: np.ndarray, k_bottom: np.ndarray, a1: float, a2: float, lam: float) -> np.ndarray:
    """YOCO++ residual: lam * (a1 * bottom-layer rows + a2 * middle-layer rows)."""
    return lam * (a1 * np.asarray(k_bottom, dtype=np.float64) + a2 * np.asarray(k_mid, dtype=np.float64))


def kv_project_ref(x: np.ndarray, gamma: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, eps: float,
                   combine: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """K̂, V̂ = RMSNorm(x) W_K, RMSNorm(x) W_V for rows x [T, d_model]; [T, Hkv*d] each.

    combine (optional): {"k1", "v1" ([T, Hkv*d] bottom-layer rows), "ak": (a1, a2),
    "av": (a1, a2), "lam"} applies the YOCO++ residual to both.
    """
    y = rmsnorm_ref(x, gamma, eps)
    k = y @ np.asarray(w_k, dtype=np.float64)
    v = y @ np.asarray(w_v, dtype=np.float64)
    if combine is not None:
        lam = combine.get("lam", YOCOPP_LAMBDA)
        k = kv_combine_ref(k, combine["k1"], combine["ak"][0], combine["ak"][1], lam)
        v = kv_combine_ref(v, combine["v1"], combine["av"][0], combine["av"][1], lam)
    return k, v


def project_append_ref(k_pool: np.ndarray, v_pool: np.ndarray, seq_start: Sequence[int], seq_len: Sequence[int],
                       seq_cap: Sequence[int], cu_seqlens: Sequence[int], x: np.ndarray, gamma: np.ndarray,
                       w_k: np.ndarray, w_v: np.ndarray, eps: float, combine: Optional[dict] = None):
    """Project packed rows x [T, d_model] (sequence b: rows cu[b]..cu[b+1]-1) and
    append them to each sequence's rows of the pools [rows, Hkv, d].

    Sequence b's i-th row lands at pool row seq_start[b] + seq_len[b] + i; then
    seq_len[b] grows by its row count. A sequence whose rows do not all fit into
    seq_cap[b] keeps everything and raises the flag. Returns (k', v', seq_len', flag).
    """
    hkv, d = k_pool.shape[1], k_pool.shape[2]
    k, v = kv_project_ref(x, gamma, w_k, w_v, eps, combine)
    k2 = np.array(k_pool, dtype=np.float64, copy=True)
    v2 = np.array(v_pool, dtype=np.float64, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    flag = 0
    for b in range(len(lens)):
        r0, r1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        t = r1 - r0
        if lens[b] + t > int(seq_cap[b]):
            flag = 1
            continue
        base = int(seq_start[b]) + int(lens[b])
        k2[base:base + t] = k[r0:r1].reshape(t, hkv, d)
        v2[base:base + t] = v[r0:r1].reshape(t, hkv, d)
        lens[b] += t
    return k2, v2, lens, flag
