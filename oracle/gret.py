"""fp64 CPU oracle of gated retention (gRet), YOCO's default Self-Decoder
attention.

TEST INFRASTRUCTURE ONLY (see oracle/xattn.py): only the tests, the smoke check
and the benchmark's CPU leg use it; it shares no code with the HIP kernels.

What it computes ("YOCO 深度技术分析", liuhc.cn, section 2.2, the three
equivalent forms; section 5.3.2, chunk size 256; the xingfushuangcheng.com
translation, section "门控保留率" and its recurrent and chunkwise parts;
"YOCO", section "Self-Decoder：把历史编码成可复用的全局表示", S_t and y_t):

* parallel form: gRet = (Q K^T ⊙ D) V with the data-controlled decay
  D[n, m] = γ_{m+1} γ_{m+2} ... γ_n for m <= n and 0 for m > n;
* recurrent form: S_n = γ_n S_{n-1} + K_n^T V_n, o_n = Q_n S_n;
* chunkwise form: inside a chunk the parallel form, across chunks the state
  recurrence (chunk size B = 256 on the pages).

Q, K (already multiplied by the caller's Θ), V and γ (one decay per token and
head, the head-wise gate γ = sigmoid(X W_γ)^(1/τ)) are inputs. Readings where the
pages are silent (listed in the design notes): the decay product for n = m is
empty (1), so a token sees its own K^T V undecayed, which is what makes the
parallel and recurrent forms agree; an optional initial state S_0 enters the
recurrence as S_{-1}, i.e. o_n gains Q_n (γ_0 ... γ_n) S_0; no scale and no
normalisation inside (the per-head GroupNorm and the swish gate lie outside).
All arithmetic is float64 on exact upcasts of the stored values.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["gret_decay_matrix", "gret_parallel_ref", "gret_recurrent_ref", "gret_chunkwise_ref",
           "gret_prefill_ref", "gret_decode_ref", "GRET_CHUNK"]

GRET_CHUNK = 256   # the pages' chunk size


def gret_decay_matrix(gamma: np.ndarray) -> np.ndarray:
    """D[n, m] = prod_{i = m+1}^{n} gamma[i] for m <= n, else 0 (gamma: [N])."""
    g = np.asarray(gamma, dtype=np.float64)
    n = g.shape[0]
    d = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        d[i, i] = 1.0
        for j in range(i - 1, -1, -1):
            d[i, j] = d[i, j + 1] * g[j + 1]
    return d


def gret_parallel_ref(q, k, v, gamma, s0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One head: o = (q k^T ⊙ D) v (+ (prefix decay * q) s0), and the state after the last row.

    q, k: [N, dk]; v: [N, dv]; gamma: [N]; s0: [dk, dv] or None. Returns (o [N, dv], s_N [dk, dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    n = q.shape[0]
    d = gret_decay_matrix(g)
    o = ((q @ k.T) * d) @ v
    prefix = np.cumprod(g) if n else np.zeros(0)          # gamma_0 ... gamma_n
    if s0 is None:
        s_n = np.zeros((k.shape[1], v.shape[1]))
    else:
        s0 = np.asarray(s0, dtype=np.float64)
        o = o + (prefix[:, None] * q) @ s0
        s_n = (prefix[-1] if n else 1.0) * s0
    if n:
        s_n = s_n + (d[n - 1][:, None] * k).T @ v
    return o, s_n


def gret_recurrent_ref(q, k, v, gamma, s0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One head, token by token: S_n = gamma_n S_{n-1} + k_n^T v_n, o_n = q_n S_n."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = np.zeros((k.shape[1], v.shape[1])) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        s = float(gamma[t]) * s + np.outer(k[t], v[t])
        o[t] = q[t] @ s
    return o, s


def gret_chunkwise_ref(q, k, v, gamma, s0: Optional[np.ndarray] = None,
                       chunk: int = GRET_CHUNK) -> Tuple[np.ndarray, np.ndarray]:
    """One head in the chunkwise form: per chunk, the parallel form inside it plus
    the carried state decayed to each row, then the state passed on."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    s = np.zeros((k.shape[1], v.shape[1])) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    for c0 in range(0, q.shape[0], chunk):
        c1 = min(c0 + chunk, q.shape[0])
        qc, kc, vc, gc = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1]
        d = gret_decay_matrix(gc)                 # decay inside the chunk
        into = np.cumprod(gc)                     # decay from the chunk's start to each row, inclusive
        o[c0:c1] = ((qc @ kc.T) * d) @ vc + (into[:, None] * qc) @ s
        out_of = d[-1]                            # decay from each row to the chunk's end
        s = into[-1] * s + (out_of[:, None] * kc).T @ vc
    return o, s


def gret_prefill_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, gamma: np.ndarray, cu_seqlens: Sequence[int],
                     s0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Packed sequences (rows cu[b] .. cu[b+1]-1), every head: q, k [T, H, dk]; v [T, H, dv];
    gamma [T, H]; s0 [B, H, dk, dv] or None. Returns out [T, H, dv] and the final
    states [B, H, dk, dv] (the parallel form)."""
    total, h, dk = q.shape
    dv = v.shape[2]
    nb = len(cu_seqlens) - 1
    out = np.zeros((total, h, dv))
    st = np.zeros((nb, h, dk, dv))
    for b in range(nb):
        r0, r1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for hh in range(h):
            o, s = gret_parallel_ref(q[r0:r1, hh], k[r0:r1, hh], v[r0:r1, hh], gamma[r0:r1, hh],
                                     None if s0 is None else s0[b, hh])
            out[r0:r1, hh] = o
            st[b, hh] = s
    return out, st


def gret_decode_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, gamma: np.ndarray,
                    state: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One token per sequence (q, k [B, H, dk]; v [B, H, dv]; gamma [B, H]) on the
    states [B, H, dk, dv]: the recurrent form's step. Returns (out [B, H, dv], new states)."""
    nb, h, _ = q.shape
    out = np.zeros((nb, h, v.shape[2]))
    st = np.array(state, dtype=np.float64, copy=True)
    for b in range(nb):
        for hh in range(h):
            o, s = gret_recurrent_ref(q[b, hh][None], k[b, hh][None], v[b, hh][None], gamma[b, hh:hh + 1],
                                      state[b, hh])
            out[b, hh] = o[0]
            st[b, hh] = s
    return out, st
