"""fp64 CPU oracle of YOCO's Cross-Decoder attention over the one shared K̂,V̂.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module; only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` do. It shares no code with the HIP kernels.

What it computes is the plain definition, written out step by step:

* Every Cross-Decoder layer l attends with its own queries Q̂^l to the single
  shared pair K̂, V̂ that the Self-Decoder output produced once
  ("YOCO", zdszero.github.io: section "架构总览" (architecture overview),
  the equations for K̂, V̂ and Q̂^l, and section "Cross-Decoder：共享 KV，但不共享
  Query", the Attn_l equation)::

      Attn_l = softmax(Q̂^l K̂^T / sqrt(d_k) + M_causal) V̂

* M_causal lets the query at position i see shared-cache rows j no later than i,
  i.e. j <= i (same page, end of "架构总览").
* Grouped-query attention: several query heads read one KV head ("YOCO 深度技术分析",
  liuhc.cn: section 2.1 (architecture), Cross-Decoder bullet list; the shared KV
  may itself use fewer KV heads: "YOCO", section "与其他 KV 优化方法的区别").
* Decode: the new token passes the Self-Decoder first, so its own K̂,V̂ row is in
  the cache before the Cross-Decoder layers read it ("YOCO", section "Decode：
  新 token 仍需经过两部分").
* Sliding-window attention, the Self-Decoder's efficient attention: the current
  position sees only the tokens of a fixed window of size C, so one layer's
  decode cache holds O(C) rows instead of O(N) ("YOCO", section "Self-Decoder：
  把历史编码成可复用的全局表示"; "YOCO 深度技术分析", section 2.3, C = 1024).
  The same attention with the band mask instead of the causal mask; a decode
  window cache is a ring of C rows.

Readings where the pages are silent (each is listed in the design notes):

* d_k is the head dimension; the scale is passed explicitly.
* The query head h reads KV head h // (Hq / Hkv) (contiguous groups).
* The mask is inclusive (j <= i) and exact (masked rows carry zero weight).
* Prefill queries and keys index the same positions; a chunk of m new query
  rows after n cached rows (m <= n) sits at the last m positions; a decode
  query sits at position seq_len - 1 after its row was appended. With more
  query rows than cache rows (m > n) the queries start at position 0 and those
  at positions n and later, whose own row is not in the cache, get the empty
  result (O = 0, LSE = -inf).
* No positional transform inside the cross-attention.
* LSE is the natural-log log-sum-exp of the scaled scores; an empty sequence
  yields O = 0 and LSE = -inf.
* A window of size C holds the C most recent positions, the query's own
  included: position p sees rows max(0, p - C + 1) .. p. Window 0 means no
  window (plain causal). A ring window cache keeps token t in slot t mod C, so
  its valid slots are exactly the last min(t + 1, C) tokens, in rotated order;
  softmax attention does not depend on the order of its keys.

All arithmetic is float64 on exact upcasts of the stored values. Query rows are
processed in blocks only to bound memory: each row's arithmetic is the
definition above, independently of every other row.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "kv_head_of",
    "visible_rows",
    "window_start",
    "prefill_position",
    "has_own_row",
    "decode_position",
    "scores",
    "softmax_weights",
    "log_sum_exp",
    "attend_rows",
    "prefill_ref",
    "decode_ref",
    "kv_append_ref",
    "ring_append_ref",
]


# ---------------------------------------------------------------------------
# The definition's steps, one small function each.
# ---------------------------------------------------------------------------

def kv_head_of(h: int, q_heads: int, kv_heads: int) -> int:
    """KV head read by query head h: contiguous groups of Hq/Hkv query heads."""
    return h // (q_heads // kv_heads)


def visible_rows(p: int) -> int:
    """Number of shared-cache rows the query at position p sees: rows 0..p."""
    return p + 1


def window_start(p: int, window: int) -> int:
    """First row the query at position p sees under a window of `window` positions (0: none)."""
    return max(0, p - window + 1) if window > 0 else 0


def prefill_position(r: int, n_q: int, n_kv: int) -> int:
    """Position of query row r when a sequence has n_q query rows and n_kv cache rows.

    The queries are the last n_q positions of the sequence (a full prompt when
    n_q == n_kv; a chunk of new tokens after the cached ones otherwise); with
    more queries than rows they start at position 0.
    """
    return r + max(n_kv - n_q, 0)


def has_own_row(p: int, n_kv: int) -> bool:
    """Whether the token at position p has its K̂,V̂ row among the n_kv cache rows.

    A token's row is written before any Cross-Decoder layer reads the cache
    ("YOCO", section "Decode：新 token 仍需经过两部分"), so a query whose own row
    is not there has no defined attention. Such a row gets the result of an
    empty key set: O = 0 and LSE = -inf (the convention for a sequence with no
    rows).
    """
    return p < n_kv


def decode_position(n: int) -> int:
    """Position of the decode query once its own row is appended: the last of n valid rows."""
    return n - 1


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s[r, j] = scale * <q[r], k[j]>  (q: [r, d], k: [n, d])."""
    return scale * (q @ k.T)


def softmax_weights(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row-wise softmax pieces of s (masked entries are -inf).

    Returns (w, m, z): m = max_j s_j, w_j = exp(s_j - m), z = sum_j w_j, so that
    softmax(s)_j = w_j / z and log-sum-exp(s) = m + log z.
    """
    m = np.max(s, axis=-1, keepdims=True)
    w = np.exp(s - m)
    z = np.sum(w, axis=-1, keepdims=True)
    return w, m, z


def log_sum_exp(m: np.ndarray, z: np.ndarray) -> np.ndarray:
    """log sum_j exp(s_j) from the softmax pieces: m + log z."""
    return m + np.log(z)


def attend_rows(q: np.ndarray, positions: np.ndarray, k: np.ndarray, v: np.ndarray,
                scale: float, window: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Causal attention of query rows q [r, d] at `positions` [r] to rows k, v [n, d].

    Row i of the result is sum_j softmax_j(scale q_i.k_j, j <= p_i) v_j and its LSE;
    with a window, only rows window_start(p_i, window) <= j take part.
    """
    q = np.asarray(q, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    r = q.shape[0]
    out = np.zeros((r, v.shape[1]), dtype=np.float64)
    lse = np.full((r,), -np.inf, dtype=np.float64)
    if r == 0:
        return out, lse
    n_vis = max(visible_rows(int(p)) for p in positions)
    kk = np.asarray(k[:n_vis], dtype=np.float64)
    vv = np.asarray(v[:n_vis], dtype=np.float64)
    s = scores(q, kk, scale)
    j = np.arange(n_vis)[None, :]
    lim = np.array([visible_rows(int(p)) for p in positions])[:, None]
    first = np.array([window_start(int(p), window) for p in positions])[:, None]
    s = np.where((j < lim) & (j >= first), s, -np.inf)
    w, m, z = softmax_weights(s)
    out = (w @ vv) / z
    lse = log_sum_exp(m, z)[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# The three operations of the path, on the pool layout.
# ---------------------------------------------------------------------------

def prefill_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, seq_start: Sequence[int],
                seq_len: Sequence[int], cu_seqlens: Sequence[int], scale: float,
                rows: Optional[Dict[int, Iterable[int]]] = None, block: int = 512,
                window: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Causal cross-attention of every packed query row to its sequence's shared rows.

    q: [total_q, Hq, d]; k_pool, v_pool: [rows, Hkv, d]. Query row r of sequence b
    (packed row cu_seqlens[b] + r) sits at position prefill_position(r, m, n) (m
    query rows, n = seq_len[b] cache rows: r itself for a full prompt) and sees
    cache rows seq_start[b] + 0 .. seq_start[b] + that position; a row whose
    position has no cache row of its own (has_own_row) gets O = 0, LSE = -inf.
    `rows` (optional) restricts the work to {b: [r, ...]}; rows not computed are NaN.
    `window` > 0 restricts each query to the rows of its window (sliding-window
    attention). Returns out [total_q, Hq, d] and lse [Hq, total_q] (float64).
    """
    total_q, hq, d = q.shape
    hkv = k_pool.shape[1]
    out = np.full((total_q, hq, d), np.nan if rows is not None else 0.0, dtype=np.float64)
    lse = np.full((hq, total_q), np.nan if rows is not None else -np.inf, dtype=np.float64)
    nseq = len(seq_len)
    for b in range(nseq):
        n = int(seq_len[b])
        q0 = int(cu_seqlens[b])
        m = int(cu_seqlens[b + 1]) - q0
        want = np.arange(m) if rows is None else np.asarray(sorted(set(rows.get(b, ()))), dtype=np.int64)
        if want.size == 0 or n == 0:
            continue
        s0 = int(seq_start[b])
        for h in range(hq):
            kh = kv_head_of(h, hq, hkv)
            kb = k_pool[s0:s0 + n, kh, :]
            vb = v_pool[s0:s0 + n, kh, :]
            pos_all = np.array([prefill_position(int(x), m, n) for x in want], dtype=np.int64)
            own = np.array([has_own_row(int(p), n) for p in pos_all], dtype=bool)
            out[q0 + want[~own], h, :] = 0.0
            lse[h, q0 + want[~own]] = -np.inf
            want_own, pos_own = want[own], pos_all[own]
            for i in range(0, want_own.size, block):
                r = want_own[i:i + block]
                o, l = attend_rows(q[q0 + r, h, :], pos_own[i:i + block], kb, vb, scale, window)
                out[q0 + r, h, :] = o
                lse[h, q0 + r] = l
    return out, lse


def decode_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, seq_start: Sequence[int],
               seq_len: Sequence[int], scale: float, window: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """One query per sequence at position seq_len[b] - 1, against rows 0..seq_len[b]-1
    (only the last `window` of them when window > 0).

    q: [B, Hq, d]. Returns out [B, Hq, d] and lse [B, Hq] (float64). A sequence with
    no rows gives out = 0 and lse = -inf.
    """
    bsz, hq, d = q.shape
    hkv = k_pool.shape[1]
    out = np.zeros((bsz, hq, d), dtype=np.float64)
    lse = np.full((bsz, hq), -np.inf, dtype=np.float64)
    for b in range(bsz):
        n = int(seq_len[b])
        if n == 0:
            continue
        s0 = int(seq_start[b])
        for kh in range(hkv):
            kb = np.asarray(k_pool[s0:s0 + n, kh, :], dtype=np.float64)
            vb = np.asarray(v_pool[s0:s0 + n, kh, :], dtype=np.float64)
            for h in range(hq):
                if kv_head_of(h, hq, hkv) != kh:
                    continue
                o, l = attend_rows(q[b, h:h + 1, :], np.array([decode_position(n)]), kb, vb, scale, window)
                out[b, h] = o[0]
                lse[b, h] = l[0]
    return out, lse


def kv_append_ref(k_pool: np.ndarray, v_pool: np.ndarray, seq_start: Sequence[int],
                  seq_len: Sequence[int], seq_cap: Sequence[int], k_new: np.ndarray,
                  v_new: np.ndarray):
    """Write each sequence's new K̂,V̂ row at its next free row; one more valid row.

    A sequence whose cache is full keeps its pool rows and length and raises the
    overflow flag. Returns (k_pool', v_pool', seq_len', overflow) as new arrays.
    """
    k2 = np.array(k_pool, copy=True)
    v2 = np.array(v_pool, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    overflow = 0
    for b in range(len(lens)):
        if lens[b] >= int(seq_cap[b]):
            overflow = 1
            continue
        row = int(seq_start[b]) + int(lens[b])
        k2[row] = k_new[b]
        v2[row] = v_new[b]
        lens[b] += 1
    return k2, v2, lens, overflow


def ring_append_ref(k_ring: np.ndarray, v_ring: np.ndarray, seq_start: Sequence[int],
                    seq_len: Sequence[int], seq_cap: Sequence[int], k_new: np.ndarray,
                    v_new: np.ndarray):
    """Append to ring window caches: sequence b's token number seq_len[b] goes to
    slot seq_len[b] mod seq_cap[b] of its seq_cap[b] rows, replacing the token
    seq_cap[b] positions older; seq_len[b] counts every token appended so far.

    A sequence with no rows (seq_cap 0) stores nothing and raises the flag.
    Returns (k_ring', v_ring', seq_len', flag) as new arrays.
    """
    k2 = np.array(k_ring, copy=True)
    v2 = np.array(v_ring, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    flag = 0
    for b in range(len(lens)):
        cap = int(seq_cap[b])
        if cap <= 0:
            flag = 1
            continue
        row = int(seq_start[b]) + int(lens[b]) % cap
        k2[row] = k_new[b]
        v2[row] = v_new[b]
        lens[b] += 1
    return k2, v2, lens, flag
