"""Planted needles for discriminating decode parity at long contexts.

At 128K-1M rows with the acceptance inputs (entries N(0,1)/sqrt(d)) the logits
are nearly flat, the output is an average of ~10^5 rows of size ~1e-3, and an
all-zero output passes the max-abs bound. A needle is a K^ row that the
checked query heads all score highly: for the g query heads q_h of one KV
group (the rows of Q_g) the least-norm solution k of
    scale * Q_g k = t            (t_h = the wanted logits)
gives each head the logit t_h, far above the background (~0), and the needle's
V^ row is an independent N(0,1) row. With many needles of nearly equal logits
the output is a mixture of their V^ rows of size ~0.1-1: every needle carries
a share of the result, so an output that misses any group of rows holding a
needle, reads the wrong KV head or the wrong rows, or ignores Q or K^, is far
off in row-relative terms.

Needles are spaced `stride` rows apart and dealt round-robin to the C checked
queries (needle i belongs to query i mod C), so each query has a needle every
C * stride rows; the last row of each sequence's prompt and the row of position
0 are needles too. This module builds inputs only; every expected value comes
from the oracle.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np
import torch


def solve_needle(qg: np.ndarray, logits: np.ndarray, scale: float) -> np.ndarray:
    """Least-norm k with scale * qg @ k = logits (qg: [g, d] float64)."""
    gram = qg @ qg.T
    return qg.T @ np.linalg.solve(gram, np.asarray(logits, dtype=np.float64) / scale)


def needle_rows(n: int, stride: int) -> List[int]:
    """Rows holding needles in a sequence of n prompt rows: 0, stride, 2 stride, ... and n - 1."""
    rows = list(range(0, n, stride))
    if n > 0 and rows[-1] != n - 1:
        rows.append(n - 1)
    return rows


def plant(k_pool: torch.Tensor, v_pool: torch.Tensor, seq_start: Sequence[int], seq_len: Sequence[int],
          queries: Sequence[torch.Tensor], scale: float, stride: int, seed: int, logit: float = 20.0,
          spread: float = 1.0) -> int:
    """Write needles into k_pool / v_pool ([rows, Hkv, d], in place, any float dtype).

    queries: the C checked decode queries, each [B, Hq, d]. Needle i of
    sequence b, KV head kh belongs to query i mod C: its logit for every head
    of the group is logit + spread * u (u ~ U[0,1), one per needle), and its
    V^ row is N(0,1). Returns the number of needles per (sequence, KV head).
    """
    rng = np.random.default_rng(seed)
    hkv, d = int(k_pool.shape[1]), int(k_pool.shape[2])
    qs = [q.to(torch.float64).numpy() for q in queries]
    hq = qs[0].shape[1]
    g = hq // hkv
    count = 0
    for b in range(len(seq_len)):
        rows = needle_rows(int(seq_len[b]), stride)
        count = max(count, len(rows))
        s0 = int(seq_start[b])
        for kh in range(hkv):
            ks = np.empty((len(rows), d))
            for i, _ in enumerate(rows):
                qg = qs[i % len(qs)][b, kh * g:(kh + 1) * g, :]
                t = logit + spread * rng.random()
                ks[i] = solve_needle(qg, np.full(g, t), scale)
            vs = rng.standard_normal((len(rows), d))
            idx = torch.tensor([s0 + r for r in rows], dtype=torch.long)
            k_pool[idx, kh, :] = torch.from_numpy(ks).to(k_pool.dtype)
            v_pool[idx, kh, :] = torch.from_numpy(vs).to(v_pool.dtype)
    return count


def aligned_rows(query: torch.Tensor, kv_heads: int, scale: float, seed: int, dtype: torch.dtype,
                 logit: float = 20.0):
    """Appended K^,V^ rows [B, Hkv, d] that are needles of `query` ([B, Hq, d])."""
    rng = np.random.default_rng(seed)
    q = query.to(torch.float64).numpy()
    b, hq, d = q.shape
    g = hq // kv_heads
    k = np.empty((b, kv_heads, d))
    for s in range(b):
        for kh in range(kv_heads):
            k[s, kh] = solve_needle(q[s, kh * g:(kh + 1) * g], np.full(g, logit + rng.random()), scale)
    v = rng.standard_normal((b, kv_heads, d))
    return torch.from_numpy(k).to(dtype), torch.from_numpy(v).to(dtype)


def share_rows(lens: Sequence[int], shares: int, block: int = 128):
    """Row ranges of each share of the balanced decode split: the blocks of all
    sequences, in order, cut into `shares` equal parts (share w starts at block
    floor(w * total / shares)). Returns, per share, a list of (sequence, first
    row, end row)."""
    blocks = [(n + block - 1) // block for n in lens]
    total = sum(blocks)
    parts = min(shares, total)
    out = []
    for w in range(parts):
        first, last = (w * total) // parts, ((w + 1) * total) // parts
        pieces, pre = [], 0
        for b, u in enumerate(blocks):
            lo, hi = max(first, pre), min(last, pre + u)
            if lo < hi:
                pieces.append((b, (lo - pre) * block, min((hi - pre) * block, int(lens[b]))))
            pre += u
        out.append(pieces)
    return out


# Needle spacing per full-size decode workload, chosen so that every share of
# the decode split holds at least two needles of each checked query (checked
# on the CPU against the split plan by tests/test_checker_needles.py).
STRIDE = {"decode_128k": 1024, "decode_1m": 512, "ragged": 512}
