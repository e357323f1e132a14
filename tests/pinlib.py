"""Pins of the fp64 oracle to things other than itself.

Each ``check_*`` function raises AssertionError (or any exception) when the
oracle disagrees with what the pages and the mathematics fix. They are plain
functions so that the mutation tests can run them against an oracle with a
planted mistake and require that at least one of them fails.

What pins what:

* brute force: pure-Python scalar loops (math.exp / math.fsum, no max
  subtraction) on tiny shapes -- the definition of causal softmax attention
  with contiguous GQA groups, written independently of NumPy;
* torch's scaled_dot_product_attention in float64 on the CPU with
  is_causal=True and enable_gqa=True -- a library routine for the square
  (queries = keys) causal GQA case;
* closed forms: K = 0 gives the prefix mean of V and LSE = log(p + 1); V = c
  gives c; one row gives V[0]; a planted needle gives that row; a hand-worked
  two-key case from tests/golden/;
* invariants: decode at p equals prefill row p; rows past p do not matter;
  shifting every key by u leaves O and moves LSE by scale*q.u; GQA equals MHA
  with repeated KV heads; packed sequences equal separate calls; (cQ, s/c)
  equals (Q, s); softmax weights sum to 1;
* append: the new row lands at seq_start + seq_len, overflow leaves all alone.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle.gret as og
import oracle.producer as op
import oracle.xattn as ox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _pool_case(rng, lens, hq, hkv, d, junk=3):
    """Packed queries + pool with `junk` finite capacity rows after each sequence."""
    caps = [n + junk for n in lens]
    starts = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(sum(caps))
    k = rng.standard_normal((rows, hkv, d))
    v = rng.standard_normal((rows, hkv, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((int(cu[-1]), hq, d))
    return q, k, v, starts, np.asarray(lens, dtype=np.int64), cu


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def _brute_prefill(q, k, v, starts, lens, cu, scale):
    total, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(total)]
    lse = [[0.0] * total for _ in range(hq)]
    for b in range(len(lens)):
        for r in range(int(lens[b])):
            row = int(cu[b]) + r
            for h in range(hq):
                kh = h // g
                e = []
                for j in range(r + 1):
                    key = k[int(starts[b]) + j, kh]
                    dot = math.fsum(float(q[row, h, t]) * float(key[t]) for t in range(d))
                    e.append(math.exp(scale * dot))
                z = math.fsum(e)
                for t in range(d):
                    out[row][h][t] = math.fsum(e[j] * float(v[int(starts[b]) + j, kh, t])
                                               for j in range(r + 1)) / z
                lse[h][row] = math.log(z)
    return np.array(out), np.array(lse)


def check_bruteforce():
    rng = _rng(11)
    for lens, hq, hkv, d, scale in [((5,), 2, 1, 3, 0.7), ((4, 7), 4, 2, 4, 0.5), ((9,), 4, 1, 8, 0.35),
                                    ((1, 3, 6), 2, 2, 2, 1.3), ((12,), 8, 2, 5, 0.45)]:
        q, k, v, st, ln, cu = _pool_case(rng, lens, hq, hkv, d)
        o, l = ox.prefill_ref(q, k, v, st, ln, cu, scale)
        ob, lb = _brute_prefill(q, k, v, st, ln, cu, scale)
        assert np.max(np.abs(o - ob)) <= 1e-13, ("brute force out", lens, np.max(np.abs(o - ob)))
        assert np.max(np.abs(l - lb)) <= 1e-13, ("brute force lse", lens)
        # decode of the last row of each sequence = brute-force row
        qd = np.stack([q[int(cu[b + 1]) - 1] for b in range(len(lens))])
        od, ld = ox.decode_ref(qd, k, v, st, ln, scale)
        for b in range(len(lens)):
            row = int(cu[b + 1]) - 1
            assert np.max(np.abs(od[b] - ob[row])) <= 1e-13, ("brute force decode", lens, b)
            assert np.max(np.abs(ld[b] - lb[:, row])) <= 1e-13


# ---------------------------------------------------------------------------
# library special case
# ---------------------------------------------------------------------------

def check_sdpa():
    import torch.nn.functional as F
    rng = _rng(12)
    for n, hq, hkv, d in [(33, 4, 1, 16), (70, 8, 2, 32), (130, 6, 3, 8), (64, 4, 4, 64)]:
        q, k, v, st, ln, cu = _pool_case(rng, (n,), hq, hkv, d, junk=0)
        scale = 1.0 / math.sqrt(d)
        o, _ = ox.prefill_ref(q, k, v, st, ln, cu, scale)
        tq = torch.from_numpy(q).permute(1, 0, 2)[None]
        tk = torch.from_numpy(k).permute(1, 0, 2)[None]
        tv = torch.from_numpy(v).permute(1, 0, 2)[None]
        ts = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True, scale=scale)
        ref = ts[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(o - ref)) <= 1e-12, ("sdpa", n, hq, hkv, np.max(np.abs(o - ref)))


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def check_closed_forms():
    rng = _rng(13)
    n, hq, hkv, d = 40, 4, 2, 6
    q, k, v, st, ln, cu = _pool_case(rng, (n,), hq, hkv, d, junk=2)
    # K = 0 (inside the sequence): every visible row weighs the same
    kz = k.copy()
    kz[:n] = 0.0
    o, l = ox.prefill_ref(q, kz, v, st, ln, cu, 0.9)
    for h in range(hq):
        kh = h // (hq // hkv)
        prefix_mean = np.cumsum(v[:n, kh], axis=0) / np.arange(1, n + 1)[:, None]
        assert np.max(np.abs(o[:, h] - prefix_mean)) <= 1e-13, "K=0 prefix mean"
        assert np.max(np.abs(l[h] - np.log(np.arange(1, n + 1)))) <= 1e-13, "K=0 lse"
    # Q = 0 likewise
    o, _ = ox.prefill_ref(np.zeros_like(q), k, v, st, ln, cu, 0.9)
    for h in range(hq):
        kh = h // (hq // hkv)
        prefix_mean = np.cumsum(v[:n, kh], axis=0) / np.arange(1, n + 1)[:, None]
        assert np.max(np.abs(o[:, h] - prefix_mean)) <= 1e-13, "Q=0 prefix mean"
    # V = c per KV head: the weights sum to one
    c = rng.standard_normal((hkv, d))
    vc = v.copy()
    vc[:n] = c[None]
    o, _ = ox.prefill_ref(q, k, vc, st, ln, cu, 0.9)
    for h in range(hq):
        assert np.max(np.abs(o[:, h] - c[h // (hq // hkv)][None])) <= 1e-13, "V=c"
    # single row: O = V[0], LSE = scale q.k0
    q1, k1, v1, st1, ln1, cu1 = _pool_case(rng, (1,), 4, 1, 5, junk=4)
    o, l = ox.prefill_ref(q1, k1, v1, st1, ln1, cu1, 0.6)
    assert np.max(np.abs(o[0] - v1[0, 0][None])) <= 1e-15
    assert np.max(np.abs(l[:, 0] - 0.6 * (q1[0] @ k1[0, 0]))) <= 1e-13
    # planted needle: row 17 aligned with the query, far above all others
    n2, d2 = 64, 16
    q2, k2, v2, st2, ln2, cu2 = _pool_case(rng, (n2,), 1, 1, d2, junk=1)
    k2 *= 0.01
    qn = q2[n2 - 1, 0] / np.linalg.norm(q2[n2 - 1, 0])
    k2[17, 0] = 60.0 * qn
    od, _ = ox.decode_ref(q2[n2 - 1][None] / np.linalg.norm(q2[n2 - 1, 0]), k2, v2, st2, ln2, 1.0)
    assert np.max(np.abs(od[0, 0] - v2[17, 0])) <= 1e-20 + 64 * math.exp(-55) * np.max(np.abs(v2)), "needle"
    # hand-worked fixtures
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        qh = np.array(cs["q"], dtype=np.float64)
        kh_ = np.array(cs["k"], dtype=np.float64)
        vh = np.array(cs["v"], dtype=np.float64)
        nn = kh_.shape[0]
        o, l = ox.prefill_ref(qh, kh_, vh, [0], [nn], [0, nn], cs["scale"])
        exp_o = np.array(cs["expected_out"], dtype=np.float64)
        exp_l = np.array(cs["expected_lse"], dtype=np.float64)
        assert np.max(np.abs(o - exp_o)) <= 1e-14, ("hand case", cs["name"], o, exp_o)
        assert np.max(np.abs(l - exp_l)) <= 1e-14, ("hand case lse", cs["name"], l, exp_l)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def check_invariants():
    rng = _rng(14)
    lens = (23, 9, 31)
    hq, hkv, d = 6, 2, 8
    q, k, v, st, ln, cu = _pool_case(rng, lens, hq, hkv, d, junk=4)
    scale = 0.4
    o, l = ox.prefill_ref(q, k, v, st, ln, cu, scale)
    # decode at p = prefill row p, for every p of every sequence
    for b, n in enumerate(lens):
        for p in range(n):
            lens_p = np.array(ln)
            lens_p[b] = p + 1
            qd = np.zeros((len(lens), hq, d))
            qd[b] = q[int(cu[b]) + p]
            od, ld = ox.decode_ref(qd, k, v, st, lens_p, scale)
            assert np.max(np.abs(od[b] - o[int(cu[b]) + p])) <= 1e-14, ("decode = prefill row", b, p)
            assert np.max(np.abs(ld[b] - l[:, int(cu[b]) + p])) <= 1e-14
    # causal-mask invariance: rows past p, perturbed with finite values, change nothing
    b, p = 2, 12
    k2, v2 = k.copy(), v.copy()
    s0 = int(st[b])
    k2[s0 + p + 1:s0 + lens[b] + 4] += 5.0 * rng.standard_normal(k2[s0 + p + 1:s0 + lens[b] + 4].shape)
    v2[s0 + p + 1:s0 + lens[b] + 4] -= 7.0
    o2, l2 = ox.prefill_ref(q, k2, v2, st, ln, cu, scale)
    rows = slice(int(cu[b]), int(cu[b]) + p + 1)
    assert np.array_equal(o2[rows], o[rows]) and np.array_equal(l2[:, rows], l[:, rows]), "causal invariance"
    assert np.max(np.abs(o2[int(cu[b]) + p + 1:int(cu[b + 1])] - o[int(cu[b]) + p + 1:int(cu[b + 1])])) > 1e-3
    # shift of every key by u: O unchanged, LSE moves by scale * q.u
    u = rng.standard_normal((hkv, d))
    o3, l3 = ox.prefill_ref(q, k + u[None], v, st, ln, cu, scale)
    assert np.max(np.abs(o3 - o)) <= 1e-12, "key shift leaves O"
    g = hq // hkv
    for h in range(hq):
        shift = scale * (q[:, h, :] @ u[h // g])
        assert np.max(np.abs(l3[h] - l[h] - shift)) <= 1e-12, "key shift moves LSE"
    # GQA = MHA on repeated KV heads
    kr = np.repeat(k, g, axis=1)
    vr = np.repeat(v, g, axis=1)
    o4, l4 = ox.prefill_ref(q, kr, vr, st, ln, cu, scale)
    assert np.max(np.abs(o4 - o)) <= 1e-14 and np.max(np.abs(l4 - l)) <= 1e-14, "GQA = MHA repeat"
    # packed sequences = separate calls
    for b, n in enumerate(lens):
        s0 = int(st[b])
        ob, lb = ox.prefill_ref(q[int(cu[b]):int(cu[b + 1])], k[s0:s0 + n], v[s0:s0 + n], [0], [n], [0, n], scale)
        assert np.max(np.abs(ob - o[int(cu[b]):int(cu[b + 1])])) <= 1e-14, "varlen = separate"
        assert np.max(np.abs(lb - l[:, int(cu[b]):int(cu[b + 1])])) <= 1e-14
    # (c Q, scale / c) = (Q, scale)
    o5, l5 = ox.prefill_ref(4.0 * q, k, v, st, ln, cu, scale / 4.0)
    assert np.max(np.abs(o5 - o)) <= 1e-12 and np.max(np.abs(l5 - l)) <= 1e-12, "scale covariance"
    # softmax weights of any masked score row sum to one
    s = rng.standard_normal((5, 9))
    s[:, 6:] = -np.inf
    w, m, z = ox.softmax_weights(s)
    assert np.max(np.abs((w / z).sum(axis=1) - 1.0)) <= 1e-15 and np.all(w[:, 6:] == 0.0)
    # empty decode sequence: O = 0, LSE = -inf
    od, ld = ox.decode_ref(np.ones((1, 2, 3)), np.ones((4, 1, 3)), np.ones((4, 1, 3)), [0], [0], 1.0)
    assert np.all(od == 0.0) and np.all(np.isneginf(ld))


def _chunk_case(rng, lens, chunks, hq, hkv, d, junk=2):
    """Cache rows lens[b]; the last chunks[b] positions of each sequence get queries."""
    caps = [n + junk for n in lens]
    starts = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    k = rng.standard_normal((int(sum(caps)), hkv, d))
    v = rng.standard_normal((int(sum(caps)), hkv, d))
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = rng.standard_normal((int(cu[-1]), hq, d))
    return q, k, v, starts, np.asarray(lens, dtype=np.int64), cu


def check_chunked_prefill():
    """A chunk of m queries after n - m cached rows: bottom-right causal alignment.

    Pinned by (i) the full prefill of a prompt whose last m query rows are the
    chunk's (rows before the chunk do not matter to the chunk), (ii) decode for
    m = 1, (iii) torch SDPA in fp64 with an explicit lower-right causal mask."""
    import torch.nn.functional as F
    rng = _rng(16)
    lens, chunks = (40, 17, 33), (9, 1, 33)
    hq, hkv, d = 4, 2, 8
    q, k, v, st, ln, cu = _chunk_case(rng, lens, chunks, hq, hkv, d)
    o, l = ox.prefill_ref(q, k, v, st, ln, cu, 0.45)
    for b, (n, m) in enumerate(zip(lens, chunks)):
        # (i) full-prompt prefill with random earlier rows and this chunk as the last rows
        qf = rng.standard_normal((n, hq, d))
        qf[n - m:] = q[cu[b]:cu[b + 1]]
        s0 = int(st[b])
        of, lf = ox.prefill_ref(qf, k[s0:s0 + n], v[s0:s0 + n], [0], [n], [0, n], 0.45)
        assert np.max(np.abs(of[n - m:] - o[cu[b]:cu[b + 1]])) <= 1e-14, ("chunk = last rows of prefill", b)
        assert np.max(np.abs(lf[:, n - m:] - l[:, cu[b]:cu[b + 1]])) <= 1e-14
        # (iii) SDPA with a lower-right aligned causal mask
        mask = np.arange(n)[None, :] <= (np.arange(m)[:, None] + n - m)
        tq = torch.from_numpy(np.ascontiguousarray(q[cu[b]:cu[b + 1]])).permute(1, 0, 2)[None]
        tk = torch.from_numpy(np.ascontiguousarray(k[s0:s0 + n])).permute(1, 0, 2)[None]
        tv = torch.from_numpy(np.ascontiguousarray(v[s0:s0 + n])).permute(1, 0, 2)[None]
        ts = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), enable_gqa=True, scale=0.45)
        assert np.max(np.abs(ts[0].permute(1, 0, 2).numpy() - o[cu[b]:cu[b + 1]])) <= 1e-12, ("chunk vs sdpa", b)
    # more query rows than cache rows (m > n): the queries start at position 0;
    # the first n rows are the prompt's prefill, and a row at position n or later
    # has no K^,V^ row of its own in the cache (a token's row is written before
    # any Cross-Decoder layer reads: "YOCO", section "Decode：新 token 仍需经过两部分"),
    # so it gets the empty key set's result, O = 0 and LSE = -inf
    q2, k2, v2, st2, ln2, cu2 = _chunk_case(rng, (5,), (8,), 2, 1, 4)
    o2, l2 = ox.prefill_ref(q2, k2, v2, st2, ln2, cu2, 0.7)
    o2f, l2f = ox.prefill_ref(q2[:5], k2, v2, st2, ln2, np.array([0, 5]), 0.7)
    assert np.max(np.abs(o2[:5] - o2f)) <= 1e-14 and np.max(np.abs(l2[:, :5] - l2f)) <= 1e-14
    assert np.all(o2[5:] == 0.0) and np.all(np.isneginf(l2[:, 5:])), "rows without their own cache row"
    # the same rows requested one by one
    o3, l3 = ox.prefill_ref(q2, k2, v2, st2, ln2, cu2, 0.7, rows={0: [4, 5, 7]})
    assert np.max(np.abs(o3[[4, 5, 7]] - o2[[4, 5, 7]])) <= 1e-14
    assert np.array_equal(np.isneginf(l3[:, [4, 5, 7]]), np.isneginf(l2[:, [4, 5, 7]]))
    assert np.max(np.abs(l3[:, 4] - l2[:, 4])) <= 1e-14
    # (ii) one-row chunk = decode
    od, ld = ox.decode_ref(q[cu[1]:cu[2]], k, v, st[1:2], ln[1:2], 0.45)
    assert np.max(np.abs(od[0] - o[cu[1]])) <= 1e-14 and np.max(np.abs(ld[0] - l[:, cu[1]])) <= 1e-14


def check_append():
    rng = _rng(15)
    k = rng.standard_normal((24, 2, 4))
    v = rng.standard_normal((24, 2, 4))
    st, ln, cap = [0, 8, 14], [3, 6, 6], [8, 6, 8]
    kn = rng.standard_normal((3, 2, 4))
    vn = rng.standard_normal((3, 2, 4))
    k2, v2, ln2, ov = ox.kv_append_ref(k, v, st, ln, cap, kn, vn)
    assert list(ln2) == [4, 6, 7] and ov == 1, (list(ln2), ov)
    assert np.array_equal(k2[3], kn[0]) and np.array_equal(v2[3], vn[0])
    assert np.array_equal(k2[20], kn[2]) and np.array_equal(v2[20], vn[2])
    changed = [i for i in range(24) if not np.array_equal(k2[i], k[i]) or not np.array_equal(v2[i], v[i])]
    assert changed == [3, 20], changed
    _, _, ln3, ov3 = ox.kv_append_ref(k, v, [0], [2], [3], kn[:1], vn[:1])
    assert list(ln3) == [3] and ov3 == 0


# ---------------------------------------------------------------------------
# sliding window and ring window cache
# ---------------------------------------------------------------------------

def _brute_window_row(q_row, k, v, p, window, scale):
    """Pure-Python attention of one query at position p to rows max(0, p-C+1)..p."""
    lo = max(0, p - window + 1)
    e = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q_row, k[j]))) for j in range(lo, p + 1)]
    z = math.fsum(e)
    out = [math.fsum(e[j - lo] * float(v[j][t]) for j in range(lo, p + 1)) / z for t in range(len(v[0]))]
    return np.array(out), math.log(z)


def check_window():
    """Sliding-window attention: position p sees rows max(0, p - C + 1) .. p.

    Pinned by pure-Python loops, torch SDPA in fp64 with an explicit band mask,
    the closed forms C = 1 (O = V[p], LSE = the own score) and K = 0 (moving
    average of the last C rows, LSE = log of their count), C >= N equal to no
    window, invariance to rows before the window, decode = prefill's last row,
    and a chunk of queries = the last rows of the full windowed prefill."""
    import torch.nn.functional as F
    rng = _rng(17)
    # brute force, several windows, GQA 2:1 and packed sequences
    q, k, v, st, ln, cu = _pool_case(rng, (11, 6), 4, 2, 3, junk=2)
    for window in (1, 2, 4, 7):
        o, l = ox.prefill_ref(q, k, v, st, ln, cu, 0.8, window=window)
        for b in range(2):
            for r in range(int(ln[b])):
                for h in range(4):
                    s0 = int(st[b])
                    ob, lb = _brute_window_row(q[int(cu[b]) + r, h], k[s0:s0 + int(ln[b]), h // 2],
                                               v[s0:s0 + int(ln[b]), h // 2], r, window, 0.8)
                    assert np.max(np.abs(o[int(cu[b]) + r, h] - ob)) <= 1e-13, ("window brute", window, b, r)
                    assert abs(l[h, int(cu[b]) + r] - lb) <= 1e-13
    # SDPA with a band mask
    for n, hq, hkv, d, window in [(50, 4, 1, 8, 9), (130, 6, 3, 16, 64), (70, 2, 2, 4, 1)]:
        q, k, v, st, ln, cu = _pool_case(rng, (n,), hq, hkv, d, junk=0)
        o, _ = ox.prefill_ref(q, k, v, st, ln, cu, 0.3, window=window)
        i, j = np.arange(n)[:, None], np.arange(n)[None, :]
        band = torch.from_numpy((j <= i) & (j > i - window))
        tq = torch.from_numpy(q).permute(1, 0, 2)[None]
        tk = torch.from_numpy(k).permute(1, 0, 2)[None]
        tv = torch.from_numpy(v).permute(1, 0, 2)[None]
        ts = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, enable_gqa=True, scale=0.3)
        assert np.max(np.abs(ts[0].permute(1, 0, 2).numpy() - o)) <= 1e-12, ("window vs sdpa", n, window)
    # closed forms
    n, hq, hkv, d = 30, 2, 1, 5
    q, k, v, st, ln, cu = _pool_case(rng, (n,), hq, hkv, d, junk=3)
    o, l = ox.prefill_ref(q, k, v, st, ln, cu, 0.7, window=1)
    for h in range(hq):
        assert np.max(np.abs(o[:, h] - v[:n, 0])) <= 1e-15, "window 1: own row"
        assert np.max(np.abs(l[h] - 0.7 * np.einsum("rd,rd->r", q[:, h], k[:n, 0]))) <= 1e-13
    kz = k.copy()
    kz[:n] = 0.0
    for window in (3, 8):
        o, l = ox.prefill_ref(q, kz, v, st, ln, cu, 0.7, window=window)
        c = np.concatenate([np.zeros((1, d)), np.cumsum(v[:n, 0], axis=0)])
        for p in range(n):
            lo = max(0, p - window + 1)
            avg = (c[p + 1] - c[lo]) / (p + 1 - lo)
            assert np.max(np.abs(o[p, :] - avg[None])) <= 1e-13, ("K=0 moving average", window, p)
            assert np.max(np.abs(l[:, p] - math.log(p + 1 - lo))) <= 1e-13
    # window covering the whole sequence = no window
    o0, l0 = ox.prefill_ref(q, k, v, st, ln, cu, 0.7)
    ow, lw = ox.prefill_ref(q, k, v, st, ln, cu, 0.7, window=n)
    assert np.array_equal(o0, ow) and np.array_equal(l0, lw)
    # rows before the window of row p do not matter to rows p.. (they do to the rows before p)
    p, window = 20, 6
    k2, v2 = k.copy(), v.copy()
    k2[:p - window + 1] += 3.0
    v2[:p - window + 1] -= 5.0
    o2, l2 = ox.prefill_ref(q, k2, v2, st, ln, cu, 0.7, window=window)
    ow, lw = ox.prefill_ref(q, k, v, st, ln, cu, 0.7, window=window)
    assert np.array_equal(o2[p:], ow[p:]) and np.array_equal(l2[:, p:], lw[:, p:]), "rows before the window"
    assert np.max(np.abs(o2[p - 1] - ow[p - 1])) > 1e-3
    # decode with a window = the windowed prefill's row p
    for p in (0, 4, 5, 29):
        od, ld = ox.decode_ref(q[p:p + 1], k, v, st, [p + 1], 0.7, window=window)
        assert np.max(np.abs(od[0] - ow[p])) <= 1e-14 and np.max(np.abs(ld[0] - lw[:, p])) <= 1e-14
    # a chunk of the last m positions = the last rows of the full windowed prefill
    m = 7
    qc = q[n - m:]
    oc, lc = ox.prefill_ref(qc, k, v, st, ln, np.array([0, m]), 0.7, window=window)
    assert np.max(np.abs(oc - ow[n - m:])) <= 1e-14 and np.max(np.abs(lc - lw[:, n - m:])) <= 1e-14


def check_ring():
    """Ring window cache: after every append, attention over the ring's valid
    slots equals windowed decode over the whole history; slots hold token t at
    t mod C (hand-checked layout)."""
    rng = _rng(18)
    hkv, d, hq, window, steps = 2, 4, 4, 5, 13
    hist_k = rng.standard_normal((steps, 2, hkv, d))   # [t, b, Hkv, d]
    hist_v = rng.standard_normal((steps, 2, hkv, d))
    caps = [window, window]
    starts = [0, window + 3]
    ring_k = rng.standard_normal((2 * window + 3, hkv, d))   # junk before the first appends
    ring_v = rng.standard_normal((2 * window + 3, hkv, d))
    lens = np.array([0, 0])
    for t in range(steps):
        ring_k, ring_v, lens, flag = ox.ring_append_ref(ring_k, ring_v, starts, lens, caps, hist_k[t], hist_v[t])
        assert flag == 0 and list(lens) == [t + 1, t + 1]
        qd = rng.standard_normal((2, hq, d))
        valid = [min(int(x), c) for x, c in zip(lens, caps)]
        o_ring, l_ring = ox.decode_ref(qd, ring_k, ring_v, starts, valid, 0.6)
        lin_k = np.concatenate([hist_k[:t + 1, 0], hist_k[:t + 1, 1]])
        lin_v = np.concatenate([hist_v[:t + 1, 0], hist_v[:t + 1, 1]])
        o_lin, l_lin = ox.decode_ref(qd, lin_k, lin_v, [0, t + 1], [t + 1, t + 1], 0.6, window=window)
        assert np.max(np.abs(o_ring - o_lin)) <= 1e-13 and np.max(np.abs(l_ring - l_lin)) <= 1e-13, ("ring", t)
    # 13 tokens into 5 slots: slot s holds the latest t with t mod 5 = s
    for slot, tok in enumerate([10, 11, 12, 8, 9]):
        assert np.array_equal(ring_k[slot], hist_k[tok, 0]) and np.array_equal(ring_v[starts[1] + slot], hist_v[tok, 1])
    # a sequence without rows stores nothing and raises the flag
    k3, v3, l3, f3 = ox.ring_append_ref(ring_k, ring_v, [0, 5], [3, 0], [5, 0], hist_k[0], hist_v[0])
    assert f3 == 1 and list(l3) == [4, 0] and np.array_equal(k3[5:], ring_k[5:])


# ---------------------------------------------------------------------------
# the producer: RMSNorm, projection, YOCO++ combine, append into the cache
# ---------------------------------------------------------------------------

def check_rmsnorm():
    """RMSNorm against torch's rms_norm in float64, a constant row, scale
    invariance (eps = 0), the row mean of (y / gamma)^2 = 1 (eps = 0), and a
    hand-worked row."""
    import torch.nn.functional as F
    rng = _rng(19)
    x = rng.standard_normal((7, 48)) * 3.0
    g = rng.standard_normal(48)
    for eps in (1e-6, 0.5):
        y = op.rmsnorm_ref(x, g, eps)
        ref = F.rms_norm(torch.from_numpy(x), (48,), weight=torch.from_numpy(g), eps=eps).numpy()
        assert np.max(np.abs(y - ref)) <= 1e-13, ("rms_norm", eps)
    y1 = op.rmsnorm_ref(np.full((1, 5), -2.0), np.arange(1.0, 6.0), 0.0)
    assert np.max(np.abs(y1 - (-np.arange(1.0, 6.0)))) <= 1e-15, "constant row"
    y0 = op.rmsnorm_ref(x, g, 0.0)
    assert np.max(np.abs(op.rmsnorm_ref(5.5 * x, g, 0.0) - y0)) <= 1e-13, "scale invariance"
    assert np.max(np.abs(np.mean((y0 / g) ** 2, axis=1) - 1.0)) <= 1e-13
    # [3, 4], gain [1, 2], eps 0: rms = sqrt(12.5) -> [3, 8] / sqrt(12.5)
    yh = op.rmsnorm_ref(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    assert np.max(np.abs(yh - np.array([[3.0, 8.0]]) / math.sqrt(12.5))) <= 1e-15


def _brute_project(x, g, wk, wv, eps):
    out_k, out_v = [], []
    for row in x:
        ms = math.fsum(float(a) * float(a) for a in row) / len(row)
        y = [float(a) / math.sqrt(ms + eps) * float(gg) for a, gg in zip(row, g)]
        out_k.append([math.fsum(y[i] * float(wk[i, j]) for i in range(len(y))) for j in range(wk.shape[1])])
        out_v.append([math.fsum(y[i] * float(wv[i, j]) for i in range(len(y))) for j in range(wv.shape[1])])
    return np.array(out_k), np.array(out_v)


def check_project():
    """K̂ = RMSNorm(x) W_K, V̂ = RMSNorm(x) W_V: pure-Python loops on tiny shapes,
    identity weights (K̂ = the normalised row), K and V not swapped."""
    rng = _rng(20)
    x = rng.standard_normal((5, 12))
    g = rng.standard_normal(12)
    wk = rng.standard_normal((12, 8))
    wv = rng.standard_normal((12, 8))
    k, v = op.kv_project_ref(x, g, wk, wv, 1e-5)
    kb, vb = _brute_project(x, g, wk, wv, 1e-5)
    assert np.max(np.abs(k - kb)) <= 1e-13 and np.max(np.abs(v - vb)) <= 1e-13, "projection brute force"
    k, v = op.kv_project_ref(x, g, np.eye(12), 2.0 * np.eye(12), 0.0)
    y = op.rmsnorm_ref(x, g, 0.0)
    assert np.max(np.abs(k - y)) <= 1e-15 and np.max(np.abs(v - 2.0 * y)) <= 1e-15, "identity weights"


def check_combine():
    """YOCO++ residual: the pages' initialisation (a1 = 0, a2 = 1/lambda) gives
    YOCO's rows; (1/lambda, 0) gives the bottom layer's rows; lambda = 35; a
    hand-worked value."""
    rng = _rng(21)
    x = rng.standard_normal((6, 16))
    g = rng.standard_normal(16)
    wk, wv = rng.standard_normal((16, 8)), rng.standard_normal((16, 8))
    k1, v1 = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    lam = op.YOCOPP_LAMBDA
    assert lam == 35.0
    k, v = op.kv_project_ref(x, g, wk, wv, 1e-6)
    init = {"k1": k1, "v1": v1, "ak": (0.0, 1.0 / lam), "av": (0.0, 1.0 / lam), "lam": lam}
    ki, vi = op.kv_project_ref(x, g, wk, wv, 1e-6, init)
    assert np.max(np.abs(ki - k)) <= 1e-13 * np.max(np.abs(k)) and np.max(np.abs(vi - v)) <= 1e-13 * np.max(np.abs(v))
    bottom = {"k1": k1, "v1": v1, "ak": (1.0 / lam, 0.0), "av": (1.0 / lam, 0.0), "lam": lam}
    kb, vb = op.kv_project_ref(x, g, wk, wv, 1e-6, bottom)
    assert np.max(np.abs(kb - k1)) <= 1e-14 and np.max(np.abs(vb - v1)) <= 1e-14
    mixed = {"k1": k1, "v1": v1, "ak": (0.01, 0.02), "av": (0.03, -0.01), "lam": lam}
    km, vm = op.kv_project_ref(x, g, wk, wv, 1e-6, mixed)
    assert np.max(np.abs(km - 35.0 * (0.01 * k1 + 0.02 * k))) <= 1e-13
    assert np.max(np.abs(vm - 35.0 * (0.03 * v1 - 0.01 * v))) <= 1e-13
    assert abs(op.kv_combine_ref(np.array(2.0), np.array(4.0), 0.1, 0.2, 35.0) - 35.0 * (0.4 + 0.4)) <= 1e-13


def check_project_append():
    """Projected rows land after each sequence's valid rows; a chunk that does
    not fit changes nothing of its sequence and raises the flag; decode-style
    single rows are plain appends."""
    rng = _rng(22)
    hkv, d, dm = 2, 4, 10
    kp = rng.standard_normal((30, hkv, d))
    vp = rng.standard_normal((30, hkv, d))
    st, ln, cap = [0, 10, 20], [3, 0, 8], [10, 10, 10]
    cu = [0, 4, 9, 12]                     # 4, 5 and 3 new rows; sequence 2 has room for 2 only
    x = rng.standard_normal((12, dm))
    g = rng.standard_normal(dm)
    wk, wv = rng.standard_normal((dm, hkv * d)), rng.standard_normal((dm, hkv * d))
    k2, v2, ln2, flag = op.project_append_ref(kp, vp, st, ln, cap, cu, x, g, wk, wv, 1e-6)
    k, v = op.kv_project_ref(x, g, wk, wv, 1e-6)
    assert list(ln2) == [7, 5, 8] and flag == 1
    assert np.array_equal(k2[3:7].reshape(4, -1), k[0:4]) and np.array_equal(v2[10:15].reshape(5, -1), v[4:9])
    changed = [i for i in range(30) if not np.array_equal(k2[i], kp[i]) or not np.array_equal(v2[i], vp[i])]
    assert changed == list(range(3, 7)) + list(range(10, 15)), changed
    # one row per sequence = the per-token append of the projected row
    k3, v3, ln3, f3 = op.project_append_ref(kp, vp, st, ln, cap, [0, 1, 2, 3], x[:3], g, wk, wv, 1e-6)
    ka, va, lna, fa = ox.kv_append_ref(kp, vp, st, ln, cap, k[:3].reshape(3, hkv, d), v[:3].reshape(3, hkv, d))
    assert np.array_equal(k3, ka) and np.array_equal(v3, va) and list(ln3) == list(lna) and f3 == fa == 0


# ---------------------------------------------------------------------------
# gated retention (gRet)
# ---------------------------------------------------------------------------

def _brute_gret(q, k, v, g, s0=None):
    """Pure-Python recurrence on lists: S <- g S + k^T v, o = q S."""
    dk, dv = len(k[0]), len(v[0])
    st = [[0.0] * dv for _ in range(dk)] if s0 is None else [list(map(float, row)) for row in s0]
    out = []
    for t in range(len(q)):
        st = [[float(g[t]) * st[i][j] + float(k[t][i]) * float(v[t][j]) for j in range(dv)] for i in range(dk)]
        out.append([math.fsum(float(q[t][i]) * st[i][j] for i in range(dk)) for j in range(dv)])
    return np.array(out), np.array(st)


def check_gret_forms():
    """The three forms agree (the pages state they are equivalent): the parallel
    form against pure-Python loops of the recurrence, the NumPy recurrence and
    the chunkwise form at several chunk sizes, with and without an initial state."""
    rng = _rng(23)
    for n, dk, dv in [(1, 3, 2), (9, 4, 3), (40, 8, 5)]:
        q, k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
        g = rng.uniform(0.3, 1.0, n)
        for s0 in (None, rng.standard_normal((dk, dv))):
            o_p, s_p = og.gret_parallel_ref(q, k, v, g, s0)
            o_b, s_b = _brute_gret(q, k, v, g, s0)
            assert np.max(np.abs(o_p - o_b)) <= 1e-12 and np.max(np.abs(s_p - s_b)) <= 1e-12, ("brute", n)
            o_r, s_r = og.gret_recurrent_ref(q, k, v, g, s0)
            assert np.max(np.abs(o_p - o_r)) <= 1e-12 and np.max(np.abs(s_p - s_r)) <= 1e-12, ("recurrent", n)
            for chunk in (1, 3, 4, 7, n, 256):
                o_c, s_c = og.gret_chunkwise_ref(q, k, v, g, s0, chunk)
                assert np.max(np.abs(o_p - o_c)) <= 1e-12 and np.max(np.abs(s_p - s_c)) <= 1e-12, ("chunk", n, chunk)


def check_gret_closed_forms():
    """gamma = 1 is causal linear attention, tril(q k^T) v; a zero gate at t0
    forgets everything before t0; one token gives (q.k) v + gamma q S0; the decay
    matrix and a two-token case worked by hand."""
    rng = _rng(24)
    n, dk, dv = 30, 6, 4
    q, k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
    o, s = og.gret_parallel_ref(q, k, v, np.ones(n))
    assert np.max(np.abs(o - np.tril(q @ k.T) @ v)) <= 1e-12 and np.max(np.abs(s - k.T @ v)) <= 1e-12, "gamma = 1"
    g = rng.uniform(0.5, 1.0, n)
    g[12] = 0.0
    o1, s1 = og.gret_parallel_ref(q, k, v, g)
    k2, v2 = k.copy(), v.copy()
    k2[:12] += 4.0
    v2[:12] -= 3.0
    o2, s2 = og.gret_parallel_ref(q, k2, v2, g)
    assert np.array_equal(o1[12:], o2[12:]) and np.array_equal(s1, s2), "zero gate forgets"
    assert np.max(np.abs(o1[12] - (q[12] @ k[12]) * v[12])) <= 1e-12
    s0 = rng.standard_normal((dk, dv))
    o3, s3 = og.gret_parallel_ref(q[:1], k[:1], v[:1], np.array([0.7]), s0)
    assert np.max(np.abs(o3[0] - ((q[0] @ k[0]) * v[0] + 0.7 * q[0] @ s0))) <= 1e-12
    assert np.max(np.abs(s3 - (0.7 * s0 + np.outer(k[0], v[0])))) <= 1e-12
    d = og.gret_decay_matrix(np.array([0.9, 0.5, 0.25]))
    assert np.max(np.abs(d - np.array([[1, 0, 0], [0.5, 1, 0], [0.125, 0.25, 1]]))) <= 1e-16
    # hand-worked: q = [1, 2], k = [3, 4], v = [5, 6], gamma = [0.5, 0.25] (dk = dv = 1):
    # S0 = 15, o0 = 15; S1 = 0.25 * 15 + 24 = 27.75, o1 = 55.5
    oh, sh = og.gret_parallel_ref(np.array([[1.0], [2.0]]), np.array([[3.0], [4.0]]), np.array([[5.0], [6.0]]),
                                  np.array([0.5, 0.25]))
    assert np.max(np.abs(oh[:, 0] - [15.0, 55.5])) <= 1e-14 and abs(sh[0, 0] - 27.75) <= 1e-14


def check_gret_packing():
    """Packed sequences equal separate calls; a sequence split in two calls with
    the state passed on equals one call; a decode step after a prefill equals the
    last row of the longer prefill."""
    rng = _rng(25)
    lens, h, dk, dv = (17, 5, 33), 3, 4, 6
    cu = np.concatenate([[0], np.cumsum(lens)])
    tq = int(cu[-1])
    q, k = rng.standard_normal((tq, h, dk)), rng.standard_normal((tq, h, dk))
    v, g = rng.standard_normal((tq, h, dv)), rng.uniform(0.4, 1.0, (tq, h))
    s0 = rng.standard_normal((3, h, dk, dv))
    out, st = og.gret_prefill_ref(q, k, v, g, cu, s0)
    for b in range(3):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        o_b, s_b = og.gret_prefill_ref(q[r0:r1], k[r0:r1], v[r0:r1], g[r0:r1], [0, r1 - r0], s0[b:b + 1])
        assert np.max(np.abs(o_b - out[r0:r1])) <= 1e-13 and np.max(np.abs(s_b[0] - st[b])) <= 1e-13
    # split sequence 2 at row 20 of 33
    r0 = int(cu[2])
    oa, sa = og.gret_prefill_ref(q[r0:r0 + 20], k[r0:r0 + 20], v[r0:r0 + 20], g[r0:r0 + 20], [0, 20], s0[2:3])
    ob, sb = og.gret_prefill_ref(q[r0 + 20:r0 + 33], k[r0 + 20:r0 + 33], v[r0 + 20:r0 + 33], g[r0 + 20:r0 + 33],
                                 [0, 13], sa)
    assert np.max(np.abs(np.concatenate([oa, ob]) - out[r0:r0 + 33])) <= 1e-12 and np.max(np.abs(sb[0] - st[2])) <= 1e-12
    # decode the last row of every sequence from the state after the others
    stp = np.stack([og.gret_prefill_ref(q[int(cu[b]):int(cu[b + 1]) - 1], k[int(cu[b]):int(cu[b + 1]) - 1],
                                        v[int(cu[b]):int(cu[b + 1]) - 1], g[int(cu[b]):int(cu[b + 1]) - 1],
                                        [0, lens[b] - 1], s0[b:b + 1])[1][0] for b in range(3)])
    last = cu[1:] - 1
    od, sd = og.gret_decode_ref(q[last], k[last], v[last], g[last], stp)
    assert np.max(np.abs(od - out[last])) <= 1e-12 and np.max(np.abs(sd - st)) <= 1e-12


ALL_PINS = [check_bruteforce, check_sdpa, check_closed_forms, check_invariants, check_chunked_prefill, check_append,
            check_window, check_ring, check_rmsnorm, check_project, check_combine, check_project_append,
            check_gret_forms, check_gret_closed_forms, check_gret_packing]
