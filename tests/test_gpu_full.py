"""Parity at the benchmark workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same grids, same split plans).

Prefill rows are sampled (every tile boundary of the first tiles, the first and
last rows, random rows); decode calls are compared whole.

Each decode workload runs on three inputs:
  * "acceptance": the workload's own inputs (entries N(0,1)/sqrt(128)), checked
    against the max-abs bound; at these lengths the outputs are ~1e-3, so this
    bound alone cannot tell a wrong output from a right one;
  * "unit": Q and K^ entries N(0,1) (logits of unit spread), checked against
    the row-relative bound;
  * "needles": the acceptance inputs with planted needle rows (tests/needles.py)
    that every share of the decode split holds for every checked query, and an
    appended row that is a needle of the step's first checked query; checked
    against the row-relative bound.
"""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import needles
import oracle
import parity
import synth
from gpu_util import DEV, device_cache, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu

VARIANTS = ("acceptance", "unit", "needles")


def sample_rows(n, seed, extra=64):
    rows = {0, 1, 2, n - 1, n - 2, n - 3}
    for t in range(1, min(n // 32, 12)):
        rows |= {32 * t - 1, 32 * t, 32 * t + 1}
    rows |= {64 * t for t in range(1, n // 64, max(1, n // 64 // 16))}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, n, size=extra))
    return sorted(r for r in rows if 0 <= r < n)


def check_rows(out, lse, c, rows_by_seq, what, disc=False, layer=0):
    ref, ref_lse = oracle.prefill_ref(synth.to_f64(c.q[layer]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                      c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale,
                                      rows=rows_by_seq)
    idx = np.concatenate([int(c.cu_seqlens[b]) + np.asarray(r, dtype=np.int64) for b, r in rows_by_seq.items()])
    e = parity.check(out[idx], ref[idx], c.dtype, discriminating=disc, what=what)
    parity.check_lse(lse[:, idx], ref_lse[:, idx], c.dtype, what=what + " lse")
    say(f"  {what}: {len(idx)} rows, max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


@pytest.mark.parametrize("std,disc", [(128 ** -0.5, False), (1.0, True)])
def test_prefill_32k(std, disc):
    w = synth.WORKLOADS["prefill_32k"]
    say(f"prefill 32k std={std:.3f}")
    c = synth.make_prefill_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, 1, w.dtype, w.seed, std)
    out, lse = run_prefill(c)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check_rows(out, lse, c, {0: sample_rows(w.seq_lens[0], 1)}, "prefill 32k", disc)


def _decode_case(w, variant, steps, lens=None, layers=None):
    lens = list(w.seq_lens) if lens is None else lens
    layers = w.layers if layers is None else layers
    unit = dict(q_std=1.0, k_std=1.0) if variant == "unit" else {}
    return synth.make_decode_case(lens, w.q_heads, w.kv_heads, w.head_dim, layers, steps, w.dtype, w.seed,
                                  w.value_std, **unit)


def _plant(c, w, name, checked, appended_steps):
    """Needles aligned with the checked (step, layer) queries, dealt round-robin;
    the appended row of each step in appended_steps is a needle of that step's
    first checked query."""
    queries = [c.q[s, l] for s, l in checked]
    needles.plant(c.k_pool, c.v_pool, c.seq_start.numpy(), c.seq_len.numpy(), queries, c.scale,
                  needles.STRIDE[name], seed=w.seed + 100)
    for s in appended_steps:
        layer = next(l for st, l in checked if st == s)
        kn, vn = needles.aligned_rows(c.q[s, layer], w.kv_heads, c.scale, seed=w.seed + 200 + s,
                                      dtype=c.k_new.dtype)
        c.k_new[s] = kn
        c.v_new[s] = vn


class TailPool:
    """The oracle's view of the appends: kv_append_ref applied to the capacity
    rows past each sequence's prompt (the only rows an append writes), then
    scattered back into float32 copies of the pool at the checked steps."""

    def __init__(self, c):
        self.k = synth.to_f32(c.k_pool)
        self.v = synth.to_f32(c.v_pool)
        self.start = c.seq_start.numpy().astype(np.int64)
        self.n0 = c.seq_len.numpy().astype(np.int64)
        self.cap = c.seq_cap.numpy().astype(np.int64)
        sizes = self.cap - self.n0
        self.tstart = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
        idx = np.concatenate([np.arange(s + n, s + c_) for s, n, c_ in zip(self.start, self.n0, self.cap)])
        self.idx = idx
        self.tk, self.tv = self.k[idx], self.v[idx]
        self.tlen = np.zeros_like(self.n0)

    def append(self, k_new, v_new):
        self.tk, self.tv, self.tlen, ov = oracle.kv_append_ref(self.tk, self.tv, self.tstart, self.tlen,
                                                               self.cap - self.n0, synth.to_f32(k_new),
                                                               synth.to_f32(v_new))
        assert ov == 0

    def pool(self):
        self.k[self.idx] = self.tk
        self.v[self.idx] = self.tv
        return self.k, self.v, self.n0 + self.tlen


def _check_decode(cache, c, step, layer, pool, max_len, variant, what):
    k, v, ln = pool
    out, lse = run_decode(cache, c.q[step, layer], c.scale, max_kv_len=max_len)
    ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[step, layer]), k, v, c.seq_start.numpy(), ln, c.scale)
    e = parity.check(out, ref, "bf16", discriminating=variant != "acceptance", what=what)
    le = parity.check_lse(lse, ref_lse, "bf16", what=what + " lse")
    say(f"  {what}: max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e} lse {le:.2e} "
        f"(|ref| max {np.abs(ref).max():.2e})")


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_128k(variant):
    w = synth.WORKLOADS["decode_128k"]
    say(f"decode 8 x 131072, {variant}")
    c = _decode_case(w, variant, 1)
    checked = [(0, 0), (0, w.layers - 1)]
    if variant == "needles":
        _plant(c, w, "decode_128k", checked, appended_steps=[0])
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    tail = TailPool(c)
    dk.kv_append(cache, c.k_new[0].to(DEV), c.v_new[0].to(DEV), flag)
    tail.append(c.k_new[0], c.v_new[0])
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and cache.seq_len.cpu().tolist() == [131072] * 8
    pool = tail.pool()
    for step, layer in checked:
        _check_decode(cache, c, step, layer, pool, 131072, variant, f"decode 128k {variant} layer {layer}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_1m_steps(variant):
    w = synth.WORKLOADS["decode_1m"]
    checked = [(0, 0), (0, w.layers - 1), (1, 3), (w.decode_steps - 1, 7)]
    say(f"decode 1 x 1048576, {variant}, checked (step, layer) {checked}")
    c = _decode_case(w, variant, w.decode_steps)
    if variant == "needles":
        _plant(c, w, "decode_1m", checked, appended_steps=[0, 1, w.decode_steps - 1])
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    tail = TailPool(c)
    max_len = int(c.seq_len[0]) + w.decode_steps
    for step in range(w.decode_steps):
        dk.kv_append(cache, c.k_new[step].to(DEV), c.v_new[step].to(DEV), flag)
        tail.append(c.k_new[step], c.v_new[step])
        layers = [l for s, l in checked if s == step]
        if layers:
            pool = tail.pool()
            for layer in layers:
                _check_decode(cache, c, step, layer, pool, max_len, variant,
                              f"decode 1m {variant} step {step} layer {layer}")
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and int(cache.seq_len.item()) == 1048576 + 64


@pytest.mark.parametrize("std,disc", [(128 ** -0.5, False), (1.0, True)])
def test_ragged_prefill(std, disc):
    w = synth.WORKLOADS["ragged"]
    say(f"ragged prefill std={std:.3f}, lengths {w.seq_lens}")
    c = synth.make_prefill_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, 1, w.dtype, w.seed, std,
                                cap_extra=w.decode_steps)
    out, lse = run_prefill(c)
    rows = {b: sample_rows(n, 100 + b, extra=8) for b, n in enumerate(w.seq_lens)}
    check_rows(out, lse, c, rows, f"ragged prefill std={std:.3f}", disc)


@pytest.mark.parametrize("variant", VARIANTS)
def test_ragged_decode(variant):
    """The 32 decode steps (append + one layer call) after the ragged prompts
    (prefill leaves the cache as it is; it is checked above)."""
    w = synth.WORKLOADS["ragged"]
    say(f"ragged decode, {variant}")
    last = w.decode_steps - 1
    checked = [(0, 0), (last, 0)]
    c = _decode_case(w, variant, w.decode_steps, layers=1)
    if variant == "needles":
        _plant(c, w, "ragged", checked, appended_steps=[0, last])
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    tail = TailPool(c)
    max_len = max(w.seq_lens) + w.decode_steps
    for step in range(w.decode_steps):
        dk.kv_append(cache, c.k_new[step].to(DEV), c.v_new[step].to(DEV), flag)
        tail.append(c.k_new[step], c.v_new[step])
        if step in (0, last):
            _check_decode(cache, c, step, 0, tail.pool(), max_len, variant, f"ragged decode {variant} step {step}")
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
