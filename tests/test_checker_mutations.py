"""The parity checker rejects wrong outputs and accepts a correct bf16 kernel.

Wrong outputs are made by planting a mistake in the oracle on the CPU (or by
simple stand-ins: zeros, the prefix mean that ignores Q and K, a split merge
that forgets the max rescale); the correct stand-in is the exact result with
bf16 inputs, bf16-rounded P and a bf16-rounded output.
"""
import numpy as np
import pytest
import torch

import oracle.xattn as ox
import parity
import synth


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.fixture(scope="module")
def case():
    c = synth.make_prefill_case([384], 8, 2, 128, 1, "bf16", seed=7, std=1.0)
    q = synth.to_f64(c.q[0]); k = synth.to_f64(c.k_pool); v = synth.to_f64(c.v_pool)
    args = (c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale)
    ref, lse = ox.prefill_ref(q, k, v, *args)
    return q, k, v, args, ref


def _simulated_bf16_kernel(q, k, v, args):
    """Exact scores, P rounded to bf16 after the max shift, fp32-like accumulation, bf16 output."""
    st, ln, cu, scale = args
    n = int(ln[0])
    out = np.zeros_like(q)
    g = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        kh = h // g
        s = scale * (q[:, h] @ k[:n, kh].T)
        s = np.where(np.tri(n, dtype=bool), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = _bf16(np.exp(s - m))
        l = np.exp(s - m).sum(axis=1, keepdims=True)
        out[:, h] = (p @ v[:n, kh]) / l
    return _bf16(out)


def test_correct_kernel_passes(case):
    q, k, v, args, ref = case
    e = parity.check(_simulated_bf16_kernel(q, k, v, args), ref, "bf16", discriminating=True, what="sim")
    assert e["row_rel"] < 5e-3


MUTANT_ORACLE = {
    "mask_excludes_diagonal": ("visible_rows", lambda p: p if p > 0 else 1),
    "mask_one_past": ("prefill_position", lambda r, m, n: r + 1),
    "head_map_interleaved": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "no_scale": ("scores", lambda q, k, scale: q @ k.T),
    "double_scale": ("scores", lambda q, k, scale: 2 * scale * (q @ k.T)),
}


@pytest.mark.parametrize("name", sorted(MUTANT_ORACLE))
def test_checker_rejects_oracle_mutant(case, name, monkeypatch):
    q, k, v, args, ref = case
    attr, repl = MUTANT_ORACLE[name]
    monkeypatch.setattr(ox, attr, repl)
    if name == "mask_one_past":
        # row r sees rows 0..r+1: compute the rows whose extra key exists
        n = int(args[1][0])
        bad, _ = ox.prefill_ref(q, k, v, *args, rows={0: range(n - 1)})
        mut, ref_ = _bf16(bad[: n - 1]), ref[: n - 1]
    else:
        bad, _ = ox.prefill_ref(q, k, v, *args)
        mut, ref_ = _bf16(bad), ref
    with pytest.raises(AssertionError):
        parity.check(mut, ref_, "bf16", discriminating=True, what=name)


def test_checker_rejects_zeros_and_prefix_mean(case):
    q, k, v, args, ref = case
    with pytest.raises(AssertionError):
        parity.check(np.zeros_like(ref), ref, "bf16", discriminating=True)
    pm, _ = ox.prefill_ref(np.zeros_like(q), k, v, *args)
    with pytest.raises(AssertionError):
        parity.check(_bf16(pm), ref, "bf16", discriminating=True)


def test_checker_rejects_merge_without_rescale(case):
    q, k, v, args, ref = case
    st, ln, cu, scale = args
    n = int(ln[0])
    g = q.shape[1] // k.shape[1]
    out = np.zeros_like(ref)
    half = 128
    for h in range(q.shape[1]):
        kh = h // g
        for r in range(n):
            parts = []
            for lo, hi in ((0, half), (half, r + 1)):
                if hi <= lo:
                    continue
                s = scale * (k[lo:hi, kh] @ q[r, h])
                w = np.exp(s - s.max())
                parts.append((w.sum(), w @ v[lo:hi, kh]))
            lsum = sum(p[0] for p in parts)
            out[r, h] = sum(p[1] for p in parts) / lsum   # forgot exp(m_s - M)
    with pytest.raises(AssertionError):
        parity.check(_bf16(out), ref, "bf16", discriminating=True)


def test_max_abs_alone_is_weak_on_small_logits():
    """Documented weakness: on N(0,1)/sqrt(d) inputs an output that ignores Q and K
    (the prefix mean of V) passes the 2e-2 max-abs bound; the discriminating suites
    exist because of this."""
    c = synth.make_prefill_case([512], 4, 1, 128, 1, "bf16", seed=3, std=128 ** -0.5)
    args = (c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale)
    q, k, v = synth.to_f64(c.q[0]), synth.to_f64(c.k_pool), synth.to_f64(c.v_pool)
    ref, _ = ox.prefill_ref(q, k, v, *args)
    pm, _ = ox.prefill_ref(np.zeros_like(q), k, v, *args)
    parity.check(_bf16(pm), ref, "bf16", discriminating=False)
    with pytest.raises(AssertionError):
        parity.check(_bf16(pm), ref, "bf16", discriminating=True)


def test_signed_sum_check_for_gated_retention():
    """The gRet check (bulk row-relative bound plus a looser cap for rows that
    cancel) accepts bf16 weights and outputs and rejects a carried state that is
    dropped or passed on without a chunk boundary's decay."""
    import oracle.gret as og
    rng = np.random.default_rng(5)
    n, d = 1200, 64
    q = _bf16(rng.standard_normal((n, d)) * d ** -0.25)
    k = _bf16(rng.standard_normal((n, d)) * d ** -0.25)
    v = _bf16(rng.standard_normal((n, d)))
    gam = 0.8 + 0.2 * rng.random(n)
    ref, _ = og.gret_recurrent_ref(q, k, v, gam)
    sim = _bf16(_bf16((q @ k.T) * og.gret_decay_matrix(gam)) @ v)   # bf16 weights and output
    e = parity.check_signed_sum(sim[:, None], ref[:, None], "bf16", what="sim")
    assert e["row_rel"] < 1e-2
    dropped = np.concatenate([og.gret_recurrent_ref(q[c:c + 256], k[c:c + 256], v[c:c + 256], gam[c:c + 256])[0]
                              for c in range(0, n, 256)])
    with pytest.raises(AssertionError):
        parity.check_signed_sum(_bf16(dropped)[:, None], ref[:, None], "bf16")
    g2 = gam.copy()
    g2[256::256] = 1.0                       # the state enters each chunk undecayed by its first gate
    undecayed, _ = og.gret_recurrent_ref(q, k, v, g2)
    with pytest.raises(AssertionError):
        parity.check_signed_sum(_bf16(undecayed)[:, None], ref[:, None], "bf16")
