"""Parity at the benchmark workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same grids, same split plans).

Prefill rows are sampled (every tile boundary of the first tiles, the first and
last rows, random rows); decode calls are compared whole.
"""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import oracle
import parity
import synth
from gpu_util import DEV, device_cache, f64, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu


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


def test_decode_128k_two_layers():
    w = synth.WORKLOADS["decode_128k"]
    say("decode 8 x 131072")
    c = synth.make_decode_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, w.layers, 1, w.dtype, w.seed,
                               w.value_std)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dk.kv_append(cache, c.k_new[0].to(DEV), c.v_new[0].to(DEV), flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and cache.seq_len.cpu().tolist() == [131072] * 8
    kf, vf = synth.to_f32(c.k_pool), synth.to_f32(c.v_pool)
    kf, vf, ln, _ = oracle.kv_append_ref(kf, vf, c.seq_start.numpy(), c.seq_len.numpy(), c.seq_cap.numpy(),
                                         synth.to_f32(c.k_new[0]), synth.to_f32(c.v_new[0]))
    for layer in (0, w.layers - 1):
        out, lse = run_decode(cache, c.q[0, layer], c.scale, max_kv_len=131072)
        ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[0, layer]), kf, vf, c.seq_start.numpy(), ln, c.scale)
        e = parity.check(out, ref, "bf16", what=f"decode 128k layer {layer}")
        parity.check_lse(lse, ref_lse, "bf16")
        say(f"  layer {layer}: max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


def test_decode_1m_steps():
    w = synth.WORKLOADS["decode_1m"]
    say("decode 1 x 1048576, steps 0 and 63")
    c = synth.make_decode_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, w.layers, w.decode_steps,
                               w.dtype, w.seed, w.value_std)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    kf, vf = synth.to_f32(c.k_pool), synth.to_f32(c.v_pool)
    ln = c.seq_len.numpy()
    max_len = int(c.seq_len[0]) + w.decode_steps
    for step in range(w.decode_steps):
        dk.kv_append(cache, c.k_new[step].to(DEV), c.v_new[step].to(DEV), flag)
        kf, vf, ln, _ = oracle.kv_append_ref(kf, vf, c.seq_start.numpy(), ln, c.seq_cap.numpy(),
                                             synth.to_f32(c.k_new[step]), synth.to_f32(c.v_new[step]))
        if step in (0, w.decode_steps - 1):
            for layer in ((0, w.layers - 1) if step == 0 else (7,)):
                out, lse = run_decode(cache, c.q[step, layer], c.scale, max_kv_len=max_len)
                ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[step, layer]), kf, vf, c.seq_start.numpy(), ln,
                                                 c.scale)
                e = parity.check(out, ref, "bf16", what=f"decode 1m step {step} layer {layer}")
                parity.check_lse(lse, ref_lse, "bf16")
                say(f"  step {step} layer {layer}: max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and int(cache.seq_len.item()) == 1048576 + 64


def test_ragged_prefill_and_decode():
    w = synth.WORKLOADS["ragged"]
    say(f"ragged prefill + decode, lengths {w.seq_lens}")
    c = synth.make_prefill_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, 1, w.dtype, w.seed,
                                w.value_std, cap_extra=w.decode_steps)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    out, lse = run_prefill(c, cache=cache)
    rows = {b: sample_rows(n, 100 + b, extra=8) for b, n in enumerate(w.seq_lens)}
    check_rows(out, lse, c, rows, "ragged prefill")
    d = synth.make_decode_case([1] * w.batch, w.q_heads, w.kv_heads, w.head_dim, 1, w.decode_steps, w.dtype,
                               w.seed, w.value_std)
    kf, vf = synth.to_f32(c.k_pool), synth.to_f32(c.v_pool)
    ln = c.seq_len.numpy()
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    max_len = max(w.seq_lens) + w.decode_steps
    for step in range(w.decode_steps):
        dk.kv_append(cache, d.k_new[step].to(DEV), d.v_new[step].to(DEV), flag)
        kf, vf, ln, _ = oracle.kv_append_ref(kf, vf, c.seq_start.numpy(), ln, c.seq_cap.numpy(),
                                             synth.to_f32(d.k_new[step]), synth.to_f32(d.v_new[step]))
        if step in (0, w.decode_steps - 1):
            o, l = run_decode(cache, d.q[step, 0], c.scale, max_kv_len=max_len)
            ref, ref_lse = oracle.decode_ref(synth.to_f64(d.q[step, 0]), kf, vf, c.seq_start.numpy(), ln, c.scale)
            e = parity.check(o, ref, "bf16", what=f"ragged decode step {step}")
            parity.check_lse(l, ref_lse, "bf16")
            say(f"  decode step {step}: max-abs {e['max_abs']:.2e}")
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
