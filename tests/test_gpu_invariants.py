"""GPU-side invariants of the path that hold at any size, plus guard canaries."""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import parity
import synth
from gpu_util import prefill_workspace, DEV, device_cache, f64, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu


def _case(n=700, hq=16, hkv=4, d=128, std=1.0, seed=21, dtype="bf16"):
    return synth.make_prefill_case([n], hq, hkv, d, 1, dtype, seed=seed, std=std, cap_extra=40)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_at_p_equals_prefill_row_p(dtype):
    say(f"decode(p) = prefill row p, {dtype}")
    c = _case(dtype=dtype, hq=8, hkv=2)
    out, lse = run_prefill(c)
    for p in (0, 1, 63, 64, 200, 699):
        lens = torch.tensor([p + 1], dtype=torch.int32)
        cache = device_cache(c.k_pool, c.v_pool, c.seq_start, lens, c.seq_cap)
        od, ld = run_decode(cache, c.q[0][p:p + 1], c.scale)
        parity.check(od[0], out[p], dtype, discriminating=True, what=f"decode({p}) vs prefill")
        assert np.max(np.abs(ld[0] - lse[:, p])) <= (1e-5 if dtype == "f32" else 2e-3)


def test_causal_invariance_bitwise():
    """Perturbing (finitely) rows past p leaves prefill rows <= p bit for bit."""
    say("causal invariance, prefill")
    c = _case()
    out, lse = run_prefill(c)
    p = 333
    k2, v2 = c.k_pool.clone(), c.v_pool.clone()
    g = torch.Generator().manual_seed(3)
    k2[p + 1:] = (torch.randn(k2[p + 1:].shape, generator=g) * 3).to(k2.dtype)
    v2[p + 1:] = (torch.randn(v2[p + 1:].shape, generator=g) * 3).to(v2.dtype)
    c2 = synth.PrefillCase(c.q, k2, v2, c.seq_start, c.seq_len, c.seq_cap, c.cu_seqlens, c.scale, c.dtype)
    out2, lse2 = run_prefill(c2)
    assert np.array_equal(out2[:p + 1], out[:p + 1]) and np.array_equal(lse2[:, :p + 1], lse[:, :p + 1])
    assert not np.array_equal(out2[p + 1:], out[p + 1:])


def test_decode_ignores_rows_past_len_bitwise():
    say("decode ignores capacity rows past seq_len")
    c = synth.make_decode_case([3000, 517], 16, 2, 128, 1, 1, "bf16", seed=5, std=1.0, cap_extra=300)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    o1, l1 = run_decode(cache, c.q[0, 0], c.scale)
    k2, v2 = c.k_pool.clone(), c.v_pool.clone()
    for b in range(2):
        s, n, cap = int(c.seq_start[b]), int(c.seq_len[b]), int(c.seq_cap[b])
        k2[s + n:s + cap] = 7.0
        v2[s + n:s + cap] = -9.0
    cache2 = device_cache(k2, v2, c.seq_start, c.seq_len, c.seq_cap)
    o2, l2 = run_decode(cache2, c.q[0, 0], c.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_constant_v_gives_constant_output():
    """Softmax weights sum to one: V = 1 gives O = 1 to within one bf16 ulp (the
    weights entering P.V are bf16-rounded, their fp32 sum is not)."""
    say("V = 1 gives O = 1")
    c = _case(n=900)
    v1 = torch.ones_like(c.v_pool)
    c1 = synth.PrefillCase(c.q, c.k_pool, v1, c.seq_start, c.seq_len, c.seq_cap, c.cu_seqlens, c.scale, c.dtype)
    out, _ = run_prefill(c1)
    assert np.max(np.abs(out - 1.0)) <= 2.0 ** -8
    cache = device_cache(c.k_pool, v1, c.seq_start, c.seq_len, c.seq_cap)
    od, _ = run_decode(cache, c.q[0][-1:].contiguous(), c.scale)
    assert np.max(np.abs(od - 1.0)) <= 2.0 ** -8


def test_repeatable_bitwise():
    say("two runs, identical bits")
    c = _case(n=1500, std=0.5)
    a, la = run_prefill(c)
    b, lb = run_prefill(c)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    q = c.q[0][:1].contiguous()
    d1, _ = run_decode(cache, q, c.scale)
    d2, _ = run_decode(cache, q, c.scale)
    assert np.array_equal(d1, d2)


def test_output_canaries_untouched():
    """Outputs are written only inside their rows: sentinels around them survive."""
    say("output canaries")
    c = synth.make_prefill_case([130, 77], 8, 2, 128, 1, "bf16", seed=8, std=1.0)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    total = c.total_q
    big = torch.full((total + 8, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    out = big[4:4 + total]
    lse_big = torch.full((8 * total + 64,), 5.0, dtype=torch.float32, device=DEV)
    lse = lse_big[32:32 + 8 * total].view(8, total)
    dk.xattn_prefill(cache, c.q[0].to(DEV), c.cu_seqlens.to(DEV), 130, c.scale, out=out, lse=lse,
                     workspace=prefill_workspace())
    torch.cuda.synchronize()
    assert torch.all(big[:4] == 3.0) and torch.all(big[4 + total:] == 3.0)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert torch.all(lse_big[:32] == 5.0) and torch.all(lse_big[32 + 8 * total:] == 5.0)
    # decode: sentinel rows around a [B, Hq, d] output
    dbig = torch.full((2 + 2 + 2, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    ws = dk.alloc_workspace(cache, 8, 130)
    q = c.q[0][:2].contiguous().to(DEV)
    dk.xattn_decode(cache, q, 130, c.scale, ws, out=dbig[2:4])
    torch.cuda.synchronize()
    assert torch.all(dbig[:2] == 3.0) and torch.all(dbig[4:] == 3.0)


def test_append_touches_only_its_row():
    say("append writes only the new row")
    c = synth.make_decode_case([10, 20], 4, 2, 128, 1, 1, "bf16", seed=2, std=1.0, cap_extra=5)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    k0, v0 = f64(cache.k), f64(cache.v)
    dk.kv_append(cache, c.k_new[0].to(DEV), c.v_new[0].to(DEV))
    torch.cuda.synchronize()
    k1, v1 = f64(cache.k), f64(cache.v)
    changed = sorted(set(np.nonzero((k1 != k0).any(axis=(1, 2)) | (v1 != v0).any(axis=(1, 2)))[0].tolist()))
    assert changed == [10, int(c.seq_start[1]) + 20], changed
