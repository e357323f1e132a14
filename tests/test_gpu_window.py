"""Sliding-window attention (the Self-Decoder's band mask) and the ring window
cache, through the C ABI, against the fp64 oracle.

Position p attends rows max(0, p - C + 1) .. p. Covered: windows below, at and
above the 64-key tile, a window of 1 (the own row), windows covering the whole
sequence (equal to the causal calls, bitwise), chunks of queries after cached
rows, head_dim 64, fp32 storage, decode over a full cache, and a ring of C slots
fed token by token across several wrap-arounds."""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import oracle
import parity
import synth
from gpu_util import DEV, device_cache, f64, prefill_workspace, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu


def run_prefill_window(case, window, layer=0, max_q=None, queue=True):
    cache = device_cache(case.k_pool, case.v_pool, case.seq_start, case.seq_len, case.seq_cap)
    q = case.q[layer].to(DEV)
    lse = torch.full((q.shape[1], case.total_q), float("nan"), device=DEV)
    if max_q is None:
        max_q = int((case.cu_seqlens[1:] - case.cu_seqlens[:-1]).max())
    out = dk.xattn_prefill_window(cache, q, case.cu_seqlens.to(DEV), max_q, window, case.scale, lse=lse,
                                  workspace=prefill_workspace() if queue else None)
    torch.cuda.synchronize()
    return f64(out), lse.cpu().numpy().astype(np.float64)


def ref_prefill(case, window, rows=None, layer=0):
    return oracle.prefill_ref(synth.to_f64(case.q[layer]), synth.to_f32(case.k_pool), synth.to_f32(case.v_pool),
                              case.seq_start.numpy(), case.seq_len.numpy(), case.cu_seqlens.numpy(), case.scale,
                              rows=rows, window=window)


@pytest.mark.parametrize("lens,window,hq,hkv,d,dtype", [
    ((1000,), 100, 16, 4, 128, "bf16"),        # window inside one or two tiles, ragged tail
    ((777, 300, 64), 64, 16, 2, 128, "bf16"),  # window = tile, packed sequences, g = 8
    ((1300,), 1, 8, 2, 128, "bf16"),           # the own row only
    ((513,), 33, 6, 3, 64, "bf16"),            # head_dim 64, window below a tile
    ((2100, 90), 700, 32, 8, 128, "bf16"),     # window spanning many tiles
    ((300, 40), 50, 4, 1, 64, "f32"),
])
def test_window_prefill(lens, window, hq, hkv, d, dtype):
    say(f"window prefill {dtype} lens={lens} C={window} hq={hq} hkv={hkv} d={d}")
    c = synth.make_prefill_case(list(lens), hq, hkv, d, 1, dtype, seed=sum(lens) + window, std=1.0, cap_extra=5)
    out, lse = run_prefill_window(c, window)
    ref, ref_lse = ref_prefill(c, window)
    e = parity.check(out, ref, dtype, discriminating=True, what="window prefill")
    parity.check_lse(lse, ref_lse, dtype, what="window prefill lse")
    say(f"  max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


@pytest.mark.parametrize("window", [100, 700])
def test_window_prefill_running_max_jumps(window):
    # key rows scaled up mid-tile: the row max jumps by units, tens and hundreds
    # inside the band, and drops again once the scaled rows leave it
    say(f"window prefill bf16 with score jumps C={window}")
    c = synth.make_prefill_case([1000], 8, 2, 128, 1, "bf16", seed=5 + window, std=1.0, cap_extra=2)
    k = c.k_pool.to(torch.float32)
    for pos, f in {100: 4.0, 230: 16.0, 650: 30.0, 703: 100.0, 767: 60.0}.items():
        k[int(c.seq_start[0]) + pos] *= f
    c.k_pool = k.to(torch.bfloat16)
    out, lse = run_prefill_window(c, window)
    ref, ref_lse = ref_prefill(c, window)
    assert np.isfinite(out).all()
    parity.check(out, ref, "bf16", discriminating=True, what="window prefill (jumps)")
    parity.check_lse(lse, ref_lse, "bf16", what="window prefill lse (jumps)")


@pytest.mark.parametrize("lens,window,hq,hkv,d", [
    ((1000, 300, 64, 1, 0, 517), 64, 16, 4, 128),   # short, single-row and empty sequences
    ((5, 130, 64, 2000), 100, 8, 2, 128),
    ((700, 129), 33, 6, 3, 64),
])
def test_window_grid_hint(lens, window, hq, hkv, d):
    """max_q_len only sizes the grid: with a hint of 1 every workgroup walks all
    position blocks of its unit in turn, and each row comes out bitwise as with
    one workgroup per block; both match the oracle (short and single-row
    sequences, an empty one, head_dim 64)."""
    say(f"window grid hint lens={lens} C={window} hq={hq} hkv={hkv} d={d}")
    c = synth.make_prefill_case(list(lens), hq, hkv, d, 1, "bf16", seed=sum(lens) + 3 * window, std=1.0, cap_extra=3)
    out, lse = run_prefill_window(c, window)
    out1, lse1 = run_prefill_window(c, window, max_q=1)
    assert np.array_equal(out, out1) and np.array_equal(lse, lse1, equal_nan=True)
    ref, ref_lse = ref_prefill(c, window)
    parity.check(out, ref, "bf16", discriminating=True, what="window grid hint")
    parity.check_lse(lse, ref_lse, "bf16", what="window grid hint lse")


def test_window_one_is_own_row():
    c = synth.make_prefill_case([700], 8, 2, 128, 1, "bf16", seed=5, std=1.0)
    out, _ = run_prefill_window(c, 1)
    v = synth.to_f64(c.v_pool)[:700]
    for h in range(8):
        assert np.array_equal(out[:, h], v[:, h // 4]), "window 1 returns the own V row exactly"


@pytest.mark.parametrize("window", [2000, 1 << 30])
def test_window_covering_sequence_equals_causal(window):
    say(f"window {window} = causal, bitwise")
    c = synth.make_prefill_case([1500, 333], 16, 4, 128, 1, "bf16", seed=9, std=1.0)
    out_w, lse_w = run_prefill_window(c, window)
    out_c, lse_c = run_prefill(c)
    assert np.array_equal(out_w, out_c) and np.array_equal(lse_w, lse_c)


def test_window_chunk_after_cached_rows():
    say("window chunk: 100 queries after 900 cached rows, C = 200")
    c = synth.make_chunk_case([1000, 250], [100, 250], 16, 4, 128, "bf16", seed=77, std=1.0, cap_extra=2)
    out, lse = run_prefill_window(c, 200)
    ref, ref_lse = ref_prefill(c, 200)
    parity.check(out, ref, "bf16", discriminating=True, what="window chunk")
    parity.check_lse(lse, ref_lse, "bf16", what="window chunk lse")


def test_rows_before_the_window_do_not_matter():
    """Perturbing (finite) rows before every query's window leaves those queries bitwise unchanged."""
    c = synth.make_prefill_case([1200], 16, 4, 128, 1, "bf16", seed=21, std=1.0)
    window, first = 300, 700                 # rows >= first see only rows >= first - window + 1 = 401
    out0, lse0 = run_prefill_window(c, window)
    k2, v2 = c.k_pool.clone(), c.v_pool.clone()
    k2[:401] = (k2[:401].float() * 3.0 + 1.0).to(torch.bfloat16)
    v2[:401] = (v2[:401].float() - 5.0).to(torch.bfloat16)
    c2 = synth.PrefillCase(c.q, k2, v2, c.seq_start, c.seq_len, c.seq_cap, c.cu_seqlens, c.scale, "bf16")
    out1, lse1 = run_prefill_window(c2, window)
    assert np.array_equal(out1[first:], out0[first:]) and np.array_equal(lse1[:, first:], lse0[:, first:])
    assert np.abs(out1[:first] - out0[:first]).max() > 1e-2


def test_window_prefill_32k_sampled():
    """The Self-Decoder setting at full length: N = 32768, C = 1024 (YOCO's window)."""
    say("window prefill 32K, C = 1024, sampled rows")
    c = synth.make_prefill_case([32768], 16, 4, 128, 1, "bf16", seed=1, std=1.0)
    out, lse = run_prefill_window(c, 1024)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, 63, 64, 1023, 1024, 1025, 4095, 32767] + list(rng.integers(0, 32768, 40))))
    ref, ref_lse = ref_prefill(c, 1024, rows={0: rows})
    parity.check(out[rows], ref[rows], "bf16", discriminating=True, what="window 32K")
    parity.check_lse(lse[:, rows], ref_lse[:, rows], "bf16", what="window 32K lse")


@pytest.mark.parametrize("window", [1, 100, 1024, 4096])
def test_window_decode(window):
    say(f"window decode C={window}")
    lens = [5000, 100, 2049]
    c = synth.make_decode_case(lens, 16, 2, 128, 1, 1, "bf16", seed=window, std=1.0)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    q = c.q[0, 0].to(DEV)
    ws = dk.alloc_workspace(cache, 16, max(lens))
    lse = torch.full((3, 16), float("nan"), device=DEV)
    out = dk.xattn_decode_window(cache, q, max(lens), window, c.scale, ws, lse=lse, total_kv_len=sum(lens))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[0, 0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                     c.seq_start.numpy(), c.seq_len.numpy(), c.scale, window=window)
    parity.check(f64(out), ref, "bf16", discriminating=True, what="window decode")
    parity.check_lse(lse.cpu().numpy(), ref_lse, "bf16", what="window decode lse")


def test_ring_window_cache():
    """Token-by-token decode with a ring of C = 96 slots: after each append the
    decode over the ring equals windowed decode over the whole history."""
    C, steps, hq, hkv, d, B = 96, 260, 8, 2, 128, 2
    say(f"ring window cache C={C}, {steps} steps")
    hist = synth.make_decode_case([1, 1], hq, hkv, d, 1, steps, "bf16", seed=123, std=1.0)
    ring = dk.SharedKV(torch.randn(B * C + 4, hkv, d, device=DEV).to(torch.bfloat16),
                       torch.randn(B * C + 4, hkv, d, device=DEV).to(torch.bfloat16),
                       torch.tensor([0, C + 4], dtype=torch.int64, device=DEV),
                       torch.zeros(B, dtype=torch.int32, device=DEV),
                       torch.tensor([C, C], dtype=torch.int32, device=DEV))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    kn, vn = hist.k_new.to(DEV), hist.v_new.to(DEV)
    ws = dk.alloc_workspace(ring, hq, C)
    lin_k = synth.to_f32(hist.k_new).transpose(1, 0, 2, 3)   # [B, steps, Hkv, d]
    lin_v = synth.to_f32(hist.v_new).transpose(1, 0, 2, 3)
    checked = 0
    for t in range(steps):
        dk.kv_append_ring(ring, kn[t], vn[t], flag)
        if t % 37 == 36 or t in (0, C - 1, C, steps - 1):
            q = torch.randn(B, hq, d, generator=torch.Generator().manual_seed(t)).to(torch.bfloat16)
            out = dk.xattn_decode(ring, q.to(DEV), C, hist.scale, ws)
            torch.cuda.synchronize()
            kp = lin_k[:, :t + 1].reshape(B * (t + 1), hkv, d)
            vp = lin_v[:, :t + 1].reshape(B * (t + 1), hkv, d)
            ref, _ = oracle.decode_ref(synth.to_f64(q), kp, vp, [0, t + 1], [t + 1, t + 1], hist.scale, window=C)
            parity.check(f64(out), ref, "bf16", discriminating=True, what=f"ring step {t}")
            checked += 1
    assert int(flag.item()) == 0 and checked >= 8
    assert ring.seq_len.cpu().tolist() == [steps, steps]
    # slot s holds the latest token t with t mod C == s
    kr = ring.k.cpu()
    for s in (0, 5, C - 1):
        t = max(x for x in range(steps) if x % C == s)
        assert torch.equal(kr[s], hist.k_new[t, 0]) and torch.equal(kr[C + 4 + s], hist.k_new[t, 1])


def test_ring_rejects_sequence_without_rows():
    ring = dk.SharedKV(torch.zeros(8, 1, 64, device=DEV, dtype=torch.bfloat16),
                       torch.zeros(8, 1, 64, device=DEV, dtype=torch.bfloat16),
                       torch.tensor([0, 4], dtype=torch.int64, device=DEV),
                       torch.tensor([3, 0], dtype=torch.int32, device=DEV),
                       torch.tensor([4, 0], dtype=torch.int32, device=DEV))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    new = torch.ones(2, 1, 64, device=DEV, dtype=torch.bfloat16)
    dk.kv_append_ring(ring, new, new, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1 and ring.seq_len.cpu().tolist() == [4, 0]
    assert torch.all(ring.k[3].cpu() == 1) and torch.all(ring.k[4:].cpu() == 0)
