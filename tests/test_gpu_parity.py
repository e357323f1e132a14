"""GPU parity: the HIP path against the fp64 oracle, element by element.

Sizes span several tiles with ragged tails; grouped heads g = 1, 2, 3, 4, 8,
32; head_dim 64 and 128; fp32 and bf16 storage. Inputs with N(0,1) entries are
the discriminating suites (row-relative bound); N(0,1)/sqrt(d) entries are the
acceptance distribution (max-abs bound).
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import synth
from gpu_util import DEV, device_cache, f64, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu


def _oracle_prefill(c, layer=0, rows=None):
    return oracle.prefill_ref(synth.to_f64(c.q[layer]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                              c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale, rows=rows)


# --------------------------------------------------------------------------- prefill


@pytest.mark.parametrize("lens,hq,hkv,d,std,disc", [
    ((1000,), 16, 4, 128, 1.0, True),         # g=4, 16 tiles of 64 keys + ragged tail
    ((777,), 16, 4, 128, 128 ** -0.5, False),  # acceptance distribution
    ((513, 1, 64, 200), 8, 2, 128, 1.0, True),  # varlen, g=4
    ((300,), 4, 4, 128, 1.0, True),           # g=1 (MHA)
    ((301,), 6, 3, 128, 1.0, True),           # g=2
    ((257,), 6, 2, 128, 1.0, True),           # g=3 (the 24/8 geometry ratio)
    ((333,), 8, 1, 128, 1.0, True),           # g=8
    ((450,), 8, 2, 64, 1.0, True),            # head_dim 64
    ((129, 31), 32, 8, 128, 2.0, True),        # larger logits
])
def test_prefill_bf16(lens, hq, hkv, d, std, disc):
    say(f"prefill bf16 lens={lens} hq={hq} hkv={hkv} d={d} std={std}")
    c = synth.make_prefill_case(list(lens), hq, hkv, d, 1, "bf16", seed=sum(lens) + hq, std=std, cap_extra=5)
    out, lse = run_prefill(c)
    ref, ref_lse = _oracle_prefill(c)
    e = parity.check(out, ref, "bf16", discriminating=disc, what="prefill out")
    parity.check_lse(lse, ref_lse, "bf16", what="prefill lse")
    say(f"  max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


# Key rows scaled up at chosen positions make the running row max jump in the
# middle of a row: by a few units, by tens (past any bound on weights taken
# against the old reference) and by hundreds (exp2 overflows there), in the first
# (offset < 32) and in the second half of a 64-key tile, and at a tile's first
# and last key.
_JUMPS = {100: 4.0, 101: 4.0, 102: 4.0, 230: 16.0, 384: 8.0, 650: 30.0, 703: 100.0, 767: 60.0}


def _with_jumps(c, jumps=_JUMPS):
    k = c.k_pool.to(torch.float32)
    for b in range(c.seq_start.numel()):
        s0, n = int(c.seq_start[b]), int(c.seq_len[b])
        for pos, f in jumps.items():
            if pos < n:
                k[s0 + pos] *= f
    c.k_pool = k.to(c.k_pool.dtype)
    return c


@pytest.mark.parametrize("lens,hq,hkv,d,dtype", [
    ((1000,), 8, 2, 128, "bf16"),
    ((800, 720), 4, 1, 64, "bf16"),
])
def test_prefill_running_max_jumps(lens, hq, hkv, d, dtype):
    say(f"prefill {dtype} with score jumps lens={lens} hq={hq} hkv={hkv} d={d}")
    c = _with_jumps(synth.make_prefill_case(list(lens), hq, hkv, d, 1, dtype, seed=77 + d, std=1.0, cap_extra=3))
    out, lse = run_prefill(c)
    ref, ref_lse = _oracle_prefill(c)
    assert np.isfinite(out).all()
    e = parity.check(out, ref, dtype, discriminating=True, what="prefill out (jumps)")
    parity.check_lse(lse, ref_lse, dtype, what="prefill lse (jumps)")
    say(f"  max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


@pytest.mark.parametrize("lens,hq,hkv,d", [((256,), 4, 1, 64), ((100, 37), 8, 2, 128), ((70,), 4, 4, 64)])
def test_prefill_f32(lens, hq, hkv, d):
    say(f"prefill f32 lens={lens} hq={hq} hkv={hkv} d={d}")
    c = synth.make_prefill_case(list(lens), hq, hkv, d, 1, "f32", seed=9, std=1.0, cap_extra=2)
    out, lse = run_prefill(c)
    ref, ref_lse = _oracle_prefill(c)
    parity.check(out, ref, "f32", discriminating=True, what="prefill f32")
    parity.check_lse(lse, ref_lse, "f32", what="prefill f32 lse")


# --------------------------------------------------------------------------- decode


@pytest.mark.parametrize("lens,hq,hkv,d,dtype,std", [
    ((1, 100, 5000), 16, 2, 128, "bf16", 1.0),   # g=8, lengths 1 .. several splits
    ((40000, 7, 900, 13000), 8, 2, 128, "bf16", 1.0),  # ragged lengths: splits sized by the total
    ((4097, 300), 32, 8, 128, "bf16", 1.0),      # g=4
    ((2000,), 32, 1, 128, "bf16", 1.0),          # g=32: two head chunks of 16
    ((999,), 12, 4, 64, "bf16", 1.0),            # g=3, head_dim 64
    ((3000, 17), 16, 2, 128, "bf16", 128 ** -0.5),
    ((255, 40), 4, 1, 64, "f32", 1.0),
    ((1000,), 8, 2, 128, "f32", 1.0),
    ((20000,), 8, 1, 64, "bf16", 1.0),           # one long sequence: many pieces per sequence in the merge
    ((20000,), 8, 2, 128, "f32", 1.0),           # the same for fp32 storage
    ((3000, 2500), 32, 8, 64, "bf16", 1.0),      # eight KV heads (whole-row K^ loads), head_dim 64
])
def test_decode(lens, hq, hkv, d, dtype, std):
    say(f"decode {dtype} lens={lens} hq={hq} hkv={hkv} d={d} std={std}")
    c = synth.make_decode_case(list(lens), hq, hkv, d, 1, 1, dtype, seed=len(lens) * 7 + hq, std=std, cap_extra=3)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    out, lse = run_decode(cache, c.q[0, 0], c.scale)
    ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[0, 0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                     c.seq_start.numpy(), c.seq_len.numpy(), c.scale)
    e = parity.check(out, ref, dtype, discriminating=std >= 1.0, what="decode out")
    parity.check_lse(lse, ref_lse, dtype, what="decode lse")
    say(f"  max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


def test_decode_empty_sequence():
    say("decode with an empty sequence")
    c = synth.make_decode_case([0, 50], 8, 2, 128, 1, 1, "bf16", seed=3, std=1.0)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    out, lse = run_decode(cache, c.q[0, 0], c.scale)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[0, 0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                     c.seq_start.numpy(), c.seq_len.numpy(), c.scale)
    parity.check(out, ref, "bf16", discriminating=False)
    parity.check_lse(lse, ref_lse, "bf16")


def test_decode_max_kv_len_underestimate_still_exact():
    """max_kv_len is a sizing hint: the kernels count the rows themselves."""
    say("decode with an under-estimated max_kv_len")
    c = synth.make_decode_case([3000], 16, 2, 128, 1, 1, "bf16", seed=4, std=1.0)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    out, _ = run_decode(cache, c.q[0, 0], c.scale, max_kv_len=700, total_kv_len=0)
    ref, _ = oracle.decode_ref(synth.to_f64(c.q[0, 0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                               c.seq_start.numpy(), c.seq_len.numpy(), c.scale)
    parity.check(out, ref, "bf16", discriminating=True)


_MIXED = (0, 5, 129, 0, 0, 300, 1, 128, 127, 0, 7000, 256, 2)
_MANY = tuple(int(x) for x in np.random.default_rng(5).integers(0, 400, size=100))


@pytest.mark.parametrize("lens,hints,dtype", [
    (_MIXED, "true", "bf16"),       # one block per share, empty sequences between
    (_MIXED, "under", "bf16"),      # one share for everything: a share spans every sequence
    (_MIXED, "over", "bf16"),       # far more shares than blocks: most shares empty
    (_MANY, "true", "bf16"),        # 100 sequences: the block count runs over two scan chunks
    (_MANY, "under", "bf16"),
    (_MIXED, "under", "f32"),
    (_MIXED, "over", "f32"),
])
def test_decode_balanced_shares(lens, hints, dtype):
    """The balanced split: shares of equal block counts over all sequences,
    whatever the hints say, with every sequence's pieces merged exactly."""
    say(f"decode balanced shares {dtype} hints={hints} B={len(lens)}")
    c = synth.make_decode_case(list(lens), 16, 2, 128, 1, 1, dtype, seed=len(lens), std=1.0, cap_extra=2)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    mx, tot = max(lens), sum(lens)
    kw = {"true": dict(max_kv_len=mx, total_kv_len=tot), "under": dict(max_kv_len=1, total_kv_len=1),
          "over": dict(max_kv_len=200000, total_kv_len=0)}[hints]
    out, lse = run_decode(cache, c.q[0, 0], c.scale, **kw)
    ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[0, 0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                     c.seq_start.numpy(), c.seq_len.numpy(), c.scale)
    empty = np.array(lens) == 0
    assert np.all(out[empty] == 0.0) and np.all(np.isneginf(lse[empty]))
    parity.check(out[~empty], ref[~empty], dtype, discriminating=True, what="decode out")
    parity.check_lse(lse, ref_lse, dtype, what="decode lse")


# --------------------------------------------------------------------------- append


@pytest.mark.parametrize("dtype,hkv,d", [
    ("bf16", 2, 64),
    ("f32", 2, 64),
    ("bf16", 16, 128),   # 4 KB rows: one 16-byte piece per thread
    ("f32", 24, 128),    # 12 KB rows: three pieces per thread
])
def test_append_writes_row_and_flags_overflow(dtype, hkv, d):
    say(f"kv_append {dtype} hkv={hkv} d={d}")
    c = synth.make_decode_case([5, 9, 2], 4 * hkv if hkv < 8 else hkv, hkv, d, 1, 1, dtype, seed=11 + hkv, std=1.0)
    cap = c.seq_cap.clone()
    cap[1] = 9   # sequence 1 is full
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, cap)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    import decoder_shared_kv_amd as dk
    dk.kv_append(cache, c.k_new[0].to(DEV), c.v_new[0].to(DEV), flag)
    torch.cuda.synchronize()
    kr, vr, lr, ov = oracle.kv_append_ref(synth.to_f64(c.k_pool), synth.to_f64(c.v_pool), c.seq_start.numpy(),
                                          c.seq_len.numpy(), cap.numpy(), synth.to_f64(c.k_new[0]),
                                          synth.to_f64(c.v_new[0]))
    assert cache.seq_len.cpu().tolist() == list(lr) and int(flag.item()) == ov == 1
    assert np.array_equal(f64(cache.k), kr) and np.array_equal(f64(cache.v), vr)


def test_tiny_f32_flow():
    """Tiny fp32 workload: rows 0..254 written directly, row 255 appended, then
    per layer a causal prefill over 256 rows and a decode of position 255."""
    w = synth.WORKLOADS["tiny_f32"]
    say("tiny fp32 flow")
    dc = synth.make_decode_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, w.layers, 1, "f32",
                                seed=w.seed, std=w.value_std)
    cache = device_cache(dc.k_pool, dc.v_pool, dc.seq_start, dc.seq_len, dc.seq_cap)
    import decoder_shared_kv_amd as dk
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dk.kv_append(cache, dc.k_new[0].to(DEV), dc.v_new[0].to(DEV), flag)
    kr, vr, lr, _ = oracle.kv_append_ref(synth.to_f64(dc.k_pool), synth.to_f64(dc.v_pool), dc.seq_start.numpy(),
                                         dc.seq_len.numpy(), dc.seq_cap.numpy(), synth.to_f64(dc.k_new[0]),
                                         synth.to_f64(dc.v_new[0]))
    torch.cuda.synchronize()
    assert int(flag.item()) == 0 and cache.seq_len.cpu().tolist() == [256]
    pc = synth.make_prefill_case([256], w.q_heads, w.kv_heads, w.head_dim, w.layers, "f32", seed=w.seed + 100,
                                 std=w.value_std)
    for layer in range(w.layers):
        q = pc.q[layer]
        pcl = synth.PrefillCase([q], None, None, dc.seq_start, None, None, pc.cu_seqlens, w.scale, "f32")
        out, lse = run_prefill(pcl, cache=cache)
        ref, ref_lse = oracle.prefill_ref(synth.to_f64(q), kr, vr, dc.seq_start.numpy(), lr, pc.cu_seqlens.numpy(),
                                          w.scale)
        parity.check(out, ref, "f32", discriminating=True, what=f"tiny prefill layer {layer}")
        parity.check_lse(lse, ref_lse, "f32")
        od, ld = run_decode(cache, q[255:256], w.scale)
        refd, refl = oracle.decode_ref(synth.to_f64(q[255:256]), kr, vr, dc.seq_start.numpy(), lr, w.scale)
        parity.check(od, refd, "f32", discriminating=True, what=f"tiny decode layer {layer}")
        parity.check_lse(ld, refl, "f32")
        assert np.max(np.abs(od[0] - out[255])) <= 1e-5
