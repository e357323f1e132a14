"""The long-context decode suites can fail (CPU only; nothing here runs a kernel).

1. At every full-size decode workload, with the needle spacing the GPU tests
   use and the split plan the library computes for them, every share of the
   decode split holds needles of every checked query.
2. On a scaled-down copy of the 8-sequence workload, built the same way, the
   parity checker rejects the oracle's output with any one share's rows left
   out (and an all-zero output, and the wrong KV head), while the acceptance
   bound alone would pass such outputs on the acceptance inputs.
"""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import needles
import oracle.xattn as ox
import parity
import synth


def _plan(w, lens):
    shares, _ = dk.decode_splits(len(lens), w.q_heads, w.kv_heads, w.head_dim, torch.bfloat16, max(lens), sum(lens))
    return needles.share_rows(lens, shares)


@pytest.mark.parametrize("name,checked", [("decode_128k", 2), ("decode_1m", 4), ("ragged", 2)])
def test_every_share_holds_needles_of_every_checked_query(name, checked):
    w = synth.WORKLOADS[name]
    lens = [n + 1 for n in w.seq_lens]             # after the first append
    stride = needles.STRIDE[name]
    for pieces in _plan(w, lens):
        seen = set()
        for b, lo, hi in pieces:
            rows = needles.needle_rows(lens[b] - 1, stride)
            seen |= {i % checked for i, r in enumerate(rows) if lo <= r < hi}
        assert seen == set(range(checked)), (name, pieces)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.fixture(scope="module")
def small():
    """8 sequences of 4096 rows (after the append), Hq = 16, Hkv = 2, d = 128:
    the 8 x 131072 decode at 1/32 of its length with needles at 1/32 of its
    spacing, so that a share of the split (256 shares of one 128-row block)
    holds the same fraction of the rows and two needles per checked query, as
    a 4096-row share does at full size."""
    lens0 = [4095] * 8
    c = synth.make_decode_case(lens0, 16, 2, 128, 16, 1, "bf16", seed=41, std=128 ** -0.5)
    queries = [c.q[0, 0], c.q[0, 15]]
    needles.plant(c.k_pool, c.v_pool, c.seq_start.numpy(), lens0, queries, c.scale, stride=32, seed=42)
    kn, vn = needles.aligned_rows(c.q[0, 0], 2, c.scale, seed=43, dtype=torch.bfloat16)
    k, v, ln, _ = ox.kv_append_ref(synth.to_f64(c.k_pool), synth.to_f64(c.v_pool), c.seq_start.numpy(),
                                   c.seq_len.numpy(), c.seq_cap.numpy(), synth.to_f64(kn), synth.to_f64(vn))
    return c, k, v, ln


def _decode(c, k, v, ln, layer=0):
    return ox.decode_ref(synth.to_f64(c.q[0, layer]), k, v, c.seq_start.numpy(), ln, c.scale)


def test_needle_reference_is_large_and_a_simulated_kernel_passes(small):
    c, k, v, ln = small
    for layer in (0, 15):
        ref, _ = _decode(c, k, v, ln, layer)
        assert np.abs(ref).reshape(-1, 128).max(axis=1).min() > 0.05, "needle outputs are O(0.1)"
        parity.check(_bf16(ref), ref, "bf16", discriminating=True, what="rounded reference")


def test_dropping_any_share_is_rejected(small):
    c, k, v, ln = small
    ref, _ = _decode(c, k, v, ln)
    lens = [int(x) for x in ln]
    shares, _ = dk.decode_splits(8, 16, 2, 128, torch.bfloat16, max(lens), sum(lens))
    plan = needles.share_rows(lens, shares)
    assert len(plan) == 256
    starts = c.seq_start.numpy()
    for pieces in plan:
        keep = np.ones(k.shape[0], dtype=bool)
        drop_len = np.zeros(8, dtype=np.int64)
        for b, lo, hi in pieces:
            keep[starts[b] + lo:starts[b] + hi] = False
            drop_len[b] += hi - lo
        # the pool without the share's rows: later rows of each sequence move up
        new_start = np.array([int(np.count_nonzero(keep[:s])) for s in starts], dtype=np.int64)
        bad, _ = ox.decode_ref(synth.to_f64(c.q[0, 0]), k[keep], v[keep], new_start, ln - drop_len, c.scale)
        with pytest.raises(AssertionError):
            parity.check(_bf16(bad), ref, "bf16", discriminating=True, what=f"share {pieces}")


def test_zero_output_and_wrong_head_are_rejected_only_by_the_needles(small):
    c, k, v, ln = small
    ref, _ = _decode(c, k, v, ln)
    with pytest.raises(AssertionError):
        parity.check(np.zeros_like(ref), ref, "bf16", discriminating=True, what="zeros")
    ox_head = ox.kv_head_of
    try:
        ox.kv_head_of = lambda h, hq, hkv: (h // (hq // hkv) + 1) % hkv
        wrong, _ = _decode(c, k, v, ln)
    finally:
        ox.kv_head_of = ox_head
    with pytest.raises(AssertionError):
        parity.check(_bf16(wrong), ref, "bf16", discriminating=True, what="wrong KV head")
    # the same all-zero output passes the acceptance bound on the acceptance inputs
    plain = synth.make_decode_case([4095] * 8, 16, 2, 128, 1, 1, "bf16", seed=41, std=128 ** -0.5)
    pref, _ = ox.decode_ref(synth.to_f64(plain.q[0, 0]), synth.to_f64(plain.k_pool), synth.to_f64(plain.v_pool),
                            plain.seq_start.numpy(), plain.seq_len.numpy(), plain.scale)
    parity.check(np.zeros_like(pref), pref, "bf16", what="zeros on the acceptance inputs")
