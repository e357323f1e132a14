"""Seeded inputs are deterministic, shaped as the workloads say and rounded once."""
import math

import numpy as np
import torch

import synth


def test_same_seed_same_bits():
    a = synth.make_prefill_case([7, 5], 4, 2, 16, 2, "bf16", seed=5, std=0.3)
    b = synth.make_prefill_case([7, 5], 4, 2, 16, 2, "bf16", seed=5, std=0.3)
    for x, y in [(a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.q[0], b.q[0]), (a.q[1], b.q[1])]:
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = synth.make_prefill_case([7, 5], 4, 2, 16, 2, "bf16", seed=6, std=0.3)
    assert not torch.equal(a.k_pool, c.k_pool)


def test_layout_and_offsets():
    c = synth.make_prefill_case([3, 9, 4], 6, 3, 8, 1, "f32", seed=0, std=1.0, cap_extra=2)
    assert c.k_pool.shape == (3 + 9 + 4 + 6, 3, 8)
    assert c.seq_start.tolist() == [0, 5, 16] and c.seq_cap.tolist() == [5, 11, 6]
    assert c.cu_seqlens.tolist() == [0, 3, 12, 16] and c.q[0].shape == (16, 6, 8)
    assert c.seq_start.dtype == torch.int64 and c.seq_len.dtype == torch.int32
    d = synth.make_decode_case([4, 2], 8, 2, 16, 3, 5, "bf16", seed=1, std=1.0)
    assert d.seq_cap.tolist() == [9, 7] and d.q.shape == (5, 3, 2, 8, 16) and d.k_new.shape == (5, 2, 2, 16)


def test_bf16_rounding_is_round_to_nearest_even_of_fp32_draw():
    c = synth.make_prefill_case([64], 2, 1, 32, 1, "bf16", seed=2, std=0.25)
    rng = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(2).spawn(8)]
    x = rng[0].standard_normal((64, 1, 32), dtype=np.float32) * np.float32(0.25)
    bits = x.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(c.k_pool.view(torch.int16).numpy().view(np.uint16), rne)


def test_workloads():
    w = synth.WORKLOADS
    assert w["prefill_32k"].seq_lens == (32768,) and w["prefill_32k"].group == 4
    assert w["decode_128k"].seq_lens[0] + w["decode_128k"].decode_steps == 131072
    assert w["decode_1m"].seq_lens == (1048576,) and w["decode_1m"].decode_steps == 64
    lens = w["ragged"].seq_lens
    assert len(lens) == 16 and all(4096 <= n < 65536 for n in lens)
    assert math.isclose(w["decode_128k"].scale, 128 ** -0.5)
