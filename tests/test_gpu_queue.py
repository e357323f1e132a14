"""The bf16 prefill's work queue (a persistent grid taking items from per-XCD
queues) against the static grid and the fp64 oracle.

The queue changes only which workgroup computes an item, never its arithmetic,
so both launch forms must agree bitwise; both are also checked against the
oracle. Covered: each of the three item orders of the schedule (fewer units than
XCDs, a multiple of the XCD count with empty items of short sequences to skip,
neither), the sliding window, head_dim 64, a grid hint shorter than the longest
sequence (several passes per item), and the workspace left zero after every
call so that it can be reused as is.
"""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import oracle
import parity
import synth
from gpu_util import DEV, device_cache, f64, prefill_workspace, say

pytestmark = pytest.mark.gpu


def _run(c, queue, window=0, max_q=None):
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    q = c.q[0].to(DEV)
    lse = torch.full((q.shape[1], c.total_q), float("nan"), device=DEV)
    if max_q is None:
        max_q = int((c.cu_seqlens[1:] - c.cu_seqlens[:-1]).max())
    ws = prefill_workspace() if queue else None
    cu = c.cu_seqlens.to(DEV)
    if window:
        out = dk.xattn_prefill_window(cache, q, cu, max_q, window, c.scale, lse=lse, workspace=ws)
    else:
        out = dk.xattn_prefill(cache, q, cu, max_q, c.scale, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    if queue:
        assert int(torch.count_nonzero(ws)) == 0, "the work queue's counters are not back at zero"
    return f64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("lens,hq,hkv,d,window,max_q", [
    ((4096,), 16, 4, 128, 0, None),            # 4 units: each XCD pair shares one unit's blocks
    ((3000, 1, 1500, 64), 8, 2, 128, 0, None),  # 8 units: unit-major per XCD, empty items skipped
    ((700, 300), 6, 2, 128, 0, None),          # g = 3: 12 units, unit-major order
    ((2000, 300, 5000, 17), 8, 2, 128, 256, None),  # sliding window (shortest blocks first)
    ((900, 33), 8, 2, 64, 0, None),            # head_dim 64
    ((1000, 700), 8, 2, 128, 0, 100),          # grid hint of 100 rows: several passes per item
])
def test_queue_equals_static_grid_and_oracle(lens, hq, hkv, d, window, max_q):
    say(f"queue vs static: lens={lens} hq={hq} hkv={hkv} d={d} window={window} max_q={max_q}")
    c = synth.make_prefill_case(list(lens), hq, hkv, d, 1, "bf16", seed=sum(lens) + hq, std=1.0, cap_extra=3)
    o_q, l_q = _run(c, True, window, max_q)
    o_s, l_s = _run(c, False, window, max_q)
    assert np.array_equal(o_q, o_s), "queue and static grid differ"
    assert np.array_equal(l_q, l_s, equal_nan=True), "queue and static grid LSE differ"
    ref, ref_lse = oracle.prefill_ref(synth.to_f64(c.q[0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                      c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale,
                                      window=window)
    e = parity.check(o_q, ref, "bf16", discriminating=True, what="queue prefill")
    parity.check_lse(l_q, ref_lse, "bf16", what="queue prefill lse")
    say(f"  bitwise equal; row-rel {e['row_rel']:.2e}")


def test_queue_reused_back_to_back():
    """Five calls in a row on one workspace (without a synchronisation between
    them) give the same result as the first, and leave the counters at zero."""
    say("queue reused back to back")
    c = synth.make_prefill_case([2500, 800], 16, 4, 128, 1, "bf16", seed=77, std=1.0)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    q, cu = c.q[0].to(DEV), c.cu_seqlens.to(DEV)
    ws = dk.alloc_prefill_workspace(DEV)
    outs = [dk.xattn_prefill(cache, q, cu, 2500, c.scale, workspace=ws) for _ in range(5)]
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
