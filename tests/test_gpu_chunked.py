"""Chunked prefill / multi-token decode: m new query rows per sequence against a
shared cache of n >= m rows (queries at the last m positions), and the m > n
corner (rows at positions n and later have no cache row of their own and get
O = 0, LSE = -inf), against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import parity
import synth
from gpu_util import run_prefill, say

pytestmark = pytest.mark.gpu


def _ref(c):
    return oracle.prefill_ref(synth.to_f64(c.q[0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                              c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale)


@pytest.mark.parametrize("kv,qn,hq,hkv,d,dtype", [
    ((1000, 257, 64), (100, 1, 64), 16, 4, 128, "bf16"),
    ((3000,), (200,), 16, 2, 128, "bf16"),        # g = 8, chunk spans several tiles with a ragged tail
    ((777, 90), (33, 90), 6, 3, 64, "bf16"),       # head_dim 64, g = 2
    ((50,), (80,), 8, 2, 128, "bf16"),             # more query rows than cache rows
    ((20, 100), (90, 30), 4, 2, 64, "bf16"),       # m > n beside a plain chunk; whole waves without rows
    ((30,), (45,), 4, 1, 64, "f32"),               # m > n, fp32 path
    ((300, 40), (17, 40), 4, 1, 64, "f32"),
])
def test_chunked_prefill(kv, qn, hq, hkv, d, dtype):
    say(f"chunked prefill {dtype} kv={kv} q={qn} hq={hq} hkv={hkv} d={d}")
    c = synth.make_chunk_case(list(kv), list(qn), hq, hkv, d, dtype, seed=sum(kv) + sum(qn), std=1.0, cap_extra=3)
    out, lse = run_prefill(c)
    ref, ref_lse = _ref(c)
    missing = np.isneginf(ref_lse)
    assert np.all(np.isneginf(lse[missing])), "rows without their own cache row: LSE = -inf"
    e = parity.check(out, ref, dtype, discriminating=True, what="chunked prefill")
    parity.check_lse(lse, ref_lse, dtype, what="chunked prefill lse")
    say(f"  max-abs {e['max_abs']:.2e} row-rel {e['row_rel']:.2e}")


def test_chunk_equals_last_rows_of_full_prefill():
    """The same query rows give the same result as a chunk or as the tail of a prompt."""
    say("chunk = tail of the full prefill")
    n, m = 1500, 130
    full = synth.make_prefill_case([n], 16, 4, 128, 1, "bf16", seed=31, std=1.0)
    out_full, lse_full = run_prefill(full)
    chunk = synth.PrefillCase([full.q[0][n - m:].contiguous()], full.k_pool, full.v_pool, full.seq_start,
                              full.seq_len, full.seq_cap, torch.tensor([0, m], dtype=torch.int32),
                              full.scale, "bf16")
    out_c, lse_c = run_prefill(chunk)
    assert np.array_equal(out_c, out_full[n - m:]) or parity.errors(out_c, out_full[n - m:])["row_rel"] < 1e-2
    assert np.max(np.abs(lse_c - lse_full[:, n - m:])) < 1e-4
