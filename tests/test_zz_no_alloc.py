"""The decode entry point that allocates nothing (its partials live in the
library's device-resident scratch) against the workspace entry point, through
the C ABI: two calls in a row, the second with a smaller input, each equal to
yoco_xattn_decode's result on the same inputs (same kernels, same plan, so
bitwise), and both within the bf16 parity bound of the fp64 oracle."""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import oracle
import parity
import synth
from gpu_util import DEV, device_cache, f64, say

pytestmark = pytest.mark.gpu


def _case(lens, hq, hkv, d, dtype, seed):
    c = synth.make_decode_case(list(lens), hq, hkv, d, 1, 1, dtype, seed, 1.0)
    cache = device_cache(c.k_pool, c.v_pool, c.seq_start, c.seq_len, c.seq_cap)
    return c, cache


def _both(c, cache, max_len, total):
    q = c.q[0, 0].to(DEV).contiguous()
    ws = dk.alloc_workspace(cache, q.shape[1], max_len)
    out_ws = torch.empty_like(q)
    lse_ws = torch.empty(q.shape[:2], device=DEV, dtype=torch.float32)
    dk.xattn_decode(cache, q, max_len, c.scale, ws, out=out_ws, lse=lse_ws, total_kv_len=total)
    out_na = torch.full_like(q, float("nan"))
    lse_na = torch.full(q.shape[:2], float("nan"), device=DEV, dtype=torch.float32)
    dk.xattn_decode_noalloc(cache, q, max_len, c.scale, out_na, lse=lse_na, total_kv_len=total)
    torch.cuda.synchronize()
    return f64(out_ws), f64(lse_ws), f64(out_na), f64(lse_na)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 16, 2, 128), ("bf16", 32, 8, 128), ("f32", 4, 1, 64)])
def test_noalloc_decode_matches_workspace_decode(dtype, hq, hkv, d):
    # first call: several sequences of some thousand rows; second: fewer, shorter
    # sequences, so stale partials of the first call would show if misused
    for lens, seed in (((5000, 1234, 777, 3000), 11), ((300, 5), 12)):
        say(f"noalloc decode {dtype} hq={hq} hkv={hkv} d={d} lens={lens}")
        c, cache = _case(lens, hq, hkv, d, dtype, seed)
        n = int(max(lens))
        o_ws, l_ws, o_na, l_na = _both(c, cache, n, int(sum(lens)))
        assert np.array_equal(o_ws, o_na), "outputs differ from the workspace entry point"
        assert np.array_equal(l_ws, l_na), "LSE differs from the workspace entry point"
        ref, ref_lse = oracle.decode_ref(synth.to_f64(c.q[0, 0]), synth.to_f32(c.k_pool), synth.to_f32(c.v_pool),
                                         c.seq_start.numpy(), c.seq_len.numpy(), c.scale)
        e = parity.check(o_na, ref, dtype, discriminating=True, what="noalloc decode")
        parity.check_lse(l_na, ref_lse, dtype, what="noalloc decode lse")
        say(f"  equal to the workspace call; row-rel {e['row_rel']:.2e}")


def test_noalloc_rejects_plans_beyond_its_scratch():
    """Too many sequences: the call returns the workspace error and leaves out untouched."""
    say("noalloc decode beyond the scratch")
    b, hq, hkv, d = 1024, 32, 8, 128
    k = torch.zeros(b * 8, hkv, d, dtype=torch.bfloat16, device=DEV)
    cache = dk.SharedKV(k, k.clone(), torch.arange(b, dtype=torch.int64, device=DEV) * 8,
                        torch.full((b,), 8, dtype=torch.int32, device=DEV),
                        torch.full((b,), 8, dtype=torch.int32, device=DEV))
    assert dk.workspace_size(b, hq, hkv, d, torch.bfloat16, 1 << 20) > dk.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(b, hq, d, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(dk.YocoError) as ei:
        dk.xattn_decode_noalloc(cache, q, 1 << 20, 0.1, out)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
