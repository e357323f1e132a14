"""Gated retention through the C ABI against the fp64 oracle: chunkwise prefill
(packed sequences, partial chunks, head_dim 64 and 128, with and without an
initial state, gates that close completely), the final states, recurrent
decode steps, and the chain prefill -> decode."""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import oracle
import parity
import synth
from gpu_util import DEV, f64, say

pytestmark = pytest.mark.gpu


def _inputs(lens, heads, d, seed, with_state):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(lens))
    std = d ** -0.25                      # q.k ~ N(0, 1): unit-spread scores
    q = (torch.randn(T, heads, d, generator=g) * std).to(torch.bfloat16)
    k = (torch.randn(T, heads, d, generator=g) * std).to(torch.bfloat16)
    v = torch.randn(T, heads, d, generator=g).to(torch.bfloat16)
    gam = 0.8 + 0.2 * torch.rand(T, heads, generator=g)
    gam[torch.rand(T, heads, generator=g) < 0.05] = 1.0
    gam[torch.rand(T, heads, generator=g) < 0.02] = 0.01
    if T > 40:
        gam[37, 0] = 0.0                  # a gate that closes completely
    s0 = torch.randn(len(lens), heads, d, d, generator=g) * 0.1 if with_state else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return q, k, v, gam.float(), s0, cu


def _state_check(st, ref, what):
    err = np.abs(st - ref).reshape(st.shape[0] * st.shape[1], -1).max(axis=1)
    mag = np.abs(ref).reshape(ref.shape[0] * ref.shape[1], -1).max(axis=1)
    rel = float((err / np.maximum(mag, 1e-30)).max())
    assert rel <= 1e-2, f"{what}: state relative error {rel:.3e}"
    return rel


def _run_prefill(q, k, v, gam, s0, cu, lens):
    heads, d = q.shape[1], q.shape[2]
    ws = torch.empty(dk.gret_workspace_size(len(lens), heads, d, sum(lens)), dtype=torch.uint8, device=DEV)
    st = torch.full((len(lens), heads, d, d), float("nan"), device=DEV)
    out = dk.gret_prefill(q.to(DEV), k.to(DEV), v.to(DEV), gam.to(DEV), cu.to(DEV), ws,
                          state_in=None if s0 is None else s0.to(DEV), state_out=st)
    torch.cuda.synchronize()
    return f64(out), st.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("lens,heads,d,with_state", [
    ([1000], 4, 128, False),            # 3 full chunks and a partial one
    ([256, 300, 17], 2, 128, True),     # a whole chunk, a chunk and a bit, a tiny one
    ([700], 3, 64, True),               # head_dim 64
    ([5000, 1234], 4, 128, True),
    ([3, 600, 0, 257, 1, 90] * 11 + [1300], 2, 128, True),   # 67 sequences (a wave's chunk count and more),
                                                              # empty and one-row sequences
])
def test_gret_prefill(lens, heads, d, with_state):
    say(f"gret prefill lens={lens} H={heads} d={d} state={with_state}")
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=sum(lens) + d, with_state=with_state)
    out, st = _run_prefill(q, k, v, gam, s0, cu, lens)
    ref, ref_st = oracle.gret_prefill_ref(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), gam.double().numpy(),
                                          cu.numpy(), None if s0 is None else s0.double().numpy())
    e = parity.check(out, ref, "bf16", discriminating=True, what="gret prefill")
    rel = _state_check(st, ref_st, "gret prefill")
    say(f"  out row-rel {e['row_rel']:.2e}, state rel {rel:.2e}")


# Inputs long enough (chunks x heads >= 512) that the library groups 2 or 8
# chunks per segment: segments that end mid-sequence, partial segments at
# sequence ends, one-chunk sequences, initial states carried into later
# segments. Heads are checked in a subset at the larger size to keep the fp64
# oracle within seconds.
@pytest.mark.parametrize("lens,heads,d,check_heads", [
    ([5000, 1234, 7000, 300], 16, 128, None),          # 2 chunks per segment
    ([20000, 3000], 8, 64, None),                     # head_dim 64, 2 chunks per segment
    ([9000, 300, 17000, 6468], 16, 128, [0, 7, 15]),  # 8 chunks per segment
    ([0, 9000, 1, 4500, 0, 300], 16, 128, [0, 5, 15]),  # 2 chunks per segment, empty and one-row sequences
])
def test_gret_prefill_segments(lens, heads, d, check_heads):
    say(f"gret prefill over multi-chunk segments lens={lens} H={heads} d={d}")
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=len(lens) + heads + d, with_state=True)
    out, st = _run_prefill(q, k, v, gam, s0, cu, lens)
    sel = list(range(heads)) if check_heads is None else check_heads
    # the fp64 recurrence, row by row (the parallel form's decay matrix is
    # quadratic in Python loops at these lengths)
    ref = np.zeros((q.shape[0], len(sel), d))
    ref_st = np.zeros((len(lens), len(sel), d, d))
    qf, kf, vf = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    for b in range(len(lens)):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        for i, h in enumerate(sel):
            ref[r0:r1, i], ref_st[b, i] = oracle.gret_recurrent_ref(qf[r0:r1, h], kf[r0:r1, h], vf[r0:r1, h],
                                                                    gam[r0:r1, h].double().numpy(),
                                                                    s0[b, h].double().numpy())
    e = parity.check_signed_sum(out[:, sel], ref, "bf16", what="gret prefill, segments")
    rel = _state_check(st[:, sel], ref_st, "gret prefill, segments")
    say(f"  out row-rel {e['row_rel']:.2e} (99.9th percentile {e['row_rel_p999']:.2e}), state rel {rel:.2e}")


def test_gret_decode_steps():
    say("gret decode: 5 recurrent steps from a prefill's state")
    lens, heads, d = [300, 77, 1], 4, 128
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=3, with_state=True)
    _, st_ref = oracle.gret_prefill_ref(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), gam.double().numpy(),
                                        cu.numpy(), s0.double().numpy())
    state = torch.from_numpy(st_ref.astype(np.float32)).to(DEV)
    cur = st_ref.astype(np.float32).astype(np.float64)
    g = torch.Generator().manual_seed(4)
    for step in range(5):
        qd = (torch.randn(3, heads, d, generator=g) * d ** -0.25).to(torch.bfloat16)
        kd = (torch.randn(3, heads, d, generator=g) * d ** -0.25).to(torch.bfloat16)
        vd = torch.randn(3, heads, d, generator=g).to(torch.bfloat16)
        gd = (0.8 + 0.2 * torch.rand(3, heads, generator=g)).float()
        out = dk.gret_decode(qd.to(DEV), kd.to(DEV), vd.to(DEV), gd.to(DEV), state)
        torch.cuda.synchronize()
        ref, cur = oracle.gret_decode_ref(synth.to_f64(qd), synth.to_f64(kd), synth.to_f64(vd), gd.double().numpy(),
                                          cur)
        parity.check(f64(out), ref, "bf16", discriminating=True, what=f"gret decode step {step}")
        err = np.abs(state.cpu().numpy() - cur).max() / np.abs(cur).max()
        assert err <= 1e-5, f"decode state step {step}: {err:.2e}"   # the step is fp32 throughout


@pytest.mark.parametrize("batch,heads,d", [
    (8, 16, 128),    # the decode benchmark's shape
    (5, 3, 64),      # head_dim 64
    (1, 1, 128),
])
def test_gret_decode_shapes(batch, heads, d):
    say(f"gret decode B={batch} H={heads} d={d}: two steps from a random state")
    g = torch.Generator().manual_seed(batch * 100 + heads + d)
    st0 = torch.randn(batch, heads, d, d, generator=g) * 0.3
    state = st0.to(DEV)
    cur = st0.double().numpy()
    for step in range(2):
        qd = (torch.randn(batch, heads, d, generator=g) * d ** -0.25).to(torch.bfloat16)
        kd = (torch.randn(batch, heads, d, generator=g) * d ** -0.25).to(torch.bfloat16)
        vd = torch.randn(batch, heads, d, generator=g).to(torch.bfloat16)
        gd = (0.5 + 0.5 * torch.rand(batch, heads, generator=g)).float()
        out = dk.gret_decode(qd.to(DEV), kd.to(DEV), vd.to(DEV), gd.to(DEV), state)
        torch.cuda.synchronize()
        ref, cur = oracle.gret_decode_ref(synth.to_f64(qd), synth.to_f64(kd), synth.to_f64(vd), gd.double().numpy(),
                                          cur)
        parity.check(f64(out), ref, "bf16", discriminating=True, what=f"gret decode step {step}")
        err = np.abs(state.cpu().numpy() - cur).max() / np.abs(cur).max()
        assert err <= 1e-5, f"decode state step {step}: {err:.2e}"   # the step is fp32 throughout


def test_gret_prefill_then_decode_equals_longer_prefill():
    """Decode of row n from the state after rows 0..n-1 = row n of the prefill of n + 1 rows."""
    lens, heads, d = [513], 2, 128
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=8, with_state=False)
    out_full, st_full = _run_prefill(q, k, v, gam, None, cu, lens)
    n = 512
    _, st_n = _run_prefill(q[:n], k[:n], v[:n], gam[:n], None, torch.tensor([0, n], dtype=torch.int32), [n])
    state = torch.from_numpy(st_n.astype(np.float32)).to(DEV)
    out = dk.gret_decode(q[n:].to(DEV), k[n:].to(DEV), v[n:].to(DEV), gam[n:].to(DEV), state)
    torch.cuda.synchronize()
    assert parity.errors(f64(out), out_full[n:n + 1])["row_rel"] < 2e-2
    assert np.abs(state.cpu().numpy() - st_full).max() / np.abs(st_full).max() < 2e-2


def test_gret_state_passing_equals_one_call():
    lens, heads, d = [900], 2, 64
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=12, with_state=True)
    out_full, st_full = _run_prefill(q, k, v, gam, s0, cu, lens)
    a = 333
    out_a, st_a = _run_prefill(q[:a], k[:a], v[:a], gam[:a], s0, torch.tensor([0, a], dtype=torch.int32), [a])
    out_b, st_b = _run_prefill(q[a:], k[a:], v[a:], gam[a:], torch.from_numpy(st_a.astype(np.float32)),
                               torch.tensor([0, 900 - a], dtype=torch.int32), [900 - a])
    assert parity.errors(np.concatenate([out_a, out_b]), out_full)["row_rel"] < 2e-2
    assert np.abs(st_b - st_full).max() / np.abs(st_full).max() < 2e-2


def test_gret_32k_two_heads_against_recurrence():
    """A 32K-row sequence (128 chunks), heads checked against the fp64 recurrence."""
    say("gret prefill 32K rows, 16 heads; heads 0 and 9 against the fp64 recurrence")
    lens, heads, d = [32768], 16, 128
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=21, with_state=False)
    out, st = _run_prefill(q, k, v, gam, None, cu, lens)
    for h in (0, 9):
        ref, ref_st = oracle.gret_recurrent_ref(synth.to_f64(q[:, h]), synth.to_f64(k[:, h]), synth.to_f64(v[:, h]),
                                                gam[:, h].double().numpy())
        parity.check(out[:, h][:, None], ref[:, None], "bf16", discriminating=True, what=f"32K head {h}")
        _state_check(st[:1, h:h + 1], ref_st[None, None], f"32K head {h}")


def test_gret_128k_long_segments_against_recurrence():
    """131072 rows x 16 heads: 16 chunks per segment and more segments than
    CUs (two rounds of workgroups); heads 0 and 15 against the fp64 recurrence."""
    say("gret prefill 128K rows, 16 heads; heads 0 and 15 against the fp64 recurrence")
    lens, heads, d = [131072], 16, 128
    q, k, v, gam, s0, cu = _inputs(lens, heads, d, seed=34, with_state=True)
    out, st = _run_prefill(q, k, v, gam, s0, cu, lens)
    for h in (0, 15):
        ref, ref_st = oracle.gret_recurrent_ref(synth.to_f64(q[:, h]), synth.to_f64(k[:, h]), synth.to_f64(v[:, h]),
                                                gam[:, h].double().numpy(), s0[0, h].double().numpy())
        e = parity.check_signed_sum(out[:, h][:, None], ref[:, None], "bf16", what=f"128K head {h}")
        rel = _state_check(st[:1, h:h + 1], ref_st[None, None], f"128K head {h}")
        say(f"  head {h}: out row-rel {e['row_rel']:.2e} (99.9th percentile {e['row_rel_p999']:.2e}), state rel {rel:.2e}")
