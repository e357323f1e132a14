"""The shared cache's producer through the C ABI against the fp64 oracle:
RMSNorm(X) [W_K | W_V] appended to each sequence's rows, with and without the
YOCO++ residual, prompt-sized chunks and one row per sequence (decode), ragged
row counts, a sequence that does not fit, and the 3B geometry at 32K rows."""
import numpy as np
import pytest
import torch

import decoder_shared_kv_amd as dk
import oracle
import parity
import synth
from gpu_util import DEV, f64, say

pytestmark = pytest.mark.gpu


def _setup(lens_before, caps, chunks, hkv, d, d_model, seed, gain_std=0.1):
    g = torch.Generator().manual_seed(seed)
    B = len(caps)
    starts = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(sum(caps)) + 3
    kp = torch.randn(rows, hkv, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(rows, hkv, d, generator=g).to(torch.bfloat16)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    T = int(cu[-1])
    x = torch.randn(T, d_model, generator=g).to(torch.bfloat16)
    gain = (1.0 + gain_std * torch.randn(d_model, generator=g)).to(torch.bfloat16)
    wk = (torch.randn(d_model, hkv * d, generator=g) / d_model ** 0.5).to(torch.bfloat16)
    wv = (torch.randn(d_model, hkv * d, generator=g) / d_model ** 0.5).to(torch.bfloat16)
    cache = dk.SharedKV(kp.to(DEV), vp.to(DEV), torch.from_numpy(starts).to(DEV),
                        torch.tensor(lens_before, dtype=torch.int32, device=DEV),
                        torch.tensor(caps, dtype=torch.int32, device=DEV))
    host = dict(kp=kp, vp=vp, starts=starts, lens=np.array(lens_before), caps=np.array(caps), cu=cu, x=x, gain=gain,
                wk=wk, wv=wv)
    return cache, host


def _run(cache, host, hkv, d, eps, residual=None):
    wp = dk.kv_project_pack(host["gain"].to(DEV), host["wk"].to(DEV), host["wv"].to(DEV), hkv, d)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    res = None
    if residual is not None:
        res = dict(residual, k1=residual["k1"].to(DEV), v1=residual["v1"].to(DEV))
    dk.kv_project_append(cache, host["x"].to(DEV), torch.from_numpy(host["cu"]).to(DEV), wp, eps, res, flag)
    torch.cuda.synchronize()
    return flag


def _ref(host, eps, residual=None):
    comb = None
    if residual is not None:
        comb = {"k1": synth.to_f64(residual["k1"]), "v1": synth.to_f64(residual["v1"]), "ak": residual["a_k"],
                "av": residual["a_v"], "lam": residual["lam"]}
    return oracle.project_append_ref(synth.to_f64(host["kp"]), synth.to_f64(host["vp"]), host["starts"], host["lens"],
                                     host["caps"], host["cu"], synth.to_f64(host["x"]), synth.to_f64(host["gain"]),
                                     synth.to_f64(host["wk"]), synth.to_f64(host["wv"]), eps, comb)


def _compare(cache, host, ref, what):
    k_ref, v_ref, lens_ref, flag_ref = ref
    k, v = f64(cache.k), f64(cache.v)
    lens = cache.seq_len.cpu().numpy()
    assert list(lens) == list(lens_ref), (what, lens, lens_ref)
    written = np.zeros(k.shape[0], dtype=bool)
    for b in range(len(lens)):
        s0 = int(host["starts"][b])
        written[s0 + int(host["lens"][b]):s0 + int(lens_ref[b])] = True
    # rows not written stay bitwise as they were
    assert np.array_equal(k[~written], synth.to_f64(host["kp"])[~written]), what
    assert np.array_equal(v[~written], synth.to_f64(host["vp"])[~written]), what
    if written.any():
        e = parity.check(k[written], k_ref[written], "bf16", discriminating=True, what=what + " K")
        parity.check(v[written], v_ref[written], "bf16", discriminating=True, what=what + " V")
        say(f"  {what}: {int(written.sum())} rows, K row-rel {e['row_rel']:.2e}")
    return flag_ref


@pytest.mark.parametrize("lens_before,caps,chunks,hkv,d,d_model", [
    ([0, 0], [400, 100], [300, 77], 8, 128, 512),        # two prompts, ragged tail of a 256-row tile
    ([5, 17, 0], [700, 40, 300], [600, 20, 257], 2, 128, 1024),
    ([0], [64], [64], 1, 64, 192),                       # K and V halves inside one 128-column tile
    ([3, 9, 100, 0, 1, 2, 7, 8], [200] * 8, [1] * 8, 8, 128, 3072),   # decode: one row per sequence
    ([0], [50], [1], 2, 64, 320),                        # a single row
    ([2, 0], [40, 40], [9, 7], 4, 128, 448),             # 16 rows: the few-rows kernel's limit
    ([2, 0], [40, 40], [9, 8], 4, 128, 448),             # 17 rows: the tiled kernel
])
def test_project_append(lens_before, caps, chunks, hkv, d, d_model):
    say(f"producer lens={lens_before} chunks={chunks} hkv={hkv} d={d} d_model={d_model}")
    cache, host = _setup(lens_before, caps, chunks, hkv, d, d_model, seed=sum(chunks) + d_model)
    flag = _run(cache, host, hkv, d, 1e-6)
    flag_ref = _compare(cache, host, _ref(host, 1e-6), "project")
    assert int(flag.item()) == flag_ref == 0


def test_sequence_that_does_not_fit():
    say("producer: sequence 1 has no room for its chunk")
    cache, host = _setup([10, 30, 0], [100, 40, 50], [50, 11, 40], 4, 128, 256, seed=3)
    flag = _run(cache, host, 4, 128, 1e-5)
    flag_ref = _compare(cache, host, _ref(host, 1e-5), "overflow")
    assert int(flag.item()) == 1 and flag_ref == 1


@pytest.mark.parametrize("a_k,a_v,chunks", [((0.0, 1.0 / 35.0), (0.0, 1.0 / 35.0), [513, 130]),
                                             ((0.01, 0.02), (-0.03, 0.025), [513, 130]),
                                             ((0.01, 0.02), (-0.03, 0.025), [1, 1])])
def test_yoco_pp_residual(a_k, a_v, chunks):
    say(f"producer with YOCO++ residual a_k={a_k} a_v={a_v} chunks={chunks}")
    cache, host = _setup([0, 4], [600, 300], chunks, 8, 128, 768, seed=11)
    g = torch.Generator().manual_seed(12)
    T = int(host["cu"][-1])
    residual = {"k1": torch.randn(T, 8 * 128, generator=g).to(torch.bfloat16),
                "v1": torch.randn(T, 8 * 128, generator=g).to(torch.bfloat16), "lam": 35.0, "a_k": a_k, "a_v": a_v}
    _run(cache, host, 8, 128, 1e-6, residual)
    _compare(cache, host, _ref(host, 1e-6, residual), "yoco++")


def test_project_32k_sampled():
    """The YOCO-3B geometry (d_model 3072, 8 KV heads of 128) over a 32K-row prompt."""
    say("producer 32K rows, d_model 3072, Hkv 8")
    T, hkv, d, dm = 32768, 8, 128, 3072
    cache, host = _setup([0], [T], [T], hkv, d, dm, seed=7)
    flag = _run(cache, host, hkv, d, 1e-6)
    assert int(flag.item()) == 0 and int(cache.seq_len.item()) == T
    rng = np.random.default_rng(5)
    rows = np.array(sorted(set([0, 1, 255, 256, 32767] + list(rng.integers(0, T, 60)))))
    k_ref, v_ref = oracle.kv_project_ref(synth.to_f64(host["x"][rows]), synth.to_f64(host["gain"]),
                                         synth.to_f64(host["wk"]), synth.to_f64(host["wv"]), 1e-6)
    idx = torch.from_numpy(rows).to(DEV)
    k = f64(cache.k[idx]).reshape(len(rows), -1)
    v = f64(cache.v[idx]).reshape(len(rows), -1)
    parity.check(k.reshape(-1, hkv, d), k_ref.reshape(-1, hkv, d), "bf16", discriminating=True, what="32K K")
    parity.check(v.reshape(-1, hkv, d), v_ref.reshape(-1, hkv, d), "bf16", discriminating=True, what="32K V")


def test_decode_after_produce_matches_oracle_chain():
    """Produce a prompt's rows, then decode against them: the full chain against
    the oracle's chain (projection, then attention)."""
    cache, host = _setup([0], [300], [300], 2, 128, 256, seed=21)
    _run(cache, host, 2, 128, 1e-6)
    k_ref, v_ref, lens_ref, _ = _ref(host, 1e-6)
    q = torch.randn(1, 8, 128, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    ws = dk.alloc_workspace(cache, 8, 300)
    out = dk.xattn_decode(cache, q.to(DEV), 300, 128 ** -0.5, ws)
    torch.cuda.synchronize()
    # the oracle attends to the oracle's own (unrounded) rows: the chain's tolerance covers the rounding
    ref, _ = oracle.decode_ref(synth.to_f64(q), k_ref, v_ref, [0], [300], 128 ** -0.5)
    parity.check(f64(out), ref, "bf16", discriminating=True, what="produce + decode")
