"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Every mutation replaces one step of the oracle with a plausible wrong version:
a wrong head map, an off-by-one or missing causal limit, a dropped or doubled
scale, a sign flip, a transposed operand, a missing normalisation, a dropped
max term in the LSE, a wrong decode or prefill position, an append at the wrong
row or without the overflow check, a window one row too wide or too narrow,
ignored or aligned to fixed blocks, a ring append into the wrong slot or
without wrap-around, an RMSNorm with sum for mean, eps outside the root, no or
early gain, K and V weights swapped, the YOCO++ weights swapped or lambda
dropped, projected rows appended at the sequence start or partially; a gRet
decay that includes the row's own gate or drops the diagonal, a recurrence
that decays the new term or reads the state before the update, a chunkwise
carry without the decay into the row, an initial state not decayed by the
first gate.
"""
import numpy as np
import pytest

import oracle.gret as og
import oracle.producer as op
import oracle.xattn as ox
import pinlib


def _append_wrong_row(k_pool, v_pool, seq_start, seq_len, seq_cap, k_new, v_new):
    k2, v2 = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    ov = 0
    for b in range(len(lens)):
        if lens[b] >= int(seq_cap[b]):
            ov = 1
            continue
        row = int(seq_start[b]) + int(lens[b]) - 1
        k2[row], v2[row] = k_new[b], v_new[b]
        lens[b] += 1
    return k2, v2, lens, ov


def _append_no_cap(k_pool, v_pool, seq_start, seq_len, seq_cap, k_new, v_new):
    k2, v2 = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    for b in range(len(lens)):
        row = int(seq_start[b]) + int(lens[b])
        k2[row], v2[row] = k_new[b], v_new[b]
        lens[b] += 1
    return k2, v2, lens, 0


def _ring_slot_shift(k_ring, v_ring, seq_start, seq_len, seq_cap, k_new, v_new):
    k2, v2 = np.array(k_ring, copy=True), np.array(v_ring, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    flag = 0
    for b in range(len(lens)):
        cap = int(seq_cap[b])
        if cap <= 0:
            flag = 1
            continue
        row = int(seq_start[b]) + (int(lens[b]) + 1) % cap
        k2[row], v2[row] = k_new[b], v_new[b]
        lens[b] += 1
    return k2, v2, lens, flag


def _ring_no_wrap(k_ring, v_ring, seq_start, seq_len, seq_cap, k_new, v_new):
    k2, v2 = np.array(k_ring, copy=True), np.array(v_ring, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    flag = 0
    for b in range(len(lens)):
        cap = int(seq_cap[b])
        if cap <= 0:
            flag = 1
            continue
        row = int(seq_start[b]) + min(int(lens[b]), cap - 1)
        k2[row], v2[row] = k_new[b], v_new[b]
        lens[b] += 1
    return k2, v2, lens, flag


def _rms_sum_not_mean(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gamma


def _rms_eps_outside(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * gamma


def _rms_no_gain(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rms_gain_first(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64) * gamma
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _project_swapped(x, gamma, w_k, w_v, eps, combine=None):
    y = op.rmsnorm_ref(x, gamma, eps)
    return y @ np.asarray(w_v, dtype=np.float64), y @ np.asarray(w_k, dtype=np.float64)


def _append_chunk_at_start(k_pool, v_pool, seq_start, seq_len, seq_cap, cu, x, gamma, w_k, w_v, eps, combine=None):
    hkv, d = k_pool.shape[1], k_pool.shape[2]
    k, v = op.kv_project_ref(x, gamma, w_k, w_v, eps, combine)
    k2, v2 = np.array(k_pool, dtype=np.float64), np.array(v_pool, dtype=np.float64)
    lens = np.array(seq_len, dtype=np.int64)
    flag = 0
    for b in range(len(lens)):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if lens[b] + r1 - r0 > int(seq_cap[b]):
            flag = 1
            continue
        base = int(seq_start[b])
        k2[base:base + r1 - r0] = k[r0:r1].reshape(-1, hkv, d)
        v2[base:base + r1 - r0] = v[r0:r1].reshape(-1, hkv, d)
        lens[b] += r1 - r0
    return k2, v2, lens, flag


def _append_partial_chunk(k_pool, v_pool, seq_start, seq_len, seq_cap, cu, x, gamma, w_k, w_v, eps, combine=None):
    hkv, d = k_pool.shape[1], k_pool.shape[2]
    k, v = op.kv_project_ref(x, gamma, w_k, w_v, eps, combine)
    k2, v2 = np.array(k_pool, dtype=np.float64), np.array(v_pool, dtype=np.float64)
    lens = np.array(seq_len, dtype=np.int64)
    flag = 0
    for b in range(len(lens)):
        for r in range(int(cu[b]), int(cu[b + 1])):
            if lens[b] >= int(seq_cap[b]):
                flag = 1
                break
            k2[int(seq_start[b]) + lens[b]] = k[r].reshape(hkv, d)
            v2[int(seq_start[b]) + lens[b]] = v[r].reshape(hkv, d)
            lens[b] += 1
    return k2, v2, lens, flag


def _decay_includes_own(gamma):
    g = np.asarray(gamma, dtype=np.float64)
    n = g.shape[0]
    d = np.zeros((n, n))
    for i in range(n):
        d[i, i] = g[i]
        for j in range(i - 1, -1, -1):
            d[i, j] = d[i, j + 1] * g[j]
    return d


def _decay_strict(gamma):
    return og.__dict__["_orig_decay"](gamma) - np.eye(len(gamma))


def _recurrent_decay_after(q, k, v, gamma, s0=None):
    s = np.zeros((k.shape[1], v.shape[1])) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        s = float(gamma[t]) * (s + np.outer(k[t], v[t]))
        o[t] = q[t] @ s
    return o, s


def _recurrent_output_before_update(q, k, v, gamma, s0=None):
    s = np.zeros((k.shape[1], v.shape[1])) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        o[t] = q[t] @ s
        s = float(gamma[t]) * s + np.outer(k[t], v[t])
    return o, s


def _chunk_state_not_decayed(q, k, v, gamma, s0=None, chunk=256):
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, gamma))
    s = np.zeros((k.shape[1], v.shape[1])) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    for c0 in range(0, q.shape[0], chunk):
        c1 = min(c0 + chunk, q.shape[0])
        d = og.gret_decay_matrix(g[c0:c1])
        o[c0:c1] = ((q[c0:c1] @ k[c0:c1].T) * d) @ v[c0:c1] + q[c0:c1] @ s
        s = np.prod(g[c0:c1]) * s + (d[-1][:, None] * k[c0:c1]).T @ v[c0:c1]
    return o, s


def _parallel_prefix_excludes_first(q, k, v, gamma, s0=None):
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, gamma))
    d = og.gret_decay_matrix(g)
    o = ((q @ k.T) * d) @ v
    s_n = np.zeros((k.shape[1], v.shape[1]))
    if s0 is not None:
        prefix = np.concatenate([[1.0], np.cumprod(g[1:])]) if len(g) else np.zeros(0)
        o = o + (prefix[:, None] * q) @ np.asarray(s0, dtype=np.float64)
        s_n = (prefix[-1] if len(g) else 1.0) * np.asarray(s0, dtype=np.float64)
    if len(g):
        s_n = s_n + (d[-1][:, None] * k).T @ v
    return o, s_n


def _softmax_no_exp(s):
    m = np.max(s, axis=-1, keepdims=True)
    w = np.where(np.isfinite(s), s - m + 10.0, 0.0)
    return w, m, np.sum(w, axis=-1, keepdims=True)


def _softmax_unnormalised_sum(s):
    m = np.max(s, axis=-1, keepdims=True)
    w = np.exp(s - m)
    return w, m, np.ones_like(m)


MUTATIONS = {
    "head_map_interleaved": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "head_map_zero": ("kv_head_of", lambda h, hq, hkv: 0),
    "mask_excludes_diagonal": ("visible_rows", lambda p: p),
    "mask_one_too_many": ("visible_rows", lambda p: p + 2),
    "no_scale": ("scores", lambda q, k, scale: q @ k.T),
    "scale_squared": ("scores", lambda q, k, scale: scale * scale * (q @ k.T)),
    "sqrt_scale": ("scores", lambda q, k, scale: np.sqrt(scale) * (q @ k.T)),
    "negated_scores": ("scores", lambda q, k, scale: -scale * (q @ k.T)),
    "no_exp": ("softmax_weights", _softmax_no_exp),
    "no_normalisation": ("softmax_weights", _softmax_unnormalised_sum),
    "lse_drops_max": ("log_sum_exp", lambda m, z: np.log(z)),
    "lse_log2": ("log_sum_exp", lambda m, z: m + np.log2(z)),
    "prefill_position_shift": ("prefill_position", lambda r, m, n: r + max(n - m, 0) + 1),
    "rows_past_cache_see_every_row": ("has_own_row", lambda p, n: True),
    "last_own_row_treated_as_missing": ("has_own_row", lambda p, n: p < n - 1),
    "chunk_aligned_top_left": ("prefill_position", lambda r, m, n: r),
    "chunk_offset_off_by_one": ("prefill_position", lambda r, m, n: r + max(n - m - 1, 0)),
    "decode_position_before_append": ("decode_position", lambda n: n - 2),
    "decode_position_past_end": ("decode_position", lambda n: n),
    "append_wrong_row": ("kv_append_ref", _append_wrong_row),
    "append_ignores_capacity": ("kv_append_ref", _append_no_cap),
    "window_one_too_many": ("window_start", lambda p, w: max(0, p - w) if w > 0 else 0),
    "window_one_too_few": ("window_start", lambda p, w: max(0, p - w + 2) if w > 0 else 0),
    "window_ignored": ("window_start", lambda p, w: 0),
    "window_in_fixed_blocks": ("window_start", lambda p, w: (p // w) * w if w > 0 else 0),
    "ring_slot_shifted": ("ring_append_ref", _ring_slot_shift),
    "ring_does_not_wrap": ("ring_append_ref", _ring_no_wrap),
    "rmsnorm_sum_not_mean": ("op.rmsnorm_ref", _rms_sum_not_mean),
    "rmsnorm_eps_outside_sqrt": ("op.rmsnorm_ref", _rms_eps_outside),
    "rmsnorm_no_gain": ("op.rmsnorm_ref", _rms_no_gain),
    "rmsnorm_gain_before_norm": ("op.rmsnorm_ref", _rms_gain_first),
    "projection_k_v_swapped": ("op.kv_project_ref", _project_swapped),
    "combine_weights_swapped": ("op.kv_combine_ref", lambda km, kb, a1, a2, lam: lam * (a2 * kb + a1 * km)),
    "combine_without_lambda": ("op.kv_combine_ref", lambda km, kb, a1, a2, lam: a1 * kb + a2 * km),
    "project_append_at_sequence_start": ("op.project_append_ref", _append_chunk_at_start),
    "project_append_partial_chunk": ("op.project_append_ref", _append_partial_chunk),
    "gret_decay_includes_own_gate": ("og.gret_decay_matrix", _decay_includes_own),
    "gret_decay_without_diagonal": ("og.gret_decay_matrix", _decay_strict),
    "gret_recurrence_decays_new_term": ("og.gret_recurrent_ref", _recurrent_decay_after),
    "gret_output_before_state_update": ("og.gret_recurrent_ref", _recurrent_output_before_update),
    "gret_chunk_state_not_decayed_to_row": ("og.gret_chunkwise_ref", _chunk_state_not_decayed),
    "gret_prefix_decay_excludes_first": ("og.gret_parallel_ref", None),
}


def test_unmutated_oracle_passes_all_pins():
    for check in pinlib.ALL_PINS:
        check()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS[name]
    module = ox
    if attr.startswith("op."):
        module, attr = op, attr[3:]
    elif attr.startswith("og."):
        module, attr = og, attr[3:]
        monkeypatch.setitem(og.__dict__, "_orig_decay", og.gret_decay_matrix)
        if repl is None:
            repl = _parallel_prefix_excludes_first
    monkeypatch.setattr(module, attr, repl)
    caught = []
    for check in pinlib.ALL_PINS:
        try:
            check()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            caught.append(check.__name__)
    assert caught, f"mutation {name} passed every pin"
