"""The comparison every parity test uses.

Two numbers per comparison, both against the fp64 oracle on the same stored inputs:

* max-abs error: the acceptance bound (1e-5 for fp32 storage, 2e-2 for bf16);
* row-relative error: max over (row, head) of max|err| / max|ref| over that
  row's head_dim values. On inputs whose logits have unit spread (Q, K ~ N(0,1))
  this separates a correct kernel (< 1e-2 in bf16) from a wrong one (> 0.3);
  the max-abs bound alone does not on N(0,1)/sqrt(d) inputs.

The bf16 row-relative bound follows from the arithmetic: inputs are exact, the
scores are fp32, P is rounded to bf16 before the P.V product (relative error
2^-9 per weight, averaging out over the row), accumulation is fp32 and the
output is rounded once to bf16 (2^-9 relative). 1e-2 leaves a margin of ~5x
over the worst case seen in simulation.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = {"f32": 1e-5, "bf16": 2e-2}
ROW_REL = {"f32": 1e-5, "bf16": 1e-2}
LSE_ABS = {"f32": 1e-5, "bf16": 2e-3}


def errors(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise AssertionError(f"shape {out.shape} != {ref.shape}")
    if not np.all(np.isfinite(out)):
        return {"max_abs": float("inf"), "row_rel": float("inf")}
    err = np.abs(out - ref)
    max_abs = float(err.max()) if err.size else 0.0
    d = out.shape[-1]
    e2 = err.reshape(-1, d).max(axis=1)
    r2 = np.abs(ref).reshape(-1, d).max(axis=1)
    row_rel = float((e2 / np.maximum(r2, 1e-30)).max()) if e2.size else 0.0
    return {"max_abs": max_abs, "row_rel": row_rel}


def check(out, ref, dtype, discriminating=False, what=""):
    """Raise AssertionError unless out matches ref to the bounds for dtype.

    Acceptance inputs (discriminating=False): the max-abs bound. Discriminating
    inputs (unit-spread logits, outputs of magnitude ~1 or more): the row-relative
    bound, which scales with the output like bf16 rounding does; fp32 keeps the
    max-abs bound as well.
    """
    e = errors(out, ref)
    if not discriminating or dtype == "f32":
        assert e["max_abs"] <= MAX_ABS[dtype], f"{what}: max-abs {e['max_abs']:.3e} > {MAX_ABS[dtype]}"
    if discriminating:
        assert e["row_rel"] <= ROW_REL[dtype], f"{what}: row-relative {e['row_rel']:.3e} > {ROW_REL[dtype]}"
    return e


def check_signed_sum(out, ref, dtype, what=""):
    """The row-relative check for outputs that are signed sums with no
    normalisation (gated retention: o_j = sum_m D[j,m] (q_j . k_m) v_m). Each
    term carries the bf16 rounding of its weight, but a row whose terms cancel
    has a max|ref| well below the terms' scale, so its row-relative error grows
    with the cancellation, and over 10^5 rows a few rows cancel strongly. The
    bulk keeps the softmax bound (99.9% of rows within ROW_REL) and no row may
    exceed 4 x ROW_REL; a missing or wrong term (a dropped state, a wrong chunk)
    gives errors of order 1 in most rows."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise AssertionError(f"shape {out.shape} != {ref.shape}")
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    d = out.shape[-1]
    e2 = np.abs(out - ref).reshape(-1, d).max(axis=1)
    r2 = np.abs(ref).reshape(-1, d).max(axis=1)
    rel = e2 / np.maximum(r2, 1e-30)
    bulk = float(np.quantile(rel, 0.999))
    worst = float(rel.max())
    assert bulk <= ROW_REL[dtype], f"{what}: 99.9th percentile row-relative {bulk:.3e} > {ROW_REL[dtype]}"
    assert worst <= 4 * ROW_REL[dtype], f"{what}: row-relative {worst:.3e} > {4 * ROW_REL[dtype]}"
    return {"row_rel": worst, "row_rel_p999": bulk}


def check_lse(lse, ref, dtype, what=""):
    lse = np.asarray(lse, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(ref)
    fin = ~both_inf
    assert np.all(np.isfinite(lse[fin])) and np.all(np.isfinite(ref[fin])), f"{what}: non-finite LSE"
    err = float(np.abs(lse[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert err <= LSE_ABS[dtype], f"{what}: LSE max-abs {err:.3e} > {LSE_ABS[dtype]}"
    return err
