"""Shared helpers for the GPU parity tests: run the library, compare with the
fp64 oracle on the same seeded inputs, and report the errors."""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np
import torch

import attn_inputs
from oracle import attention_fp64, attention_unfused_bf16

O_TOL = 1e-2  # max |O_gpu - O_oracle|
LSE_TOL = 1e-3  # max |LSE_gpu - LSE_oracle|
# |O| from which the bf16 rounding of the output takes most of O_TOL by itself: half
# an ulp is 2^-7 = 0.0078 for |O| in [2, 4), 0.0156 from 4 on, which leaves at most
# 0.0022 of O_TOL, and none from 4 on, for the 16-bit P the pages prescribe (the
# standard bf16 computation, the yardstick, reaches 0.0145 at the wide-score workload).
O_WIDE = 2.0


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x|: the error that rounding a value of that size to the
    bf16 output carries by itself. bf16 keeps 8 significant bits, so for |x| in
    [2^e, 2^(e+1)) the ulp is 2^(e-7): half of it is 0.0078 for |x| in [2, 4) and
    0.0156 for [4, 8). From |x| = O_WIDE on the O tolerance is applied on top of it
    (the raw figures are still recorded). The rounding happens at the computed value's
    size, which can sit just above a power of two while the exact value sits just
    below it, so callers evaluate it at the larger of the two magnitudes."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 8)


def announce(msg: str):
    """Name the case before a GPU step, so a crash log says what was running."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def o_errors(o, O_ref):
    """Element-wise O error statistics of o against O_ref (float64 arrays of one
    shape). Elements whose size (the larger of |o| and |O_ref|) is below O_WIDE are
    gated on the raw |dO|; the others on |dO| beyond the half bf16 ulp at their
    size."""
    dO = np.abs(o - O_ref)
    size = np.maximum(np.abs(O_ref), np.abs(o))
    wide = size >= O_WIDE
    out = {
        "max_dO": float(dO.max()) if o.size else 0.0,
        "max_abs_O_ref": float(np.abs(O_ref).max()) if o.size else 0.0,
        "max_dO_narrow": float(dO[~wide].max()) if (~wide).any() else 0.0,
        "n_wide": int(wide.sum()),
        "max_dO_wide_beyond_rounding": float((dO[wide] - bf16_half_ulp(size[wide])).max()) if wide.any() else None,
        "n_over_tol": int((dO > O_TOL).sum()),
        "n_elements": int(o.size),
    }
    out["max_dO_beyond_rounding"] = (float((dO - bf16_half_ulp(size)).max()) if o.size else 0.0)
    return out


def gpu_errors(q, k, v, o_gpu, lse_gpu, scale, rows=None, with_unfused=True):
    """Errors of GPU outputs (torch tensors, any device) against the fp64 oracle on
    ``rows`` (flat indices; None = all). Returns the o_errors statistics, max |dLSE|
    and the bf16 unfused yardstick error E_unf on the same rows."""
    qd, kd, vd = (attn_inputs.bf16_to_f64(t) for t in (q, k, v))
    O_ref, L_ref = attention_fp64(qd, kd, vd, scale, rows=rows)
    d = q.shape[-1]
    o = o_gpu.detach().cpu().double().numpy().reshape(-1, d)
    lse = lse_gpu.detach().cpu().double().numpy().reshape(-1)
    if rows is None:
        O_ref = O_ref.reshape(-1, d)
        L_ref = L_ref.reshape(-1)
    else:
        o = o[rows]
        lse = lse[rows]
    out = o_errors(o, O_ref)
    out["max_dLSE"] = float(np.abs(lse - L_ref).max()) if lse.size else 0.0
    out["finite"] = bool(np.isfinite(o).all() and np.isfinite(lse).all())
    out["rows_checked"] = int(o.shape[0])
    if with_unfused:
        O_unf, _ = attention_unfused_bf16(q, k, v, scale, rows=rows)
        if rows is None:
            O_unf = O_unf.reshape(-1, d)
        out["E_unf"] = float(np.abs(O_unf - O_ref).max()) if O_unf.size else 0.0
    return out


def assert_parity(err, context="", check_yardstick=True):
    """The gates: max |dO| <= O_TOL on every element smaller than O_WIDE (raw, no
    rounding allowance), and beyond the half bf16 ulp on the wider ones; max |dLSE|
    <= LSE_TOL; and raw max |dO| <= 2 x E_unf (the pages' error bar against the
    standard computation)."""
    assert err["finite"], f"{context}: non-finite output"
    assert err["max_dO_narrow"] <= O_TOL, (
        f"{context}: max|dO| over elements with |O| < {O_WIDE} is {err['max_dO_narrow']:.3e} > {O_TOL}")
    if err["n_wide"]:
        assert err["max_dO_wide_beyond_rounding"] <= O_TOL, (
            f"{context}: max(|dO| - bf16 half-ulp) over {err['n_wide']} elements with |O| >= {O_WIDE} is "
            f"{err['max_dO_wide_beyond_rounding']:.3e} > {O_TOL}")
    assert err["max_dLSE"] <= LSE_TOL, f"{context}: max|dLSE| {err['max_dLSE']:.3e} > {LSE_TOL}"
    if check_yardstick and "E_unf" in err:
        assert err["max_dO"] <= 2.0 * err["E_unf"], (
            f"{context}: max|dO| {err['max_dO']:.3e} > 2 x E_unf {err['E_unf']:.3e}")


def record(kind: str, name: str, err: dict, **extra):
    """Print the raw error figures of a case and, when FA_PARITY_RECORD names a
    file, append them to it as one JSON line."""
    rec = {"kind": kind, "case": name, **extra, **err}
    print("  parity " + json.dumps(rec), flush=True)
    path = os.environ.get("FA_PARITY_RECORD")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def to_gpu(*ts):
    return tuple(t.to("cuda") for t in ts)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def decode_errors(q, k, v, o_gpu, lse_gpu, scale, heads=None):
    """Errors of decode outputs against the fp64 oracle, head by head: ``heads`` is a
    list of (b, h) pairs (None = every head); all query rows of each head are
    compared. Returns the same keys as gpu_errors, each the maximum over the heads."""
    B, H = q.shape[:2]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    out = None
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        e = gpu_errors(q[sl], k[sl], v[sl], o_gpu[sl], lse_gpu[sl], scale)
        out = e if out is None else _merge(out, e)
    return out


def _merge(a, b):
    """Combine the error statistics of two disjoint sets of rows."""
    out = {}
    for key, x in a.items():
        y = b[key]
        if key in ("n_wide", "n_over_tol", "n_elements", "rows_checked"):
            out[key] = x + y
        elif key == "finite":
            out[key] = x and y
        elif x is None or y is None:
            out[key] = y if x is None else x
        else:
            out[key] = max(x, y)
    return out
