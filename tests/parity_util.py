"""Shared helpers for the GPU parity tests: run the library, compare with the
fp64 oracle on the same seeded inputs, and report the errors."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import attn_inputs
from oracle import attention_fp64, attention_unfused_bf16

O_TOL = 1e-2  # max |O_gpu - O_oracle| beyond the output's own bf16 rounding (see bf16_half_ulp)
LSE_TOL = 1e-3  # max |LSE_gpu - LSE_oracle|


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x|: the error that rounding a value of that size to the
    bf16 output carries by itself. bf16 keeps 8 significant bits, so for |x| in
    [2^e, 2^(e+1)) the ulp is 2^(e-7). For |x| >= 4 this exceeds 1e-2 by itself,
    which is why the absolute O tolerance is applied on top of it (the comparison
    with the unfused yardstick, which carries the same rounding, stays as stated).
    The rounding happens at the computed value's size, which can sit just above a
    power of two while the exact value sits just below it, so callers evaluate it
    at the larger of the two magnitudes."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 8)


def announce(msg: str):
    """Name the case before a GPU step, so a crash log says what was running."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_errors(q, k, v, o_gpu, lse_gpu, scale, rows=None, with_unfused=True):
    """Errors of GPU outputs (torch tensors, any device) against the fp64 oracle on
    ``rows`` (flat indices; None = all). Returns dict with max |dO|, max |dLSE| and
    the bf16 unfused yardstick error E_unf on the same rows."""
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
    dO = np.abs(o - O_ref)
    out = {
        "max_dO": float(dO.max()) if o.size else 0.0,
        "max_dO_beyond_rounding": float((dO - bf16_half_ulp(np.maximum(np.abs(O_ref), np.abs(o)))).max())
        if o.size else 0.0,
        "max_dLSE": float(np.abs(lse - L_ref).max()) if lse.size else 0.0,
        "finite": bool(np.isfinite(o).all() and np.isfinite(lse).all()),
    }
    if with_unfused:
        O_unf, _ = attention_unfused_bf16(q, k, v, scale, rows=rows)
        if rows is None:
            O_unf = O_unf.reshape(-1, d)
        out["E_unf"] = float(np.abs(O_unf - O_ref).max()) if O_unf.size else 0.0
    return out


def assert_parity(err, context="", check_yardstick=True):
    assert err["finite"], f"{context}: non-finite output"
    assert err["max_dO_beyond_rounding"] <= O_TOL, (
        f"{context}: max(|dO| - bf16 half-ulp) {err['max_dO_beyond_rounding']:.3e} > {O_TOL} "
        f"(raw max|dO| {err['max_dO']:.3e})")
    assert err["max_dLSE"] <= LSE_TOL, f"{context}: max|dLSE| {err['max_dLSE']:.3e} > {LSE_TOL}"
    if check_yardstick and "E_unf" in err:
        assert err["max_dO"] <= 2.0 * err["E_unf"], (
            f"{context}: max|dO| {err['max_dO']:.3e} > 2 x E_unf {err['E_unf']:.3e}")


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
    out = {"max_dO": 0.0, "max_dO_beyond_rounding": -1.0, "max_dLSE": 0.0, "finite": True, "E_unf": 0.0}
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        e = gpu_errors(q[sl], k[sl], v[sl], o_gpu[sl], lse_gpu[sl], scale)
        for key in ("max_dO", "max_dO_beyond_rounding", "max_dLSE", "E_unf"):
            out[key] = max(out[key], e[key])
        out["finite"] = out["finite"] and e["finite"]
    return out

