"""Pins for the fp64 oracle (CPU only, no GPU).

Each pin checks the oracle against something other than itself: closed forms
derived by hand (tests/golden/closed_form_cases.json), invariants the pages state
(exactness of the tiled/online form, row independence, normalisation), brute
force on tiny inputs, and library routines. ``test_planted_mistakes_are_caught``
plants plausible mistakes in copies of the oracle and checks that the pins fail.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import attn_inputs
from oracle import (attention_brute_force, attention_fp64, attention_online_fp64,
                    attention_split_fp64, attention_unfused_bf16)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
TOL = 1e-12


def rand_qkv(B, H, N, d, seed, sigma=1.0):
    q, k, v = attn_inputs.make_qkv(B, H, N, d, seed, sigma_qk=sigma)
    return attn_inputs.bf16_to_f64(q), attn_inputs.bf16_to_f64(k), attn_inputs.bf16_to_f64(v)


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


# ---------------------------------------------------------------------------
# Pin suite. Each check takes an implementation impl(q, k, v, scale) -> (O, LSE)
# on [B,H,N,d] float64 arrays and raises AssertionError when the pin fails.
# ---------------------------------------------------------------------------

def check_golden(impl):
    for c in golden_cases():
        q = np.array(c["q"])[None, None]
        k = np.array(c["k"])[None, None]
        v = np.array(c["v"])[None, None]
        O, L = impl(q, k, v, c["scale"])
        np.testing.assert_allclose(O[0, 0], np.array(c["O"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(L[0, 0], np.array(c["LSE"]), rtol=0, atol=1e-12, err_msg=c["name"])


def check_q_zero(impl):
    """Q = 0: every score is 0, so O is the mean of the V rows and LSE = ln N."""
    for N, d in ((1, 4), (5, 3), (64, 16), (100, 8)):
        _, k, v = rand_qkv(1, 2, N, d, seed=N)
        q = np.zeros_like(k)
        O, L = impl(q, k, v, 1.0 / math.sqrt(d))
        np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=TOL)
        np.testing.assert_allclose(L, np.full(L.shape, math.log(N)), atol=TOL)


def check_scale_zero(impl):
    q, k, v = rand_qkv(1, 1, 37, 8, seed=3)
    O, L = impl(q, k, v, 0.0)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=TOL)
    np.testing.assert_allclose(L, np.full(L.shape, math.log(37)), atol=TOL)


def check_v_constant(impl):
    """All V rows equal c: the weights sum to one, so every output row is c."""
    q, k, _ = rand_qkv(2, 1, 50, 6, seed=5, sigma=2.0)
    c = np.array([0.5, -1.25, 3.0, 0.0, 7.5, -2.0])
    v = np.broadcast_to(c, k.shape).copy()
    O, _ = impl(q, k, v, 0.4)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), atol=TOL)


def check_single_key(impl):
    """N = 1: O = v_0 and LSE = the single scaled score."""
    q, k, v = rand_qkv(2, 3, 1, 16, seed=7)
    scale = 0.3
    O, L = impl(q, k, v, scale)
    np.testing.assert_allclose(O, v, atol=TOL)
    np.testing.assert_allclose(L, scale * (q * k).sum(-1), atol=TOL)


def check_identity_values(impl):
    """d = N and V = I: O's rows are the softmax weights themselves. They must be
    positive, sum to one, and have ratios exp(s_ij - s_ik)."""
    N = 12
    q, k, _ = rand_qkv(1, 1, N, N, seed=11)
    v = np.eye(N)[None, None]
    scale = 0.25
    O, L = impl(q, k, v, scale)
    P = O[0, 0]
    assert (P > 0).all()
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=TOL)
    s = scale * np.einsum("ic,jc->ij", q[0, 0], k[0, 0])
    np.testing.assert_allclose(np.log(P[:, 1:] / P[:, :1]), s[:, 1:] - s[:, :1], atol=1e-10)
    np.testing.assert_allclose(np.log(P) + L[0, 0][:, None], s, atol=1e-10)


def check_permutation(impl):
    """Permuting K and V rows jointly leaves O and LSE unchanged."""
    q, k, v = rand_qkv(1, 2, 70, 8, seed=13, sigma=2.5)
    perm = np.random.default_rng(0).permutation(70)
    O1, L1 = impl(q, k, v, 0.35)
    O2, L2 = impl(q, k[:, :, perm], v[:, :, perm], 0.35)
    np.testing.assert_allclose(O1, O2, atol=TOL)
    np.testing.assert_allclose(L1, L2, atol=TOL)


def check_brute_force(impl):
    for N, d, seed in ((1, 3, 1), (2, 2, 2), (7, 5, 3), (16, 8, 4), (13, 1, 5)):
        q, k, v = rand_qkv(1, 1, N, d, seed=seed)
        scale = 1.0 / math.sqrt(d)
        O, L = impl(q, k, v, scale)
        Ob, Lb = attention_brute_force(q[0, 0], k[0, 0], v[0, 0], scale)
        np.testing.assert_allclose(O[0, 0], np.array(Ob), atol=TOL)
        np.testing.assert_allclose(L[0, 0], np.array(Lb), atol=TOL)


def check_bounds(impl):
    """max_j s_j <= LSE <= max_j s_j + ln N; each O[i, c] lies within V's column range."""
    q, k, v = rand_qkv(1, 1, 90, 8, seed=17, sigma=2.5)
    scale = 0.35
    O, L = impl(q, k, v, scale)
    s = scale * np.einsum("ic,jc->ij", q[0, 0], k[0, 0])
    smax = s.max(axis=1)
    assert (L[0, 0] >= smax - 1e-12).all() and (L[0, 0] <= smax + math.log(90) + 1e-12).all()
    assert (O[0, 0] >= v[0, 0].min(axis=0) - 1e-12).all()
    assert (O[0, 0] <= v[0, 0].max(axis=0) + 1e-12).all()


def check_library(impl):
    """Reduces to torch's own fp64 routines: logsumexp and softmax followed by a matmul."""
    q, k, v = rand_qkv(2, 2, 33, 16, seed=19)
    scale = 0.25
    O, L = impl(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=TOL)
    np.testing.assert_allclose(O, torch.matmul(torch.softmax(s, dim=-1), tv).numpy(), atol=TOL)


def check_few_queries_many_keys(impl):
    """Decode shapes, N query rows against Nk != N keys: Q = 0 gives the mean of
    all Nk value rows and LSE = ln Nk; brute force and torch's fp64 routines on
    rectangular inputs."""
    q, _, _ = rand_qkv(1, 2, 3, 8, seed=41)
    _, k, v = rand_qkv(1, 2, 50, 8, seed=42)
    O, L = impl(np.zeros_like(q), k, v, 0.35)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=TOL)
    np.testing.assert_allclose(L, np.full(L.shape, math.log(50)), atol=TOL)
    for nq, nk, seed in ((2, 11, 43), (5, 1, 44), (1, 16, 45)):
        q, _, _ = rand_qkv(1, 1, nq, 4, seed=seed)
        _, k, v = rand_qkv(1, 1, nk, 4, seed=seed + 100, sigma=2.0)
        O, L = impl(q, k, v, 0.5)
        Ob, Lb = attention_brute_force(q[0, 0], k[0, 0], v[0, 0], 0.5)
        np.testing.assert_allclose(O[0, 0], np.array(Ob), atol=TOL)
        np.testing.assert_allclose(L[0, 0], np.array(Lb), atol=TOL)
    q, _, _ = rand_qkv(2, 2, 4, 16, seed=46)
    _, k, v = rand_qkv(2, 2, 300, 16, seed=47, sigma=2.5)
    O, L = impl(q, k, v, 0.25)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    s = 0.25 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=TOL)
    np.testing.assert_allclose(O, torch.matmul(torch.softmax(s, dim=-1), tv).numpy(), atol=TOL)


PINS = [check_golden, check_q_zero, check_scale_zero, check_v_constant, check_single_key,
        check_identity_values, check_permutation, check_brute_force, check_bounds, check_library,
        check_few_queries_many_keys]


def failing_pins(impl):
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except Exception:  # an error in a mutant counts as a caught mistake
            failed.append(pin.__name__)
    return failed


# ---------------------------------------------------------------------------
# The oracle against every pin
# ---------------------------------------------------------------------------

def two_pass(q, k, v, scale):
    return attention_fp64(q, k, v, scale)


def online_normalised_7(q, k, v, scale):
    return attention_online_fp64(q, k, v, scale, bc=7)


def online_deferred_5_br3(q, k, v, scale):
    return attention_online_fp64(q, k, v, scale, bc=5, br=3, deferred=True)


def split_7(q, k, v, scale):
    return attention_split_fp64(q, k, v, scale, chunk=7)


def split_64(q, k, v, scale):
    return attention_split_fp64(q, k, v, scale, chunk=64)


@pytest.mark.parametrize("impl", [two_pass, online_normalised_7, online_deferred_5_br3, split_7, split_64])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(impl, pin):
    pin(impl)


# ---------------------------------------------------------------------------
# Online (tiled) forms against the two-pass definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bc", [64, 7, 37, 1, 300])
@pytest.mark.parametrize("deferred", [False, True])
@pytest.mark.parametrize("sigma", [1.0, 2.5])
def test_online_equals_two_pass(bc, deferred, sigma):
    q, k, v = rand_qkv(2, 2, 200, 16, seed=23, sigma=sigma)
    O1, L1 = attention_fp64(q, k, v, 0.25)
    O2, L2 = attention_online_fp64(q, k, v, 0.25, bc=bc, br=64, deferred=deferred)
    np.testing.assert_allclose(O2, O1, atol=TOL, rtol=0)
    np.testing.assert_allclose(L2, L1, atol=TOL, rtol=0)


def test_online_ascending_scores_rescale_every_tile():
    """Keys sorted by increasing score for query 0: the running max rises in every
    tile, so every tile exercises the rescale of the accumulated state."""
    q, k, v = rand_qkv(1, 1, 256, 8, seed=29, sigma=2.5)
    s0 = k[0, 0] @ q[0, 0, 0]
    order = np.argsort(s0)
    k, v = k[:, :, order], v[:, :, order]
    for deferred in (False, True):
        O1, L1 = attention_fp64(q, k, v, 0.5)
        O2, L2 = attention_online_fp64(q, k, v, 0.5, bc=16, deferred=deferred)
        np.testing.assert_allclose(O2, O1, atol=TOL, rtol=0)
        np.testing.assert_allclose(L2, L1, atol=TOL, rtol=0)


@pytest.mark.parametrize("chunk", [1, 7, 64, 256, 1000, 5000])
@pytest.mark.parametrize("sigma", [1.0, 2.5])
def test_split_equals_two_pass(chunk, sigma):
    """The merged split (decode shape: 4 queries, 1000 keys) reproduces the
    two-pass result for any chunk size, including one chunk and chunks of one key."""
    q, _, _ = rand_qkv(2, 2, 4, 16, seed=51, sigma=sigma)
    _, k, v = rand_qkv(2, 2, 1000, 16, seed=52, sigma=sigma)
    O1, L1 = attention_fp64(q, k, v, 0.25)
    O2, L2 = attention_split_fp64(q, k, v, 0.25, chunk=chunk)
    np.testing.assert_allclose(O2, O1, atol=TOL, rtol=0)
    np.testing.assert_allclose(L2, L1, atol=TOL, rtol=0)


def test_split_rows_subset():
    q, _, _ = rand_qkv(2, 3, 6, 8, seed=53)
    _, k, v = rand_qkv(2, 3, 90, 8, seed=54)
    rows = attn_inputs.sample_rows(2, 3, 6, 10, seed=2)
    O, L = attention_fp64(q, k, v, 0.3, rows=rows)
    Os, Ls = attention_split_fp64(q, k, v, 0.3, chunk=16, rows=rows)
    np.testing.assert_allclose(Os, O, atol=TOL)
    np.testing.assert_allclose(Ls, L, atol=TOL)


def test_rows_subset_matches_full():
    q, k, v = rand_qkv(2, 3, 40, 8, seed=31)
    rows = attn_inputs.sample_rows(2, 3, 40, 25, seed=1)
    O, L = attention_fp64(q, k, v, 0.3)
    Os, Ls = attention_fp64(q, k, v, 0.3, rows=rows)
    np.testing.assert_array_equal(Os, O.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(Ls, L.reshape(-1)[rows])
    Oo, Lo = attention_online_fp64(q, k, v, 0.3, bc=9, rows=rows, deferred=True)
    np.testing.assert_allclose(Oo, Os, atol=TOL)
    np.testing.assert_allclose(Lo, Ls, atol=TOL)


def test_brute_force_against_closed_forms():
    """The brute-force routine itself reproduces the hand-derived cases that do not
    overflow its unshifted exponentials."""
    for c in golden_cases():
        if c["name"] == "huge_equal_scores":
            continue
        O, L = attention_brute_force(c["q"], c["k"], c["v"], c["scale"])
        np.testing.assert_allclose(np.array(O), np.array(c["O"]), atol=1e-12)
        np.testing.assert_allclose(np.array(L), np.array(c["LSE"]), atol=1e-12)


# ---------------------------------------------------------------------------
# The bf16 unfused yardstick
# ---------------------------------------------------------------------------

def test_unfused_bf16_exact_case():
    """Uniform scores with N a power of two: P = 1/N exactly in bf16, and V rows
    that are small integers make every step exact, so O equals the mean exactly."""
    N, d = 64, 8
    q = torch.zeros(1, 1, N, d, dtype=torch.bfloat16)
    k = torch.randn(1, 1, N, d, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    v = torch.randint(-4, 5, (1, 1, N, d), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    Ou, Lu = attention_unfused_bf16(q, k, v, 0.125)
    np.testing.assert_array_equal(Ou, torch.tensor(attn_inputs.bf16_to_f64(v)).mean(dim=2, keepdim=True)
                                  .to(torch.bfloat16).double().numpy().repeat(N, axis=2))
    np.testing.assert_allclose(Lu, math.log(N), atol=1e-6)


YARDSTICK = os.path.join(os.path.dirname(__file__), "golden", "yardstick_cases.json")


def check_yardstick_golden(impl):
    """The hand-derived cases of tests/golden/yardstick_cases.json: inputs on which
    every fp32 step is exact, so the bf16 rounding of P (IO page, section 6) and
    of O each decide the expected bits."""
    with open(YARDSTICK) as f:
        cases = json.load(f)["forward"]
    for c in cases:
        q, k, v = (torch.tensor(c[n], dtype=torch.float32).to(torch.bfloat16)[None, None] for n in "qkv")
        assert all(torch.equal(t.float(), torch.tensor(c[n], dtype=torch.float32)[None, None])
                   for t, n in zip((q, k, v), "qkv")), "inputs must be bf16 values"
        O, L = impl(q, k, v, c["scale"])
        np.testing.assert_array_equal(O[0, 0], np.array(c["O"]), err_msg=c["name"])
        np.testing.assert_allclose(L[0, 0], np.array(c["LSE"]), rtol=0, atol=1e-6, err_msg=c["name"])


def check_yardstick_error_bound(impl):
    """Random inputs: the deviation from the fp64 result is within the rounding the
    yardstick introduces (bf16 P, relative 2^-9 per weight; bf16 O, relative 2^-9),
    and nonzero (the 16-bit P does introduce error)."""
    q, k, v = attn_inputs.make_qkv(1, 2, 300, 64, seed=37)
    scale = 0.125
    O64, L64 = attention_fp64(attn_inputs.bf16_to_f64(q), attn_inputs.bf16_to_f64(k),
                              attn_inputs.bf16_to_f64(v), scale)
    Ou, Lu = impl(q, k, v, scale)
    vmax = float(v.abs().max())
    bound = 2.0 ** -9 * vmax + 2.0 ** -9 * np.abs(O64) + 1e-5
    assert (np.abs(Ou - O64) <= bound).all()
    assert np.abs(Ou - O64).max() > 0
    np.testing.assert_allclose(Lu, L64, atol=1e-4)


YARDSTICK_PINS = [check_yardstick_golden, check_yardstick_error_bound]


def test_unfused_bf16_yardstick_pins():
    for pin in YARDSTICK_PINS:
        pin(attention_unfused_bf16)


def _round_bf16_toward_zero(t):
    """fp32 -> bf16 by dropping the low 16 bits (truncation, not nearest-even)."""
    return (t.contiguous().view(torch.int32) & -65536).view(torch.float32)


def _mut_unfused(kind):
    """Copies of the yardstick with one plausible mistake at a rounding point."""
    def impl(q, k, v, scale, rows=None):
        B, H, N, d = q.shape
        O = np.empty((B, H, N, d))
        L = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                S = (q[b, h].float() @ k[b, h].float().T) * torch.tensor(scale, dtype=torch.float32)
                m = S.max(dim=1).values
                E = torch.exp(S - m[:, None])
                l = E.sum(dim=1)
                P = E / l[:, None]
                if kind == "p_fp16":
                    P = P.to(torch.float16).float()
                elif kind == "p_truncated":
                    P = _round_bf16_toward_zero(P)
                elif kind != "p_fp32":
                    P = P.to(torch.bfloat16).float()
                o = P @ v[b, h].float()
                O[b, h] = (o if kind == "o_fp32" else o.to(torch.bfloat16)).double().numpy()
                L[b, h] = (m + torch.log(l)).double().numpy()
        return O, L
    return impl


@pytest.mark.parametrize("kind", ["p_fp32", "o_fp32", "p_fp16", "p_truncated"])
def test_yardstick_planted_mistakes_are_caught(kind):
    failed = []
    for pin in YARDSTICK_PINS:
        try:
            pin(_mut_unfused(kind))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"yardstick mistake {kind} passed every pin"


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible error in a copy of the oracle fails a pin
# ---------------------------------------------------------------------------

def _mut_two_pass(score_fn=None, shift="row", lse="ln", norm="l"):
    def impl(q, k, v, scale):
        B, H, N, d = q.shape
        O = np.empty_like(q if q.shape[-1] == v.shape[-1] else np.empty((B, H, N, v.shape[-1])))
        L = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                S = score_fn(q[b, h], k[b, h], scale) if score_fn else scale * q[b, h] @ k[b, h].T
                m = S.max(axis=1) if shift == "row" else S.max(axis=0)
                P = np.exp(S - (m[:, None] if shift == "row" else m[None, :]))
                l = P.sum(axis=1)
                den = l if norm == "l" else float(N)
                O[b, h] = (P @ v[b, h]) / (den[:, None] if norm == "l" else den)
                L[b, h] = (m if shift == "row" else S.max(axis=1)) + (np.log(l) if lse == "ln" else np.log2(l))
        return O, L
    return impl


def _mut_online(kind):
    def impl(q, k, v, scale):
        B, H, N, d = q.shape
        O = np.empty((B, H, N, v.shape[-1]))
        L = np.empty((B, H, N))
        bc = 4
        for b in range(B):
            for h in range(H):
                Q, K, V = q[b, h], k[b, h], v[b, h]
                m = np.full(N, -np.inf)
                l = np.zeros(N)
                acc = np.zeros((N, V.shape[1]))
                stop = (N // bc) * bc if kind == "drop_ragged_tile" else N
                if stop == 0:
                    stop = N
                for c0 in range(0, stop, bc):
                    S = scale * Q @ K[c0:c0 + bc].T
                    mt = S.max(axis=1)
                    Pt = np.exp(S - mt[:, None])
                    lt = Pt.sum(axis=1)
                    mn = np.maximum(m, mt)
                    a_old = np.exp(mn - m) if kind == "rescale_sign" else np.exp(m - mn)
                    a_new = np.exp(mt - mn)
                    ln = l * a_old + lt * a_new
                    Ot = Pt @ V[c0:c0 + bc]
                    if kind == "forget_l_factor":
                        acc = (a_old[:, None] * acc + a_new[:, None] * Ot) / ln[:, None]
                    else:
                        acc = ((l * a_old)[:, None] * acc + a_new[:, None] * Ot) / ln[:, None]
                    m, l = mn, ln
                O[b, h] = acc
                L[b, h] = m + np.log(l)
        return O, L
    return impl


def _mut_split(kind, chunk=4):
    """Copies of the split-and-merge with one plausible mistake in the merge."""
    def impl(q, k, v, scale):
        Nk = k.shape[2]
        stop = (Nk // chunk) * chunk if kind == "drop_ragged_chunk" and Nk >= chunk else Nk
        parts = [attention_fp64(q, k[:, :, c0:c0 + chunk], v[:, :, c0:c0 + chunk], scale)
                 for c0 in range(0, stop, chunk)]
        lse_s = np.stack([p[1] for p in parts])
        m = lse_s.max(axis=0)
        lse = m if kind == "lse_max_only" else m + np.log(np.exp(lse_s - m).sum(axis=0))
        if kind == "equal_weights":
            w = np.full(lse_s.shape, 1.0 / len(parts))
        else:
            w = np.exp(lse_s - (m + np.log(np.exp(lse_s - m).sum(axis=0))))
        O = sum(w[s][..., None] * parts[s][0] for s in range(len(parts)))
        return O, lse
    return impl


MUTANTS = {
    "dropped_scale": _mut_two_pass(score_fn=lambda q, k, s: q @ k.T),
    "sign_flipped_scores": _mut_two_pass(score_fn=lambda q, k, s: -s * q @ k.T),
    "swapped_q_k": _mut_two_pass(score_fn=lambda q, k, s: s * k @ q.T),
    "column_max_shift": _mut_two_pass(shift="col"),
    "lse_log2": _mut_two_pass(lse="log2"),
    "normalise_by_n": _mut_two_pass(norm="n"),
    "lse_without_max": lambda q, k, v, s: (attention_fp64(q, k, v, s)[0],
                                           attention_fp64(q, k, v, s)[1]
                                           - (s * np.einsum("bhic,bhjc->bhij", q, k)).max(-1)),
    "online_rescale_sign": _mut_online("rescale_sign"),
    "online_forget_l_factor": _mut_online("forget_l_factor"),
    "online_drop_ragged_tile": _mut_online("drop_ragged_tile"),
    "split_equal_weights": _mut_split("equal_weights"),
    "split_lse_max_only": _mut_split("lse_max_only"),
    "split_drop_ragged_chunk": _mut_split("drop_ragged_chunk"),
    "transposed_v_square": lambda q, k, v, s: (attention_fp64(q, k, np.swapaxes(v, -1, -2).copy(), s)
                                               if v.shape[-1] == v.shape[-2] else
                                               (_ for _ in ()).throw(ValueError("shape"))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    failed = failing_pins(MUTANTS[name])
    assert failed, f"planted mistake {name} passed every pin"


def test_oracle_passes_all_pins():
    assert failing_pins(two_pass) == []
