"""Pins for the fp64 backward oracle (CPU only, no GPU).

The gradients are checked against things other than the oracle's own formulas:
central finite differences of the forward oracle, torch's autograd through its
own fp64 softmax, closed forms (scale = 0, dO = 0), and the invariants the
softmax Jacobian implies (the rows of dS sum to zero, so the key gradients sum to
zero; the rows of P sum to one, so the value gradients sum to the upstream rows).
Planted mistakes in copies of the oracle must each fail a pin."""
import json
import math
import os

import numpy as np
import pytest
import torch

import attn_inputs
from oracle import attention_backward_fp64, attention_backward_unfused_bf16, attention_fp64

TOL = 1e-10


def rand(B, H, N, d, seed, sigma=1.0, nk=None):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, H, N, d)) * sigma
    k = g.standard_normal((B, H, nk or N, d)) * sigma
    v = g.standard_normal((B, H, nk or N, d))
    dO = g.standard_normal((B, H, N, d))
    return q, k, v, dO


def check_finite_differences(impl):
    """dL/dX for L = sum(O * dO), by central differences of the forward oracle."""
    for (N, nk, d, sigma, seed) in ((4, 4, 3, 1.0, 1), (3, 6, 2, 2.0, 2), (5, 2, 4, 1.5, 3)):
        q, k, v, dO = rand(1, 1, N, d, seed, sigma, nk)
        scale = 0.7
        dQ, dK, dV = impl(q, k, v, dO, scale)
        h = 1e-6
        for arr, grad in ((q, dQ), (k, dK), (v, dV)):
            num = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = arr[idx]
                arr[idx] = old + h
                lp = (attention_fp64(q, k, v, scale)[0] * dO).sum()
                arr[idx] = old - h
                lm = (attention_fp64(q, k, v, scale)[0] * dO).sum()
                arr[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(grad, num, atol=1e-7, rtol=1e-6)


def check_autograd(impl):
    """torch's autograd through torch.softmax and matmul, in fp64."""
    q, k, v, dO = rand(2, 2, 9, 5, seed=4, sigma=1.5, nk=13)
    scale = 0.45
    dQ, dK, dV = impl(q, k, v, dO, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.matmul(torch.softmax(scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous()), dim=-1), tv)
    o.backward(torch.tensor(dO))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=TOL)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=TOL)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=TOL)


def check_scale_zero(impl):
    """scale = 0: P is uniform (1/Nk) and no gradient reaches Q or K; every value
    row receives the mean of the upstream rows."""
    q, k, v, dO = rand(1, 2, 6, 4, seed=5, nk=10)
    dQ, dK, dV = impl(q, k, v, dO, 0.0)
    np.testing.assert_allclose(dQ, 0.0, atol=TOL)
    np.testing.assert_allclose(dK, 0.0, atol=TOL)
    np.testing.assert_allclose(dV, np.broadcast_to(dO.sum(axis=2, keepdims=True) / 10, dV.shape), atol=TOL)


def check_zero_upstream(impl):
    q, k, v, dO = rand(1, 1, 7, 3, seed=6)
    for g in impl(q, k, v, np.zeros_like(dO), 0.5):
        np.testing.assert_allclose(g, 0.0, atol=TOL)


def check_sums(impl):
    """sum_j dK_j = 0 (rows of dS sum to zero); sum_j dV_j = sum_i dO_i (rows of P sum to one)."""
    q, k, v, dO = rand(2, 1, 11, 6, seed=7, sigma=2.0, nk=17)
    dQ, dK, dV = impl(q, k, v, dO, 0.4)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-10)
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=2), atol=1e-10)


def check_single_key(impl):
    """Nk = 1: P = 1, so dV = sum_i dO_i and dS = 0 (no gradient to Q or K)."""
    q, k, v, dO = rand(1, 1, 5, 3, seed=8, nk=1)
    dQ, dK, dV = impl(q, k, v, dO, 0.9)
    np.testing.assert_allclose(dQ, 0.0, atol=TOL)
    np.testing.assert_allclose(dK, 0.0, atol=TOL)
    np.testing.assert_allclose(dV[0, 0, 0], dO[0, 0].sum(axis=0), atol=TOL)


PINS = [check_finite_differences, check_autograd, check_scale_zero, check_zero_upstream, check_sums,
        check_single_key]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(attention_backward_fp64)


def _mutant(kind):
    def impl(q, k, v, dO, scale):
        B, H, N, d = q.shape
        dQ, dK, dV = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        for b in range(B):
            for h in range(H):
                Q, K, V, G = q[b, h], k[b, h], v[b, h], dO[b, h]
                S = scale * Q @ K.T
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E if kind == "unnormalised_p" else E / E.sum(axis=1, keepdims=True)
                dV[b, h] = (P @ G[: P.shape[1]] if kind == "untransposed_p" and P.shape[0] == P.shape[1]
                            else P.T @ G)
                dP = G @ V.T
                D = 0.0 if kind == "no_row_term" else (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - D)
                dQ[b, h] = (1.0 if kind == "dq_unscaled" else scale) * (dS @ K)
                dK[b, h] = scale * ((dS @ Q[: dS.shape[1]]) if kind == "dk_untransposed" and dS.shape[0] == dS.shape[1]
                                    else dS.T @ Q)
        return dQ, dK, dV
    return impl


MUTANTS = ["unnormalised_p", "untransposed_p", "no_row_term", "dq_unscaled", "dk_untransposed"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_backward_planted_mistakes_are_caught(kind):
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_mutant(kind))
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {kind} passed every pin"


YARDSTICK = os.path.join(os.path.dirname(__file__), "golden", "yardstick_cases.json")


def check_yardstick_golden(impl):
    """The hand-derived backward cases of tests/golden/yardstick_cases.json: every
    fp32 step is exact there, so the bf16 rounding of P, of dS and of the three
    outputs each decide the expected bits, and dP or D rounded to bf16 would
    change them."""
    with open(YARDSTICK) as f:
        cases = json.load(f)["backward"]
    for c in cases:
        ins = [torch.tensor(c[n], dtype=torch.float32).to(torch.bfloat16)[None, None]
               for n in ("q", "k", "v", "o", "dO")]
        for t, n in zip(ins, ("q", "k", "v", "o", "dO")):
            assert torch.equal(t.float()[0, 0], torch.tensor(c[n], dtype=torch.float32)), "inputs must be bf16"
        got = impl(*ins, c["scale"])
        for g, n in zip(got, ("dQ", "dK", "dV")):
            np.testing.assert_array_equal(g[0, 0], np.array(c[n]), err_msg=f"{c['name']} {n}")


def check_yardstick_close(impl):
    """Random inputs: within bf16-level relative error of the fp64 oracle, and not
    equal to it (the 16-bit P and dS introduce error)."""
    q, k, v = attn_inputs.make_qkv(1, 2, 200, 64, seed=61)
    g = torch.Generator().manual_seed(62)
    dO = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    scale = 0.125
    f = attn_inputs.bf16_to_f64
    o = torch.tensor(attention_fp64(f(q), f(k), f(v), scale)[0]).to(torch.bfloat16)
    ref = attention_backward_fp64(f(q), f(k), f(v), f(dO), scale)
    emu = impl(q, k, v, o, dO, scale)
    for r, e in zip(ref, emu):
        scale_r = np.abs(r).max()
        err = np.abs(e - r).max()
        assert 0 < err <= 0.02 * scale_r, (err, scale_r)


YARDSTICK_PINS = [check_yardstick_golden, check_yardstick_close]


def test_backward_unfused_bf16_pins():
    for pin in YARDSTICK_PINS:
        pin(attention_backward_unfused_bf16)


def _yardstick_mutant(kind):
    """Copies of the backward yardstick with one plausible mistake at a rounding point."""
    def impl(q, k, v, o, dO, scale):
        out = [np.empty(tuple(t.shape)) for t in (q, k, v)]
        sc = torch.tensor(scale, dtype=torch.float32)
        rnd = (lambda t: t) if kind == "outputs_fp32" else (lambda t: t.to(torch.bfloat16))
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                Q, K, V, O, G = (t[b, h].float() for t in (q, k, v, o, dO))
                S = (Q @ K.T) * sc
                E = torch.exp(S - S.max(dim=1, keepdim=True).values)
                P = E / E.sum(dim=1, keepdim=True)
                if kind != "p_fp32":
                    P = P.to(torch.bfloat16).float()
                dV = rnd(P.T @ G)
                dP = G @ V.T
                if kind == "dp_bf16":
                    dP = dP.to(torch.bfloat16).float()
                D = (G * O).sum(dim=1, keepdim=True)
                dS = P * (dP - D)
                if kind != "ds_fp32":
                    dS = dS.to(torch.bfloat16).float()
                dQ = rnd((dS @ K) * sc)
                dK = rnd((dS.T @ Q) * sc)
                for arr, t in zip(out, (dQ, dK, dV)):
                    arr[b, h] = t.double().numpy()
        return tuple(out)
    return impl


@pytest.mark.parametrize("kind", ["p_fp32", "ds_fp32", "dp_bf16", "outputs_fp32"])
def test_backward_yardstick_planted_mistakes_are_caught(kind):
    failed = []
    for pin in YARDSTICK_PINS:
        try:
            pin(_yardstick_mutant(kind))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"yardstick mistake {kind} passed every pin"
