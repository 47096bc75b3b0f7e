"""GPU parity of the attention backward (dQ, dK, dV) against the fp64 oracle.

The pages state no tolerance for gradients. The gate is the forward's second
gate carried over: each gradient's max |error| against the fp64 oracle is at most
twice that of the bf16 unfused backward (bf16 inputs, fp32 products, P and dS
stored as bf16, outputs rounded to bf16), computed on the CPU on the same inputs
with the oracle's O. The GPU backward runs on the GPU forward's O and LSE, the
way it is used. Small shapes compare every row; the full-size shape compares two
sampled heads."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import attention_backward_fp64, attention_backward_unfused_bf16, attention_fp64
from parity_util import announce, record, to_gpu

pytestmark = pytest.mark.gpu

NAMES = ("dQ", "dK", "dV")


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


def make_case(B, H, N, d, seed, sigma=1.0):
    q, k, v = attn_inputs.make_qkv(B, H, N, d, seed, sigma_qk=sigma)
    g = torch.Generator().manual_seed(seed + 7919)
    dO = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    return q, k, v, dO


def bwd_errors(q, k, v, dO, grads, scale, heads=None):
    """Max |error| per gradient against the oracle and the bf16 yardstick's, over
    ``heads`` ((b, h) pairs; None = all)."""
    f = attn_inputs.bf16_to_f64
    B, H = q.shape[:2]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    err = {n: 0.0 for n in NAMES}
    unf = {n: 0.0 for n in NAMES}
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qh, kh, vh, gh = (t[sl] for t in (q, k, v, dO))
        ref = attention_backward_fp64(f(qh), f(kh), f(vh), f(gh), scale)
        o_ref = torch.tensor(attention_fp64(f(qh), f(kh), f(vh), scale)[0]).to(torch.bfloat16)
        emu = attention_backward_unfused_bf16(qh, kh, vh, o_ref, gh, scale)
        for n, r, e, gpu in zip(NAMES, ref, emu, grads):
            x = gpu[sl].detach().cpu().double().numpy()
            assert np.isfinite(x).all(), n
            err[n] = max(err[n], float(np.abs(x - r).max()))
            unf[n] = max(unf[n], float(np.abs(e - r).max()))
    return err, unf


def run_bwd(fa, q, k, v, dO, scale):
    qg, kg, vg, gg = to_gpu(q, k, v, dO)
    o, lse = fa.forward(qg, kg, vg, scale=scale)
    grads = fa.backward(qg, kg, vg, o, lse, gg, scale=scale)
    torch.cuda.synchronize()
    return grads


CASES = [(1, 1, 64, 64, 1, 1.0), (1, 2, 300, 128, 2, 1.0), (2, 3, 1000, 64, 3, 1.0), (1, 1, 1, 128, 4, 1.0),
         (1, 2, 129, 128, 5, 2.5), (1, 4, 2048, 128, 6, 1.0), (2, 1, 777, 64, 7, 2.5),
         # ragged last key tile in each position of the four-stage ring (full tiles mod 4 = 2, 3)
         (1, 2, 327, 128, 8, 1.0), (1, 1, 69, 64, 9, 2.5), (1, 1, 97, 128, 10, 1.0)]


@pytest.mark.parametrize("B,H,N,d,seed,sigma", CASES)
def test_bwd_parity(fa, B, H, N, d, seed, sigma):
    announce(f"bwd B={B} H={H} N={N} d={d} sigma={sigma}")
    scale = 1.0 / np.sqrt(d)
    q, k, v, dO = make_case(B, H, N, d, seed, sigma)
    grads = run_bwd(fa, q, k, v, dO, scale)
    err, unf = bwd_errors(q, k, v, dO, grads, scale)
    record("backward", f"b{B}h{H}_n{N}_d{d}_s{sigma}", {f"max_d{n}": err[n] for n in NAMES} |
           {f"E_unf_{n}": unf[n] for n in NAMES})
    for n in NAMES:
        assert err[n] <= 2.0 * unf[n] + 1e-6, (n, err[n], unf[n])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [2, 5, 16, 31, 32, 33, 48, 63, 65, 95, 96, 100, 127, 128, 130, 160, 161, 191, 193, 250])
def test_bwd_short_lengths(fa, d, N):
    """Short and ragged sequences: few 32-row or 32-key tiles, so the kernels run
    only (or mostly) the remainder steps of their loops unrolled over the ring."""
    announce(f"bwd short N={N} d={d}")
    scale = 1.0 / np.sqrt(d)
    q, k, v, dO = make_case(1, 2, N, d, 300 + N + d)
    grads = run_bwd(fa, q, k, v, dO, scale)
    err, unf = bwd_errors(q, k, v, dO, grads, scale)
    for n in NAMES:
        assert err[n] <= 2.0 * unf[n] + 1e-6, (N, d, n, err[n], unf[n])


def test_bwd_parity_full_size_sampled_heads(fa):
    """The benchmark shape, B=1 H=32 N=8192 d=128: two sampled heads against the oracle."""
    announce("bwd B=1 H=32 N=8192 d=128, heads 0 and 31")
    w = attn_inputs.HEADLINE
    q, k, v, dO = make_case(w.B, w.H, w.N, w.d, w.seed)
    grads = run_bwd(fa, q, k, v, dO, w.scale)
    err, unf = bwd_errors(q, k, v, dO, grads, w.scale, heads=[(0, 0), (0, 31)])
    record("backward", f"{w.name}_heads_0_31", {f"max_d{n}": err[n] for n in NAMES} |
           {f"E_unf_{n}": unf[n] for n in NAMES})
    for n in NAMES:
        assert err[n] <= 2.0 * unf[n] + 1e-6, (n, err[n], unf[n])


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_negative_scale(fa, d):
    """A negative scale: the gradients of the softmax of the negated scores."""
    announce(f"bwd negative scale d={d}")
    scale = -1.0 / np.sqrt(d)
    q, k, v, dO = make_case(1, 2, 333, d, 400 + d, 2.0)
    grads = run_bwd(fa, q, k, v, dO, scale)
    err, unf = bwd_errors(q, k, v, dO, grads, scale)
    for n in NAMES:
        assert err[n] <= 2.0 * unf[n] + 1e-6, (n, err[n], unf[n])


def test_bwd_sums(fa):
    """The key gradients of a head sum to zero and the value gradients to the sum of
    the upstream rows (rows of dS sum to zero, rows of P to one), up to rounding."""
    announce("bwd sums")
    q, k, v, dO = make_case(1, 2, 500, 64, seed=11)
    dq, dk, dv = run_bwd(fa, q, k, v, dO, 0.125)
    sdk = dk.double().sum(dim=2).abs().max().item()
    sdv = (dv.double().sum(dim=2) - dO.double().cuda().sum(dim=2)).abs().max().item()
    assert sdk <= 0.02 * dk.double().abs().max().item() * 500 ** 0.5
    assert sdv <= 0.02 * dv.double().abs().max().item() * 500 ** 0.5


def test_bwd_deterministic(fa):
    announce("bwd determinism")
    q, k, v, dO = make_case(1, 3, 700, 128, seed=12)
    g1 = run_bwd(fa, q, k, v, dO, 0.088)
    g2 = run_bwd(fa, q, k, v, dO, 0.088)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_concurrent_side_streams(fa):
    """Two backward calls (d = 128 and d = 64, so both dK/dV kernels) enqueued on two
    side streams at once give the same bits as the same calls run one after the other
    on the current stream."""
    announce("bwd on two side streams")
    cases = [make_case(1, 4, 1000, 128, seed=13), make_case(2, 2, 777, 64, seed=14)]
    want = [run_bwd(fa, q, k, v, dO, None) for (q, k, v, dO) in cases]
    gpu = [to_gpu(*c) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = []
    for s, (q, k, v, dO) in zip(streams, gpu):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            o, lse = fa.forward(q, k, v, stream=s)
            got.append(fa.backward(q, k, v, o, lse, dO, stream=s))
    torch.cuda.synchronize()
    for w, g in zip(want, got):
        for a, b in zip(w, g):
            assert torch.equal(a, b)
