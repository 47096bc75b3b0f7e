"""GPU parity on seeded random shapes, beside the hand-picked cases of the other
tests: each case draws B, H, the lengths, the head dimension, the scale (the
default 1/sqrt(d) or a random one of either sign) and the score spread from a
generator seeded with its index, so the set is fixed and every case can be rerun
alone. The gates are the other parity tests' gates."""
import math

import numpy as np
import pytest
import torch

import attn_inputs
from parity_util import announce, assert_parity, decode_errors, gpu_errors, record

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


def log_uniform(rng, lo, hi):
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def draw(seed):
    """(d, scale, sigma_qk) of a case."""
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128]))
    scale = 1.0 / math.sqrt(d) if rng.random() < 0.5 else float(rng.uniform(-0.25, 0.25))
    sigma = float(rng.choice([1.0, 2.5]))
    return rng, d, scale, sigma


@pytest.mark.parametrize("case", range(16))
def test_forward_random_shape(fa, case):
    rng, d, scale, sigma = draw(5000 + case)
    B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3, 5]))
    N = log_uniform(rng, 8, 12000)
    name = f"rand{case}_b{B}h{H}_n{N}_d{d}_s{scale:+.4f}_sig{sigma}"
    announce(f"forward random {name}")
    q, k, v = attn_inputs.make_qkv(B, H, N, d, seed=6000 + case, sigma_qk=sigma)
    rows = None if B * H * N <= 2048 else attn_inputs.sample_rows(B, H, N, 256, seed=7000 + case)
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    for br in (256, 128):
        o = torch.empty_like(qg)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        fa.fa_fwd_blocks(qg, kg, vg, o, lse, br, scale=scale)
        torch.cuda.synchronize()
        err = gpu_errors(q, k, v, o, lse, scale, rows=rows)
        record("forward_random", f"{name}_br{br}", err)
        assert_parity(err, f"{name} br={br}")


@pytest.mark.parametrize("case", range(10))
def test_decode_random_shape(fa, case):
    rng, d, scale, sigma = draw(5100 + case)
    B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3]))
    Nq, Nk = int(rng.integers(1, 17)), log_uniform(rng, 1, 40000)
    name = f"rand{case}_b{B}h{H}_q{Nq}_k{Nk}_d{d}_s{scale:+.4f}_sig{sigma}"
    announce(f"decode random {name}")
    q, k, v = attn_inputs.make_decode_qkv(B, H, Nq, Nk, d, seed=6100 + case, sigma_qk=sigma)
    o, lse = fa.decode_forward(q.cuda(), k.cuda(), v.cuda(), scale=scale)
    torch.cuda.synchronize()
    err = decode_errors(q, k, v, o, lse, scale)
    record("decode_random", name, err)
    assert_parity(err, name)


@pytest.mark.parametrize("case", range(6))
def test_backward_random_shape(fa, case):
    from test_bwd_gpu import NAMES, bwd_errors

    rng, d, scale, sigma = draw(5200 + case)
    B, H = 1, int(rng.integers(1, 3))
    N = log_uniform(rng, 40, 1200)
    name = f"rand{case}_b{B}h{H}_n{N}_d{d}_s{scale:+.4f}_sig{sigma}"
    announce(f"backward random {name}")
    q, k, v = attn_inputs.make_qkv(B, H, N, d, seed=6200 + case, sigma_qk=sigma)
    g = torch.Generator().manual_seed(6300 + case)
    dO = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    qg, kg, vg, gg = (t.cuda() for t in (q, k, v, dO))
    o, lse = fa.forward(qg, kg, vg, scale=scale)
    grads = fa.backward(qg, kg, vg, o, lse, gg, scale=scale)
    torch.cuda.synchronize()
    err, unf = bwd_errors(q, k, v, dO, grads, scale)
    record("backward_random", name, {f"max_d{n}": err[n] for n in NAMES} | {f"E_unf_{n}": unf[n] for n in NAMES})
    for n in NAMES:
        assert err[n] <= 2.0 * unf[n] + 1e-6, (name, n, err[n], unf[n])
