"""GPU parity on tensors of more than 2^31 elements (over 4 GiB of bf16 each),
with one checked head at the start and one at the end: the last head begins past
element 2^31, so every offset the kernels form (head bases, rows, K/V tile
resources, the backward's row vectors) must be 64-bit to reach it.

The two checked heads hold seeded inputs; every other head holds zeros (their
outputs are defined, uniform attention, but not compared). The gates are the
other parity tests' gates."""
import numpy as np
import pytest
import torch

import attn_inputs
from parity_util import announce, assert_parity, decode_errors, default_scale, gpu_errors, record

pytestmark = pytest.mark.gpu

N = 4096
# B*H heads of N rows at head dim d: more than 2^31 elements, the last head starting past it.
SHAPES = {128: (2, 2100), 64: (2, 4200)}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


@pytest.fixture(autouse=True)
def free_memory():
    yield
    torch.cuda.empty_cache()


def checked_heads(B, H):
    return [(0, 0), (B - 1, H - 1)]


def place(shape, heads, parts):
    """A zero bf16 tensor of `shape` on the GPU with parts[i] (shape [1, 1, ...])
    copied into head heads[i]."""
    t = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    for (b, h), x in zip(heads, parts):
        t[b, h].copy_(x[0, 0])
    return t


def test_shapes_pass_2_to_the_31():
    for d, (B, H) in SHAPES.items():
        assert B * H * N * d > 2 ** 31
        assert ((B - 1) * H + (H - 1)) * N * d >= 2 ** 31


@pytest.mark.parametrize("d,br", [(128, 256), (128, 128), (64, 256), (64, 128)])
def test_forward_past_2_to_the_31(fa, d, br):
    B, H = SHAPES[d]
    announce(f"forward B={B} H={H} N={N} d={d} br={br}: heads 0 and {B * H - 1}")
    heads = checked_heads(B, H)
    inputs = [attn_inputs.make_qkv(1, 1, N, d, seed=600 + 10 * i + d) for i in range(len(heads))]
    q, k, v = (place((B, H, N, d), heads, [x[j] for x in inputs]) for j in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = default_scale(d)
    fa.fa_fwd_blocks(q, k, v, o, lse, br, scale=scale)
    torch.cuda.synchronize()
    rows = attn_inputs.sample_rows(1, 1, N, 1024, seed=700 + d + br)
    for (b, h), (qh, kh, vh) in zip(heads, inputs):
        err = gpu_errors(qh, kh, vh, o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], scale, rows=rows)
        record("forward_large", f"b{B}h{H}_n{N}_d{d}_br{br}_head{b * H + h}", err)
        assert_parity(err, f"d={d} br={br} head ({b},{h})")


@pytest.mark.parametrize("Nq", [1, 16])
def test_decode_past_2_to_the_31(fa, Nq):
    d = 128
    B, H = SHAPES[d]
    Nk = N
    announce(f"decode B={B} H={H} Nq={Nq} Nk={Nk} d={d}: heads 0 and {B * H - 1}")
    heads = checked_heads(B, H)
    inputs = [attn_inputs.make_decode_qkv(1, 1, Nq, Nk, d, seed=800 + 10 * i + Nq) for i in range(len(heads))]
    q = place((B, H, Nq, d), heads, [x[0] for x in inputs])
    k = place((B, H, Nk, d), heads, [x[1] for x in inputs])
    v = place((B, H, Nk, d), heads, [x[2] for x in inputs])
    scale = default_scale(d)
    o, lse = fa.decode_forward(q, k, v, scale=scale)
    torch.cuda.synchronize()
    for (b, h), (qh, kh, vh) in zip(heads, inputs):
        err = decode_errors(qh, kh, vh, o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], scale)
        record("decode_large", f"b{B}h{H}_q{Nq}_k{Nk}_d{d}_head{b * H + h}", err)
        assert_parity(err, f"decode Nq={Nq} head ({b},{h})")


def test_backward_past_2_to_the_31(fa):
    from test_bwd_gpu import NAMES, bwd_errors

    d = 128
    B, H = SHAPES[d]
    announce(f"backward B={B} H={H} N={N} d={d}: heads 0 and {B * H - 1}")
    heads = checked_heads(B, H)
    inputs = []
    for i in range(len(heads)):
        qh, kh, vh = attn_inputs.make_qkv(1, 1, N, d, seed=900 + i)
        g = torch.Generator().manual_seed(950 + i)
        inputs.append((qh, kh, vh, torch.randn((1, 1, N, d), generator=g).to(torch.bfloat16)))
    q, k, v, dO = (place((B, H, N, d), heads, [x[j] for x in inputs]) for j in range(4))
    scale = default_scale(d)
    o, lse = fa.forward(q, k, v, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, dO, scale=scale)
    torch.cuda.synchronize()
    del q, k, v, o, lse, dO
    for (b, h), (qh, kh, vh, gh) in zip(heads, inputs):
        grads = tuple(t[b:b + 1, h:h + 1] for t in (dq, dk, dv))
        err, unf = bwd_errors(qh, kh, vh, gh, grads, scale)
        record("backward_large", f"b{B}h{H}_n{N}_d{d}_head{b * H + h}",
               {f"max_d{n}": err[n] for n in NAMES} | {f"E_unf_{n}": unf[n] for n in NAMES})
        for n in NAMES:
            assert err[n] <= 2.0 * unf[n] + 1e-6, (b, h, n, err[n], unf[n])
