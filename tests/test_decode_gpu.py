"""GPU parity of the decode-shaped forward (few query rows against many keys)
against the fp64 oracle, with the same gates as the fused forward: max|dO| beyond
the bf16 rounding of O <= 1e-2, max|dLSE| <= 1e-3, max|dO| <= 2 x the bf16
unfused yardstick. Small shapes compare every row; the full-size workloads compare
every query row of sampled heads, in the launch configuration the benchmark times."""
import math

import numpy as np
import pytest
import torch

import attn_inputs
from attn_inputs import DecodeWorkload
from parity_util import announce, assert_parity, decode_errors, record, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


SMALL = [
    DecodeWorkload("dec_b1h1_q1_k1_d128", 1, 1, 1, 1, 128, seed=110),
    DecodeWorkload("dec_b1h1_q16_k1_d64", 1, 1, 16, 1, 64, seed=111),
    DecodeWorkload("dec_b1h2_q1_k300_d64", 1, 2, 1, 300, 64, seed=112),
    DecodeWorkload("dec_b2h3_q4_k1000_d128", 2, 3, 4, 1000, 128, seed=113),
    DecodeWorkload("dec_b1h2_q3_k129_d128", 1, 2, 3, 129, 128, seed=114),
    DecodeWorkload("dec_b1h2_q5_k777_d64", 1, 2, 5, 777, 64, seed=115),
    DecodeWorkload("dec_b3h1_q9_k257_d64", 3, 1, 9, 257, 64, seed=116),
    DecodeWorkload("dec_b1h4_q16_k4096_d128", 1, 4, 16, 4096, 128, seed=117),
    DecodeWorkload("dec_b2h2_q2_k20000_d128_wide", 2, 2, 2, 20000, 128, seed=118, sigma_qk=2.5),
    DecodeWorkload("dec_b1h1_q8_k65537_d64_wide", 1, 1, 8, 65537, 64, seed=119, sigma_qk=2.5),
]


def run_decode(fa, w, q, k, v):
    qg, kg, vg = to_gpu(q, k, v)
    o, lse = fa.decode_forward(qg, kg, vg, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("w", SMALL + list(attn_inputs.DECODE_WORKLOADS), ids=lambda w: w.name)
def test_decode_parity(fa, w):
    splits, chunk, _ = fa.fa_decode_plan(w.B, w.H, w.Nq, w.Nk, w.d)
    announce(f"decode {w.name} splits={splits} chunk={chunk}")
    q, k, v = attn_inputs.make_decode_workload(w)
    o, lse = run_decode(fa, w, q, k, v)
    heads = None
    if w.check_heads:
        heads = attn_inputs.sample_heads(w.B, w.H, w.check_heads, seed=2000 + w.seed)
    err = decode_errors(q, k, v, o, lse, w.scale, heads=heads)
    record("decode", w.name, err, splits=splits, chunk=chunk)
    assert_parity(err, w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq", list(range(1, 17)))
def test_decode_every_row_count(fa, d, Nq):
    """Every row count the decode path takes (the vector kernel at one row, the
    matrix-core kernel, rows padded to 16, from two on), with a key count that is no
    multiple of a chunk or a 32-key tile and a few heads, against the oracle."""
    Nk = 997 + 37 * Nq
    w = DecodeWorkload(f"rows_q{Nq}_k{Nk}_d{d}", 2, 3, Nq, Nk, d, seed=200 + Nq + d)
    announce(f"decode every row count {w.name}")
    q, k, v = attn_inputs.make_decode_workload(w)
    o, lse = run_decode(fa, w, q, k, v)
    assert_parity(decode_errors(q, k, v, o, lse, w.scale), w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 777), (4, 3000), (16, 5000)])
def test_decode_negative_scale(fa, d, Nq, Nk):
    """A negative scale: the softmax of the negated scores, against the oracle."""
    w = DecodeWorkload(f"neg_q{Nq}_k{Nk}_d{d}", 1, 2, Nq, Nk, d, seed=130 + Nq)
    announce(f"decode negative scale {w.name}")
    q, k, v = attn_inputs.make_decode_workload(w)
    qg, kg, vg = to_gpu(q, k, v)
    scale = -1.0 / math.sqrt(d)
    o, lse = fa.decode_forward(qg, kg, vg, scale=scale)
    torch.cuda.synchronize()
    assert_parity(decode_errors(q, k, v, o, lse, scale), w.name)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_zero_queries_average_values(fa, d):
    """Q = 0: every score is 0, so O is the mean of the Nk value rows and LSE = ln Nk."""
    announce(f"decode q=0 d={d}")
    q, k, v = attn_inputs.make_decode_qkv(2, 2, 3, 5000, d, seed=120)
    q = torch.zeros_like(q)
    w = DecodeWorkload("zero", 2, 2, 3, 5000, d, seed=120)
    o, lse = run_decode(fa, w, q, k, v)
    mean = attn_inputs.bf16_to_f64(v).mean(axis=2, keepdims=True)
    dO = np.abs(o.cpu().double().numpy() - mean)
    assert dO.max() <= 1e-2
    np.testing.assert_allclose(lse.cpu().double().numpy(), math.log(5000), atol=1e-3)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_v_power_of_two_scaling_is_exact(fa, d):
    """Scaling V by 2^40 scales every fp32 product and sum exactly, and bf16 rounding
    commutes with it: O scales exactly, LSE does not change."""
    announce(f"decode V*2^40 d={d}")
    w = DecodeWorkload("scale", 1, 3, 4, 3000, d, seed=121)
    q, k, v = attn_inputs.make_decode_workload(w)
    o1, l1 = run_decode(fa, w, q, k, v)
    o2, l2 = run_decode(fa, w, q, k, (v.float() * 2.0 ** 40).to(torch.bfloat16))
    assert torch.equal(l1, l2)
    assert torch.equal(o1.float() * 2.0 ** 40, o2.float())


def test_decode_is_deterministic_and_stream_aware(fa):
    announce("decode determinism, side stream")
    w = DecodeWorkload("det", 2, 4, 2, 9000, 128, seed=122)
    q, k, v = (t.cuda() for t in attn_inputs.make_decode_workload(w))
    o1, l1 = fa.decode_forward(q, k, v, scale=w.scale)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, l2 = fa.decode_forward(q, k, v, scale=w.scale, stream=side)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_workspace_reuse_across_shapes(fa):
    """One workspace, large enough for both, serves two different shapes in a row;
    the second (smaller) result must not depend on what the first left behind."""
    announce("decode workspace reuse")
    shapes = [DecodeWorkload("big", 2, 8, 16, 6000, 128, seed=123),
              DecodeWorkload("small", 1, 3, 2, 700, 64, seed=124)]
    need = max(fa.fa_decode_plan(w.B, w.H, w.Nq, w.Nk, w.d)[2] for w in shapes)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for w in shapes:
        q, k, v = attn_inputs.make_decode_workload(w)
        qg, kg, vg = to_gpu(q, k, v)
        o = torch.empty_like(qg)
        lse = torch.empty(qg.shape[:3], dtype=torch.float32, device="cuda")
        fa.fa_decode_fwd(qg, kg, vg, o, lse, ws, scale=w.scale)
        torch.cuda.synchronize()
        assert_parity(decode_errors(q, k, v, o, lse, w.scale), w.name)


def test_decode_rejects_bad_arguments(fa):
    q = torch.zeros(1, 1, 17, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 100, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.decode_forward(q, k, k)  # Nq = 17 > 16
    q = torch.zeros(1, 1, 2, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 2, dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fa.fa_decode_fwd(q, k, k, o, lse, ws)  # workspace too small
