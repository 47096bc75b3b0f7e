"""GPU parity of the fused kernel's 128-row query tile against the fp64 oracle
(MI355X only), and of the block-size selector's choice.

The selector picks between the two compiled query-tile heights (256 and 128 rows
per workgroup). fa_fwd_blocks runs either one explicitly; these tests hold the
128-row shape to the same gates as the 256-row one (max|dLSE| <= 1e-3, max|dO| <=
1e-2 beyond the output's own bf16 rounding, max|dO| <= 2 x the bf16 unfused
yardstick's error), on every named workload (full rows for the three smaller
ones, 4096 seeded rows for the two large ones), ragged lengths, the rescale path,
and the closed forms.
"""
import math

import pytest
import torch

import attn_inputs
from parity_util import announce, assert_parity, default_scale, gpu_errors, record, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


def run_br(fa, q, k, v, scale, br):
    qg, kg, vg = to_gpu(q, k, v)
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device=qg.device)
    fa.fa_fwd_blocks(qg, kg, vg, o, lse, br, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("w", attn_inputs.WORKLOADS, ids=lambda w: w.name)
def test_workload_parity_br128(fa, w):
    announce(f"br=128 workload {w.name} B={w.B} H={w.H} N={w.N} d={w.d} seed={w.seed}")
    q, k, v = attn_inputs.make_workload(w)
    o, lse = run_br(fa, q, k, v, w.scale, 128)
    rows = None if w.full_rows else attn_inputs.rows_for(w)
    err = gpu_errors(q, k, v, o, lse, w.scale, rows=rows)
    record("fused", w.name, err, br=128)
    assert_parity(err, f"br=128 {w.name}")


@pytest.mark.parametrize("N", [1, 33, 255, 257, 513, 1000, 2049])
def test_ragged_lengths_br256_d64(fa, N):
    """The 256-row kernel at d = 64, which the selector never picks (two co-resident
    128-row workgroups win there), through fa_fwd_blocks."""
    announce(f"br=256 d=64 ragged N={N}")
    q, k, v = attn_inputs.make_qkv(2, 3, N, 64, seed=300 + N)
    o, lse = run_br(fa, q, k, v, default_scale(64), 256)
    err = gpu_errors(q, k, v, o, lse, default_scale(64))
    assert_parity(err, f"br=256 N={N} d=64", check_yardstick=N > 1)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 32, 33, 64, 65, 127, 128, 129, 255, 257, 383, 513])
def test_ragged_lengths_br128(fa, d, N):
    announce(f"br=128 ragged N={N} d={d}")
    q, k, v = attn_inputs.make_qkv(2, 3, N, d, seed=200 + N)
    o, lse = run_br(fa, q, k, v, default_scale(d), 128)
    err = gpu_errors(q, k, v, o, lse, default_scale(d))
    assert_parity(err, f"br=128 N={N} d={d}", check_yardstick=N > 1)


@pytest.mark.parametrize("d", [64, 128])
def test_ascending_scores_br128(fa, d):
    """Keys in increasing score order for the first query: the running max moves
    across the whole sequence, so the rescale path runs many times."""
    N = 2048
    announce(f"br=128 ascending scores N={N} d={d}")
    q, k, v = attn_inputs.make_qkv(1, 1, N, d, seed=9, sigma_qk=3.0)
    order = torch.argsort(k[0, 0].double() @ q[0, 0, 0].double())
    k, v = k[:, :, order].contiguous(), v[:, :, order].contiguous()
    o, lse = run_br(fa, q, k, v, default_scale(d), 128)
    assert_parity(gpu_errors(q, k, v, o, lse, default_scale(d)), "br=128 ascending")


@pytest.mark.parametrize("d", [64, 128])
def test_q_zero_br128(fa, d):
    N = 1000
    announce(f"br=128 Q=0 N={N} d={d}")
    _, k, v = attn_inputs.make_qkv(1, 2, N, d, seed=5)
    q = torch.zeros_like(k)
    o, lse = run_br(fa, q, k, v, default_scale(d), 128)
    mean = v.double().mean(dim=2, keepdim=True).expand(-1, -1, N, -1)
    assert (o.cpu().double() - mean).abs().max().item() <= 1e-2
    assert (lse.cpu().double() - math.log(N)).abs().max().item() <= 1e-3


@pytest.mark.parametrize("d", [64, 128])
def test_v_power_of_two_scaling_br128(fa, d):
    """O is linear in V and LSE does not depend on it: V scaled by 2^100 (exact in
    bf16) scales O by exactly 2^100 and leaves LSE bit-identical."""
    N = 1000
    announce(f"br=128 V scaled by 2^100 N={N} d={d}")
    q, k, v = attn_inputs.make_qkv(1, 2, N, d, seed=15, sigma_qk=2.0)
    o1, l1 = run_br(fa, q, k, v, default_scale(d), 128)
    vs = (v.float() * 2.0 ** 100).to(torch.bfloat16)
    o2, l2 = run_br(fa, q, k, vs, default_scale(d), 128)
    assert torch.equal(l1, l2)
    assert torch.equal(o2.float(), (o1.float() * 2.0 ** 100).to(torch.bfloat16).float())


def test_br128_deterministic_and_guarded(fa):
    """Two runs agree bitwise; rows past N and memory after O/LSE stay untouched."""
    N, d = 165, 64
    announce(f"br=128 determinism and guard regions N={N}")
    q, k, v = to_gpu(*attn_inputs.make_qkv(1, 2, N, d, seed=16))
    n_o, n_l = 2 * N * d, 2 * N
    obuf = torch.full((n_o + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((n_l + 1024,), 7.0, dtype=torch.float32, device="cuda")
    o, lse = obuf[:n_o].view(1, 2, N, d), lbuf[:n_l].view(1, 2, N)
    fa.fa_fwd_blocks(q, k, v, o, lse, 128)
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    fa.fa_fwd_blocks(q, k, v, o2, l2, 128)
    torch.cuda.synchronize()
    assert bool((obuf[n_o:] == 7.0).all()) and bool((lbuf[n_l:] == 7.0).all())
    assert torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 8192, 128), (1, 32, 2048, 128), (4, 16, 1024, 64), (1, 2, 300, 64)])
def test_fa_fwd_runs_the_selected_shape(fa, B, H, N, d):
    """fa_fwd equals fa_fwd_blocks at the selector's height, bitwise, and the two
    heights agree within the parity gates."""
    br, _, _ = fa.fa_select_blocks(d, N, B, H)
    announce(f"selected shape br={br} B={B} H={H} N={N} d={d}")
    q, k, v = attn_inputs.make_qkv(B, H, N, d, seed=N + d + 7)
    qg, kg, vg = to_gpu(q, k, v)
    o, lse = fa.forward(qg, kg, vg)
    ob, lb = run_br(fa, q, k, v, default_scale(d), br)
    assert torch.equal(o, ob) and torch.equal(lse, lb)
    other = 384 - br
    oo, lo = run_br(fa, q, k, v, default_scale(d), other)
    assert (lse - lo).abs().max().item() <= 2e-3
    assert (o.float() - oo.float()).abs().max().item() <= 2e-2


def test_bad_block_height_raises(fa):
    announce("br argument errors")
    q, k, v = to_gpu(*attn_inputs.make_qkv(1, 1, 64, 128, seed=14))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
    for br in (0, 64, 192, 512):
        with pytest.raises(ValueError):
            fa.fa_fwd_blocks(q, k, v, o, lse, br)
