"""GPU check of the three-kernel (unfused) baseline against the fp64 oracle.

Its error should match the CPU emulation of the same bf16-input, fp32-accumulate,
16-bit-P computation (the yardstick of the fused parity gate)."""
import pytest
import torch

import attn_inputs
from parity_util import LSE_TOL, O_TOL, announce, default_scale, gpu_errors, record, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


CASES = [
    attn_inputs.WORKLOADS[0],
    attn_inputs.WORKLOADS[1],
    attn_inputs.Workload("b2h3_n1000_d128", 2, 3, 1000, 128, seed=21),
    attn_inputs.Workload("b1h2_n333_d64_wide", 1, 2, 333, 64, seed=22, sigma_qk=2.5),
    attn_inputs.Workload("b1h1_n1_d128", 1, 1, 1, 128, seed=23),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_unfused_matches_emulation(fa, w):
    announce(f"unfused {w.name}")
    q, k, v = attn_inputs.make_workload(w)
    qg, kg, vg = to_gpu(q, k, v)
    o, lse = fa.unfused_forward(qg, kg, vg, scale=w.scale)
    torch.cuda.synchronize()
    err = gpu_errors(q, k, v, o, lse, w.scale)
    record("unfused", w.name, err)
    assert err["finite"]
    assert err["max_dO_narrow"] <= O_TOL
    assert err["n_wide"] == 0 or err["max_dO_wide_beyond_rounding"] <= O_TOL
    assert err["max_dLSE"] <= LSE_TOL
    # same arithmetic as the CPU emulation up to fp32 summation order
    assert err["max_dO"] <= 1.5 * err["E_unf"] + 2 ** -8 * 0.5


def test_unfused_workspace_too_small_is_rejected(fa):
    announce("unfused workspace too small")
    q, k, v = to_gpu(*attn_inputs.make_qkv(1, 1, 64, 64, seed=24))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fa.fa_unfused_fwd(q, k, v, o, lse, ws)


def test_fused_and_unfused_agree(fa):
    w = attn_inputs.WORKLOADS[1]
    announce("fused vs unfused")
    q, k, v = to_gpu(*attn_inputs.make_workload(w))
    o1, l1 = fa.forward(q, k, v)
    o2, l2 = fa.unfused_forward(q, k, v)
    torch.cuda.synchronize()
    assert (o1.double() - o2.double()).abs().max().item() <= 2 * O_TOL
    assert (l1 - l2).abs().max().item() <= 2 * LSE_TOL
