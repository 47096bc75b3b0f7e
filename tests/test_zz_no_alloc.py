"""The allocation-free decode entry point, fa_decode_fwd_noalloc, through the C ABI.

It runs fa_decode_fwd's kernels with the key split's partial results in the
library's fixed per-GPU scratch array instead of a caller workspace, so its O and
LSE must equal fa_decode_fwd's bit for bit; they are also checked against the fp64
oracle with the decode gates. Two calls in a row: the first fills most of the
array, the second, smaller one must not see what the first left there."""
import math

import pytest
import torch

import attn_inputs
from attn_inputs import DecodeWorkload
from parity_util import announce, assert_parity, decode_errors, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as mod
    return mod


# The first shape puts one key chunk on each of 3072 heads: 3072 * 16 rows of
# (128 + 1) fp32 partials, 25.4 MB of the 32 MiB array. The second is small and
# ragged (three query rows, 777 keys, several chunks per head).
CALLS = [
    DecodeWorkload("noalloc_b64h48_q16_k256_d128", 64, 48, 16, 256, 128, seed=140, check_heads=6),
    DecodeWorkload("noalloc_b2h3_q3_k777_d64", 2, 3, 3, 777, 64, seed=141),
]


def test_noalloc_decode_matches_workspace_entry_point(fa):
    for w in CALLS:
        splits, chunk, need = fa.fa_decode_plan(w.B, w.H, w.Nq, w.Nk, w.d)
        assert need <= fa.DECODE_SCRATCH_BYTES
        announce(f"decode noalloc {w.name} splits={splits} chunk={chunk} scratch bytes={need}")
        q, k, v = attn_inputs.make_decode_workload(w)
        qg, kg, vg = to_gpu(q, k, v)
        scale = 1.0 / math.sqrt(w.d)
        o_ws, l_ws = fa.decode_forward(qg, kg, vg, scale=scale)
        o = torch.full_like(qg, float("nan"))
        lse = torch.full(qg.shape[:3], float("nan"), dtype=torch.float32, device=qg.device)
        fa.fa_decode_fwd_noalloc(qg, kg, vg, o, lse, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws) and torch.equal(lse, l_ws), w.name
        heads = attn_inputs.sample_heads(w.B, w.H, w.check_heads, seed=3000 + w.seed) if w.check_heads else None
        assert_parity(decode_errors(q, k, v, o, lse, scale, heads=heads), w.name)


def test_noalloc_decode_rejects_a_shape_beyond_the_array(fa):
    announce("decode noalloc: shape beyond the scratch array")
    B, H, Nq, Nk, d = 64, 64, 16, 256, 128
    assert fa.fa_decode_plan(B, H, Nq, Nk, d)[2] > fa.DECODE_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        fa.fa_decode_fwd_noalloc(q, k, k, o, lse)


def test_noalloc_decode_graph_replays(fa):
    """The allocation-free decode is meant for code under graph capture: capture one
    call, then replay it with new inputs copied into the captured buffers, with an
    eager call of another shape in between (which rewrites the scratch array), and
    compare each replay with fa_decode_fwd on the same inputs, bit for bit."""
    B, H, Nq, Nk, d = 4, 8, 6, 3000, 128
    announce(f"graph fa_decode_fwd_noalloc B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    q, k, v = to_gpu(*attn_inputs.make_decode_qkv(B, H, Nq, Nk, d, seed=150))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_decode_fwd_noalloc(q, k, v, o, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_decode_fwd_noalloc(q, k, v, o, lse)
    torch.cuda.synchronize()
    oq, ok_, ov = to_gpu(*attn_inputs.make_decode_qkv(2, 3, 1, 5000, 64, seed=151))
    for rep in range(3):
        fresh = attn_inputs.make_decode_qkv(B, H, Nq, Nk, d, seed=160 + rep)
        for dst, src in zip((q, k, v), fresh):
            dst.copy_(src)
        fa.decode_forward(oq, ok_, ov)  # another shape through the workspace entry point
        fa.fa_decode_fwd_noalloc(oq, ok_, ov, torch.empty_like(oq),
                                 torch.empty((2, 3, 1), dtype=torch.float32, device="cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = fa.decode_forward(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep}"
