"""Device memory of one forward: the fused path holds only Q, K, V, O and LSE, so
its peak grows with N; the unfused path adds S (fp32) and P (bf16) of every head,
so its peak grows with N^2 ("01 · 注意力为什么是 IO 瓶颈", section 6: the memory
saved at 2K and 4K sequence length, growing linearly with it).

The measured peaks (torch's allocator statistics of requested bytes; the library
allocates nothing itself) must equal bench.footprint_bytes exactly, and the CPU
tests check that model against the sizes of the tensors it names."""
import pytest
import torch

import attn_inputs
import bench
from parity_util import announce


def test_footprint_model_counts_the_tensors():
    B, H, N, d = 2, 3, 160, 64
    qkvo = 4 * B * H * N * d * 2
    lse = B * H * N * 4
    s_fp32 = B * H * N * N * 4
    p_bf16 = B * H * N * N * 2
    assert bench.footprint_bytes(B, H, N, d, fused=True) == qkvo + lse
    assert bench.footprint_bytes(B, H, N, d, fused=False) == qkvo + lse + s_fp32 + p_bf16


def test_footprint_ratio_grows_linearly_in_n():
    # unfused / fused = 1 + 6N / (8d + 4): doubling N nearly doubles the saving.
    for d in (64, 128):
        r = [bench.footprint_bytes(2, 16, n, d, False) / bench.footprint_bytes(2, 16, n, d, True)
             for n in (2048, 4096)]
        assert r[0] == pytest.approx(1 + 6 * 2048 / (8 * d + 4))
        assert r[1] - 1 == pytest.approx(2 * (r[0] - 1))


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 1024, 64), (2, 1, 512, 128)])
def test_peak_memory_matches_model(B, H, N, d):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_softmax_attn_amd as fa

    announce(f"memory B={B} H={H} N={N} d={d}")
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in attn_inputs.make_qkv(B, H, N, d, seed=N))
    for fused, fn in ((True, fa.forward), (False, fa.unfused_forward)):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        outs = fn(q, k, v)
        torch.cuda.synchronize()
        peak = torch.cuda.memory_stats(dev)["requested_bytes.all.peak"]
        del outs
        assert peak == bench.footprint_bytes(B, H, N, d, fused), (fused, peak)
