"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/fa.h, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def fa():
    import io_aware_softmax_attn_amd as mod
    return mod


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_unfused_fwd", "fa_unfused_workspace_bytes", "fa_select_blocks", "fa_check_args",
              "fa_status_string", "fa_version", "fa_decode_fwd", "fa_decode_plan", "fa_decode_check_args",
              "fa_fwd_tile_order", "fa_bwd", "fa_bwd_workspace_bytes", "fa_decode_fwd_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(fa):
    dll = ctypes.CDLL(fa.build.LIB_PATH)
    for n in declared_functions():
        assert hasattr(dll, n), f"libfa.so does not export {n}"


def test_exported_symbols_are_c_linkage(fa):
    nm = shutil.which("nm") or "/usr/bin/nm"
    out = subprocess.run([nm, "-D", "--defined-only", fa.build.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(fa_[a-z_0-9]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(fa):
    assert fa.fa_version() >= 10000
    for name, code in fa.STATUS.items():
        s = fa.fa_status_string(code)
        assert s and s != "unknown status", name
    assert fa.fa_status_string(12345) == "unknown status"


def test_select_blocks(fa):
    for d in (64, 128):
        for B, H, N in ((1, 1, 1), (1, 1, 8192), (4, 16, 1024), (1, 32, 8192), (1, 8, 30001), (64, 64, 65536)):
            br, bc, nw = fa.fa_select_blocks(d, N, B, H)
            assert br in (128, 256) and bc == 64 and nw == 4, (d, B, H, N)
            assert br == fa.fa_select_blocks(d, N, B, H)[0]  # a function of the shape
        # LDS budget: four K/V stages fit the 160 KB of a CU
        assert 4 * 2 * bc * d * 2 <= 160 * 1024
    # The benchmark shape fills the chip four times over with 256-row tiles: keep them.
    assert fa.fa_select_blocks(128, 8192, 1, 32)[0] == 256
    # One head of 8192 rows makes 32 tiles of 256 rows for 256 CUs: take 128 rows.
    assert fa.fa_select_blocks(128, 8192, 1, 1)[0] == 128
    # The choices the graph-timed recheck of the model confirmed, (d, N, B, H) -> rows.
    measured = {(128, 8192, 1, 32): 256, (128, 4096, 2, 16): 256, (128, 30001, 1, 8): 256, (128, 2048, 1, 32): 256,
                (128, 8192, 1, 4): 128, (128, 16384, 1, 1): 128, (64, 256, 1, 1): 128, (64, 1024, 4, 16): 128,
                (64, 2048, 4, 16): 128, (64, 2048, 2, 8): 128}
    for (d, N, B, H), br in measured.items():
        assert fa.fa_select_blocks(d, N, B, H)[0] == br, (d, N, B, H)
    with pytest.raises(ValueError):
        fa.fa_select_blocks(96, 128)
    with pytest.raises(ValueError):
        fa.fa_select_blocks(128, -1)


def test_workspace_bytes(fa):
    for B, H, N in ((1, 1, 256), (4, 16, 1024), (1, 8, 30001), (2, 3, 1)):
        ns = (N + 63) // 64 * 64
        want = (6 * B * H * N * ns + 255) // 256 * 256
        assert fa.fa_unfused_workspace_bytes(B, H, N) == want
    assert fa.fa_unfused_workspace_bytes(-1, 1, 1) == 0
    assert fa.fa_unfused_workspace_bytes(2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1) == 0


A = 1 << 20  # fake, well-separated, aligned addresses: validation never dereferences


def ptrs(n=1 << 12):
    return [A, 2 * A, 3 * A, 4 * A, 5 * A]


def check(fa, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=2, N=64, d=128, scale=0.1, ws=0, wsp=None, wsb=0):
    return fa.fa_check_args(q, k, v, o, lse, B, H, N, d, scale, ws, wsp, wsb)


def test_check_args_ok(fa):
    assert check(fa) == 0
    assert check(fa, q=A, k=A, v=A) == 0  # inputs may share memory
    assert check(fa, scale=0.0) == 0


def test_check_args_errors(fa):
    S = fa.STATUS
    assert check(fa, B=-1) == S["FA_ERR_SHAPE"]
    assert check(fa, N=-5) == S["FA_ERR_SHAPE"]
    assert check(fa, d=96) == S["FA_ERR_HEADDIM"]
    assert check(fa, d=256) == S["FA_ERR_HEADDIM"]
    assert check(fa, scale=float("nan")) == S["FA_ERR_SCALE"]
    assert check(fa, scale=float("inf")) == S["FA_ERR_SCALE"]
    assert check(fa, scale=-0.5) == 0  # any finite scale: softmax of the negated scores
    assert check(fa, q=None) == S["FA_ERR_NULL"]
    assert check(fa, lse=None) == S["FA_ERR_NULL"]
    assert check(fa, q=A + 8) == S["FA_ERR_ALIGN"]
    assert check(fa, o=4 * A + 4) == S["FA_ERR_ALIGN"]
    assert check(fa, lse=5 * A + 2) == S["FA_ERR_ALIGN"]
    assert check(fa, o=A) == S["FA_ERR_ALIAS"]
    assert check(fa, o=A + 16) == S["FA_ERR_ALIAS"]  # partial overlap with q
    assert check(fa, lse=4 * A + 64) == S["FA_ERR_ALIAS"]  # inside o
    assert check(fa, B=1 << 30, H=1 << 30, N=1 << 30) == S["FA_ERR_OVERFLOW"]
    assert check(fa, B=1 << 16, H=1 << 16, N=1 << 20) == S["FA_ERR_OVERFLOW"]  # grid too large


def test_check_args_empty_problem_ignores_pointers(fa):
    assert check(fa, q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert check(fa, q=None, k=None, v=None, o=None, lse=None, B=0) == 0


def test_check_args_workspace(fa):
    S = fa.STATUS
    need = fa.fa_unfused_workspace_bytes(1, 2, 64)
    W = 16 * A
    assert check(fa, ws=1, wsp=W, wsb=need) == 0
    assert check(fa, ws=1, wsp=None, wsb=need) == S["FA_ERR_WORKSPACE"]
    assert check(fa, ws=1, wsp=W, wsb=need - 1) == S["FA_ERR_WORKSPACE"]
    assert check(fa, ws=1, wsp=W + 4, wsb=need) == S["FA_ERR_WORKSPACE"]
    assert check(fa, ws=1, wsp=A, wsb=need) == S["FA_ERR_WORKSPACE"]  # overlaps q


def test_fwd_rejects_before_any_hip_call(fa):
    """Argument errors return their code without touching the device (no GPU here)."""
    S = fa.STATUS
    lib = fa.lib
    assert lib.fa_fwd(None, None, None, None, None, 1, 1, 64, 96, 0.1, None) == S["FA_ERR_HEADDIM"]
    assert lib.fa_fwd(A, 2 * A, 3 * A, A, 5 * A, 1, 1, 64, 128, 0.1, None) == S["FA_ERR_ALIAS"]
    assert lib.fa_fwd(None, None, None, None, None, 1, 1, 0, 128, 0.1, None) == 0  # empty: no-op
    assert lib.fa_unfused_fwd(A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 1, 64, 128, 0.1, None, 0, None) == \
        S["FA_ERR_WORKSPACE"]


def test_python_binding_type_checks(fa):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):  # CPU tensors are refused: there is no CPU path
        fa.fa_fwd(q, q, q, q.clone(), lse)
    with pytest.raises(TypeError):
        fa.fa_fwd(q.float(), q, q, q.clone(), lse)


# ---------------------------------------------------------------------------
# Decode-shaped forward: plan and validation (no GPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,Nq,Nk,d", [(16, 32, 1, 8192, 128), (1, 32, 1, 131072, 128), (1, 1, 1, 1, 128),
                                         (2, 3, 4, 1000, 64), (1, 8, 16, 30001, 128), (64, 64, 2, 100, 64),
                                         (1, 1, 1, 1 << 30, 128)])
def test_decode_plan_covers_every_key(fa, B, H, Nq, Nk, d):
    splits, chunk, ws = fa.fa_decode_plan(B, H, Nq, Nk, d)
    assert splits >= 1 and chunk >= 1
    assert (splits - 1) * chunk < Nk <= splits * chunk  # every chunk holds at least one key
    assert chunk == Nk or chunk % 128 == 0
    assert ws == (B * H * splits * Nq * (d + 1) * 4 + 255) // 256 * 256
    assert B * H * splits <= 2 ** 31 - 1


def test_decode_plan_fills_the_chip(fa):
    # About one round of resident workgroups (256 CUs x 7 per CU for one query row;
    # the matrix-core kernel for 2-16 rows: 2 per CU at d = 128, 4 at d = 64) when
    # the keys allow it; no chunk below 256 keys unless the whole sequence is shorter.
    resident = {(1, 128): 7, (1, 64): 7, (2, 128): 2, (3, 128): 2, (4, 64): 4, (5, 128): 2, (8, 128): 2,
                (16, 128): 2, (8, 64): 4, (16, 64): 4}
    for B, H, Nk in ((16, 32, 8192), (1, 32, 131072), (1, 1, 1 << 20), (4, 16, 4096), (2, 8, 30001)):
        for (nq, d), per_cu in resident.items():
            splits, chunk, _ = fa.fa_decode_plan(B, H, nq, Nk, d)
            target = 256 * per_cu
            # splits per head: what the target asks for, at most one chunk of 256 keys
            # each, then chunks rounded up to 128 keys
            want = min(-(-target // (B * H)), -(-Nk // 256))
            chunk_want = min(Nk, -(-(-(-Nk // want)) // 128) * 128)
            assert chunk == chunk_want and splits == -(-Nk // chunk_want), (B, H, Nk, nq)
            assert chunk >= 256 or chunk == Nk


def test_decode_plan_errors(fa):
    with pytest.raises(ValueError):
        fa.fa_decode_plan(1, 1, 17, 100, 128)
    with pytest.raises(ValueError):
        fa.fa_decode_plan(1, 1, 1, 100, 96)
    with pytest.raises(ValueError):
        fa.fa_decode_plan(1, 1, 1, (1 << 30) + 1, 128)


def dcheck(fa, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=2, Nq=4, Nk=300, d=128, scale=0.1,
           wsp=16 * A, wsb=None):
    if wsb is None:
        wsb = fa.fa_decode_plan(B, H, Nq, Nk, d)[2] if 0 <= Nq <= 16 and Nk >= 0 and d in (64, 128) else 0
    return fa.fa_decode_check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, wsp, wsb)


def test_decode_check_args(fa):
    S = fa.STATUS
    assert dcheck(fa) == 0
    assert dcheck(fa, q=A, k=A, v=A) == 0
    assert dcheck(fa, Nq=0, q=None, k=None, v=None, o=None, lse=None, wsp=None) == 0  # empty
    assert dcheck(fa, B=0, wsp=None) == 0
    assert dcheck(fa, Nq=17) == S["FA_ERR_SHAPE"]
    assert dcheck(fa, Nk=0) == S["FA_ERR_SHAPE"]
    assert dcheck(fa, Nk=(1 << 30) + 1, wsb=1 << 40) == S["FA_ERR_SHAPE"]
    assert dcheck(fa, Nq=-1, wsb=0) == S["FA_ERR_SHAPE"]
    assert dcheck(fa, d=96) == S["FA_ERR_HEADDIM"]
    assert dcheck(fa, scale=float("nan")) == S["FA_ERR_SCALE"]
    assert dcheck(fa, v=None) == S["FA_ERR_NULL"]
    assert dcheck(fa, k=2 * A + 8) == S["FA_ERR_ALIGN"]
    assert dcheck(fa, lse=5 * A + 1) == S["FA_ERR_ALIGN"]
    assert dcheck(fa, o=2 * A + 4096) == S["FA_ERR_ALIAS"]  # inside k (2*300*128*2 bytes)
    assert dcheck(fa, lse=4 * A + 16) == S["FA_ERR_ALIAS"]  # inside o
    assert dcheck(fa, wsp=None) == S["FA_ERR_WORKSPACE"]
    need = fa.fa_decode_plan(1, 2, 4, 300, 128)[2]
    assert dcheck(fa, wsb=need - 1) == S["FA_ERR_WORKSPACE"]
    assert dcheck(fa, wsp=16 * A + 8) == S["FA_ERR_WORKSPACE"]
    assert dcheck(fa, wsp=3 * A) == S["FA_ERR_WORKSPACE"]  # overlaps v
    assert dcheck(fa, B=1 << 30, H=1 << 30, wsb=0) == S["FA_ERR_OVERFLOW"]


def test_decode_fwd_rejects_before_any_hip_call(fa):
    S = fa.STATUS
    lib = fa.lib
    assert lib.fa_decode_fwd(A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 1, 32, 100, 128, 0.1, 16 * A, 1 << 20,
                             None) == S["FA_ERR_SHAPE"]
    assert lib.fa_decode_fwd(None, None, None, None, None, 1, 1, 0, 100, 128, 0.1, None, 0, None) == 0


def test_decode_noalloc_rejects_before_any_hip_call(fa):
    """The allocation-free decode checks its arguments, then that the shape's partial
    results fit the fixed scratch array, before any HIP call (the pointers here are
    fake)."""
    S = fa.STATUS
    lib = fa.lib
    big = 1 << 36  # fake tensors far apart

    def call(B, H, Nq, Nk, d=128, q=A, scale=0.1):
        return lib.fa_decode_fwd_noalloc(q, 2 * big, 3 * big, 4 * big, 5 * big, B, H, Nq, Nk, d, scale, None)

    assert call(1, 1, 32, 100) == S["FA_ERR_SHAPE"]
    assert call(1, 1, 4, 100, d=96) == S["FA_ERR_HEADDIM"]
    assert call(1, 1, 4, 100, q=None) == S["FA_ERR_NULL"]
    assert call(1, 1, 4, 100, scale=float("inf")) == S["FA_ERR_SCALE"]
    assert call(0, 1, 4, 100, q=None) == 0  # empty problem: a no-op
    # one key chunk per head (the grid fills the chip with heads): the partials of
    # B*H*Nq rows take (d + 1) * 4 bytes each, which passes the fixed size here
    B, H, Nq, Nk, d = 64, 64, 16, 4096, 128
    splits, _, need = fa.fa_decode_plan(B, H, Nq, Nk, d)
    assert splits == 1 and need == (B * H * Nq * (d + 1) * 4 + 255) // 256 * 256 > fa.DECODE_SCRATCH_BYTES
    assert call(B, H, Nq, Nk, d) == S["FA_ERR_SCRATCH"]
    assert "FA_DECODE_SCRATCH_BYTES" in fa.fa_status_string(S["FA_ERR_SCRATCH"])
    with pytest.raises(ValueError):
        fa._raise(S["FA_ERR_SCRATCH"], "fa_decode_fwd_noalloc")


def test_tile_order_rejects_before_any_hip_call(fa):
    S = fa.STATUS
    lib = fa.lib
    for order in (-1, 3):
        assert lib.fa_fwd_tile_order(A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 1, 64, 128, 0.1, order, None) == \
            S["FA_ERR_SHAPE"]
    assert lib.fa_fwd_tile_order(A, 2 * A, 3 * A, A, 5 * A, 1, 1, 64, 128, 0.1, 1, None) == S["FA_ERR_ALIAS"]
    assert lib.fa_fwd_tile_order(None, None, None, None, None, 1, 1, 0, 128, 0.1, 2, None) == 0


def test_bwd_workspace_and_argument_errors(fa):
    S = fa.STATUS
    lib = fa.lib
    assert fa.fa_bwd_workspace_bytes(1, 2, 64) == 1024
    assert fa.fa_bwd_workspace_bytes(1, 1, 1) == 256
    assert fa.fa_bwd_workspace_bytes(-1, 1, 1) == 0
    P = [A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A]  # q k v o lse dO dq dk dv
    W = 16 * A

    def call(p=P, B=1, H=2, N=64, d=128, scale=0.1, ws=W, wsb=1024):
        return lib.fa_bwd(*p, B, H, N, d, scale, ws, wsb, None)

    def with_(i, x):
        p = list(P)
        p[i] = x
        return p

    assert call(d=96) == S["FA_ERR_HEADDIM"]
    assert call(N=-1) == S["FA_ERR_SHAPE"]
    assert call(p=with_(5, None)) == S["FA_ERR_NULL"]  # dO
    assert call(p=with_(8, None)) == S["FA_ERR_NULL"]  # dv
    assert call(p=with_(6, 7 * A + 8)) == S["FA_ERR_ALIGN"]  # dq
    assert call(p=with_(6, A)) == S["FA_ERR_ALIAS"]  # dq is q
    assert call(p=with_(7, 6 * A + 64)) == S["FA_ERR_ALIAS"]  # dk inside dO
    assert call(p=with_(8, 8 * A)) == S["FA_ERR_ALIAS"]  # dv is dk
    assert call(ws=None) == S["FA_ERR_WORKSPACE"]
    assert call(wsb=1023) == S["FA_ERR_WORKSPACE"]
    assert call(ws=9 * A) == S["FA_ERR_WORKSPACE"]  # overlaps dv
    assert call(p=[None] * 9, N=0, ws=None, wsb=0) == 0  # empty: no-op

