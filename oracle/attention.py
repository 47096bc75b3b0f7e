"""fp64 CPU oracle of the attention forward, O = softmax(scale * Q K^T) V plus a
per-row log-sum-exp.

Test infrastructure only (see the package docstring): nothing on the GPU path
imports this module.

Conventions shared by every function here:
  * q is a float64 numpy array of shape [B, H, N, d] and k, v of shape
    [B, H, Nk, d] (the bf16 inputs widened exactly). Nk = N for the square
    forward; decode-shaped problems have a few query rows against many keys
    (N << Nk), and every definition below reads the same for them. ``scale``
    multiplies the scores before the softmax (the pages write softmax(QK^T); the
    1/sqrt(d) factor is the caller's choice).
  * LSE is the natural-log log-sum-exp of the scaled scores of a row,
    LSE_i = ln sum_j exp(s_ij) = m_i + ln l_i. The pages name this per-row fp32
    output of the forward ("写 O + LSE", ai-reference-codex page, section 4 and
    section 6) but do not define it; the natural log is the reading taken here,
    and Q = 0 then gives LSE = ln N.
  * ``rows`` (optional) is a 1-D array of flat row indices (b*H + h)*N + i; the
    functions then return O[len(rows), d] and LSE[len(rows)] for those rows only.
    Rows are independent of each other (FA1 page, "Online Softmax in
    FlashAttention": each query row is its own softmax).
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _row_groups(B: int, H: int, N: int, rows):
    """Yield (b, h, query indices, output positions) for the requested rows."""
    if rows is None:
        for b in range(B):
            for h in range(H):
                qi = np.arange(N, dtype=np.int64)
                yield b, h, qi, (b * H + h) * N + qi
        return
    rows = np.asarray(rows, dtype=np.int64)
    bh = rows // N
    for key in np.unique(bh):
        sel = np.nonzero(bh == key)[0]
        yield int(key // H), int(key % H), rows[sel] - key * N, sel


def _alloc(B, H, N, d, rows):
    if rows is None:
        return np.empty((B, H, N, d)), np.empty((B, H, N))
    n = len(rows)
    return np.empty((n, d)), np.empty((n,))


def _store(O, LSE, rows, pos, o_blk, lse_blk, B, H, N):
    if rows is None:
        Of = O.reshape(B * H * N, -1)
        Lf = LSE.reshape(B * H * N)
        Of[pos] = o_blk
        Lf[pos] = lse_blk
    else:
        O[pos] = o_blk
        LSE[pos] = lse_blk


def attention_fp64(q, k, v, scale, rows=None, block_rows: int = 512):
    """Two-pass safe-softmax attention, the textbook definition.

    Follows the FA1 page's safe softmax (section "Naive Attention 问题分析") applied
    to each row of S = scale * Q K^T, and the three steps of the ai-reference-codex
    page (section 3 table, section 5 ``naive_attention``):
        s_j = scale * <q_i, k_j>;  m = max_j s_j;  p_j = exp(s_j - m);  l = sum_j p_j
        O_i = sum_j p_j v_j / l;   LSE_i = m + ln l.
    Rows are processed in blocks of ``block_rows`` only to bound memory; the
    arithmetic of a row does not depend on the blocking.
    """
    B, H, N, d = q.shape
    O, LSE = _alloc(B, H, N, d, rows)
    for b, h, qi, pos in _row_groups(B, H, N, rows):
        K = k[b, h]
        V = v[b, h]
        for s0 in range(0, len(qi), block_rows):
            sl = slice(s0, s0 + block_rows)
            S = scale * (q[b, h][qi[sl]] @ K.T)  # step 1: scores
            m = S.max(axis=1)  # safe softmax: row max
            P = np.exp(S - m[:, None])  # step 2: numerators
            l = P.sum(axis=1)  # denominators
            o_blk = (P @ V) / l[:, None]  # step 3: O = P V, normalised
            lse_blk = m + np.log(l)
            _store(O, LSE, rows, pos[sl], o_blk, lse_blk, B, H, N)
    return O, LSE


def attention_online_fp64(q, k, v, scale, bc: int, br: int | None = None,
                          deferred: bool = False, rows=None):
    """Tiled online-softmax attention, the FA1 page's per-tile update (steps 1-5).

    K and V are cut along the sequence into tiles of ``bc`` rows (T_c = ceil(Nk/bc)
    over the Nk key rows, the last tile ragged); query rows into blocks of ``br`` (default: all of a
    head's requested rows at once). For each query block the running state
    (m_i, l_i, O_i) starts at (-inf, 0, 0) and each tile j applies:
      1. m~ = rowmax(S_ij),  P~ = exp(S_ij - m~),  l~ = rowsum(P~)
      2. m_new = max(m_i, m~),  l_new = l_i e^{m_i - m_new} + l~ e^{m~ - m_new}
      3. O~ = P~ V_j
      4-5. O_new = diag(l_new)^-1 ( diag(l_i e^{m_i - m_new}) O_i + e^{m~ - m_new} O~ )
    With ``deferred=False`` O_i is kept normalised after every tile, exactly as
    the page writes it. With ``deferred=True`` the state holds the unnormalised
    numerator N_i = diag(l_i) O_i (the page's own definition of N_i), updated as
    N_new = e^{m_i - m_new} N_i + e^{m~ - m_new} O~, and is divided by l once
    after the last tile. LSE = m + ln l after the last tile.
    """
    B, H, N, d = q.shape
    O, LSE = _alloc(B, H, N, d, rows)
    for b, h, qi, pos in _row_groups(B, H, N, rows):
        Q = q[b, h][qi]
        K = k[b, h]
        V = v[b, h]
        step = len(qi) if br is None else br
        for r0 in range(0, len(qi), step):
            Qi = Q[r0:r0 + step]
            nr = Qi.shape[0]
            m_i = np.full(nr, -np.inf)
            l_i = np.zeros(nr)
            acc = np.zeros((nr, d))  # O_i (normalised) or N_i (deferred)
            for c0 in range(0, K.shape[0], bc):
                Kj = K[c0:c0 + bc]
                Vj = V[c0:c0 + bc]
                S = scale * (Qi @ Kj.T)
                m_t = S.max(axis=1)  # step 1
                P_t = np.exp(S - m_t[:, None])
                l_t = P_t.sum(axis=1)
                m_new = np.maximum(m_i, m_t)  # step 2
                a_old = np.exp(m_i - m_new)  # e^{m_i - m_new}; 0 on the first tile
                a_new = np.exp(m_t - m_new)  # e^{m~ - m_new}
                l_new = l_i * a_old + l_t * a_new
                O_t = P_t @ Vj  # step 3
                if deferred:
                    acc = a_old[:, None] * acc + a_new[:, None] * O_t
                else:  # steps 4-5, O kept normalised
                    acc = ((l_i * a_old)[:, None] * acc + a_new[:, None] * O_t) / l_new[:, None]
                m_i, l_i = m_new, l_new
            o_blk = acc / l_i[:, None] if deferred else acc
            _store(O, LSE, rows, pos[r0:r0 + step], o_blk, m_i + np.log(l_i), B, H, N)
    return O, LSE


def attention_split_fp64(q, k, v, scale, chunk: int, rows=None):
    """Attention with the key range cut into chunks whose results are computed
    separately and merged afterwards: the split over keys of decode-shaped work.

    Chunk s holds keys [s*chunk, (s+1)*chunk) (the last one ragged). Its partial
    result is the two-pass definition restricted to those keys: O_s (normalised
    over the chunk) and LSE_s = m_s + ln l_s. The partials are then merged with
    the FA1 page's update (derivation steps 2 and 4-5) applied to whole chunks
    instead of tiles. With l_s e^{m_s - m} = e^{LSE_s - m} for any reference m,
    the update over all chunks reads
        m = max_s LSE_s,  L = m + ln sum_s e^{LSE_s - m},  O = sum_s e^{LSE_s - L} O_s,
    and L is the LSE of the whole row.
    """
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    Nk = k.shape[2]
    parts = [attention_fp64(q, k[:, :, c0:c0 + chunk], v[:, :, c0:c0 + chunk], scale, rows=rows)
             for c0 in range(0, Nk, chunk)]
    lse_s = np.stack([p[1] for p in parts])  # [S, ...rows]
    m = lse_s.max(axis=0)
    lse = m + np.log(np.exp(lse_s - m).sum(axis=0))
    w = np.exp(lse_s - lse)
    O = sum(w[s][..., None] * parts[s][0] for s in range(len(parts)))
    return O, lse


def attention_brute_force(q, k, v, scale):
    """Pure-Python triple loop with ``math.exp`` and ``math.fsum``; for tiny inputs.

    Computes the definition with no shift by the max (fine for the small scores it
    is used on) and an exactly rounded sum, so it shares neither the safe-softmax
    shift nor numpy's summation with :func:`attention_fp64`.
    q: [M][d] query rows; k, v: [N][d] key and value rows, for one head.
    Returns (O, LSE) as lists of M rows.
    """
    n_keys = len(k)
    d = len(q[0])
    dv = len(v[0])
    O, LSE = [], []
    for i in range(len(q)):
        e = [math.exp(scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d)))
             for j in range(n_keys)]
        den = math.fsum(e)
        O.append([math.fsum(e[j] * float(v[j][c]) for j in range(n_keys)) / den for c in range(dv)])
        LSE.append(math.log(den))
    return O, LSE


def attention_unfused_bf16(q, k, v, scale, rows=None):
    """The standard three-step computation at bf16 inputs and fp32 accumulation,
    with a 16-bit P, on the CPU: the error yardstick for the fused kernel.

    The ai-reference-codex page, section 3 and section 5: S = Q K^T, P = softmax(S),
    O = P V as three separate steps, each result stored between steps; section 6
    of the same page: P is converted to a 16-bit type before the PV product. Here:
        S = fp32 matmul of the bf16 values;  S *= scale (fp32)
        P = fp32 safe softmax of each row, then rounded to bf16 (nearest-even)
        O = fp32 matmul of bf16 P with bf16 V, then rounded to bf16.
    q, k, v: torch bfloat16 CPU tensors [B, H, N, d]. Returns (O, LSE) as float64
    numpy arrays (O holds bf16 values; LSE = m + ln l in fp32).
    """
    B, H, N, d = q.shape
    O, LSE = _alloc(B, H, N, d, rows)
    for b, h, qi, pos in _row_groups(B, H, N, rows):
        Kf = k[b, h].float()
        Vf = v[b, h].float()
        qi_t = torch.from_numpy(qi)
        for s0 in range(0, len(qi), 512):
            Qf = q[b, h][qi_t[s0:s0 + 512]].float()
            S = (Qf @ Kf.T) * torch.tensor(scale, dtype=torch.float32)
            m = S.max(dim=1).values
            E = torch.exp(S - m[:, None])
            l = E.sum(dim=1)
            P = (E / l[:, None]).to(torch.bfloat16)
            o_blk = (P.float() @ Vf).to(torch.bfloat16)
            lse_blk = m + torch.log(l)
            _store(O, LSE, rows, pos[s0:s0 + 512], o_blk.double().numpy(),
                   lse_blk.double().numpy(), B, H, N)
    return O, LSE
