"""fp64 CPU oracle of the attention backward: the gradients of
O = softmax(scale * Q K^T) V with respect to Q, K and V for an upstream dO.

Test infrastructure only, like the rest of this package: nothing on the GPU path
imports it, and it shares no code with the HIP kernels.

Sources. The pages describe the backward only by what it keeps: the standard
method stores the probability matrix P for the backward pass ("Flash Attention
(FA1)", section "Naive Attention 问题分析"), while FlashAttention stores only O and
the per-row LSE and recomputes P from them in the backward ("01 · 注意力为什么是 IO
瓶颈", section 6). They give no formulas, so the oracle is the plain definition, the
chain rule through the three forward steps, with LSE treated as saved state (no
gradient flows into it):
    S = scale * Q K^T,  P = softmax_rows(S),  O = P V
    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)        (softmax Jacobian per row)
    dQ = scale * dS K,   dK = scale * dS^T Q
The row term sum_k P_ik dP_ik equals dO_i . O_i, because O_i = sum_k P_ik V_k.
Conventions as in attention.py: q [B,H,N,d], k, v [B,H,Nk,d], dO [B,H,N,d], all
float64 numpy arrays (bf16 inputs widened exactly).
"""
from __future__ import annotations

import numpy as np
import torch


def attention_backward_fp64(q, k, v, dO, scale):
    """Returns (dQ, dK, dV) as float64 arrays shaped like q, k, v."""
    B, H, N, d = q.shape
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty(k.shape[:3] + (v.shape[-1],))
    for b in range(B):
        for h in range(H):
            Q, K, V, G = q[b, h], k[b, h], v[b, h], dO[b, h]
            S = scale * (Q @ K.T)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            dV[b, h] = P.T @ G
            dP = G @ V.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[b, h] = scale * (dS @ K)
            dK[b, h] = scale * (dS.T @ Q)
    return dQ, dK, dV


def attention_backward_unfused_bf16(q, k, v, o, dO, scale):
    """The standard backward as a bf16 framework runs it, on the CPU: the error
    yardstick for a GPU backward. Inputs are torch bfloat16 CPU tensors (o is the
    forward's bf16 output). Each product takes bf16 operands and accumulates in
    fp32; P and dS are stored as bf16 between steps (the standard method keeps P
    for the backward); dV, dQ, dK are rounded to bf16.
        S = fp32(Q K^T) * scale;  P = bf16(softmax_rows(S) in fp32)
        dV = bf16(P^T dO);  dP = fp32(dO V^T);  D = rowsum(fp32(dO) * fp32(O))
        dS = bf16(P * (dP - D));  dQ = bf16(scale * dS K);  dK = bf16(scale * dS^T Q)
    Returns (dQ, dK, dV) as float64 numpy arrays."""
    B, H, N, d = q.shape
    out = [np.empty(tuple(t.shape)) for t in (q, k, v)]
    sc = torch.tensor(scale, dtype=torch.float32)
    for b in range(B):
        for h in range(H):
            Q, K, V, O, G = (t[b, h].float() for t in (q, k, v, o, dO))
            S = (Q @ K.T) * sc
            E = torch.exp(S - S.max(dim=1, keepdim=True).values)
            P = (E / E.sum(dim=1, keepdim=True)).to(torch.bfloat16).float()
            dV = (P.T @ G).to(torch.bfloat16)
            dP = G @ V.T
            D = (G * O).sum(dim=1, keepdim=True)
            dS = (P * (dP - D)).to(torch.bfloat16).float()
            dQ = ((dS @ K) * sc).to(torch.bfloat16)
            dK = ((dS.T @ Q) * sc).to(torch.bfloat16)
            for arr, t in zip(out, (dQ, dK, dV)):
                arr[b, h] = t.double().numpy()
    return tuple(out)
