"""Chunk-form evaluation of the gated delta rule in fp64 -- TEST INFRASTRUCTURE ONLY.

This module follows the stage order that the page "PR #33465 完整报告"
(SGLang "[Kimi-K3][NPU] Support Kimi-K3 on NPU", section "关键源码片段",
the Ascend KDA extend path) names for prefill: L2-normalise q and k, split
each sequence into chunks of 64 tokens, take the in-chunk cumulative sum of
the gate scaled by log2(e), form the gated and beta-weighted K K^T and the
gated Q K^T, invert the unit lower-triangular system, recompute W and U, run
the inter-chunk state recurrence and form the chunk output.

The arithmetic is written from the recurrence itself (page
"【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对", sections
1.1 and 1.3: a chunk acts on the state as an affine map).  For one chunk of
L rows with gamma_i = log2(e) * sum_{s<=i} g_s (a K-vector per row):

    A_kk[i,j] = beta_i * sum_c k_ic k_jc 2^(gamma_ic - gamma_jc)      j <  i
    A_qk[i,j] = scale  * sum_c q_ic k_jc 2^(gamma_ic - gamma_jc)      j <= i
    T         = (I + A_kk)^-1
    W         = T diag(beta) (K * 2^gamma)        U = T diag(beta) V
    Kbar      = K * 2^(gamma_last - gamma)
    V_new     = U - W S_in
    O         = scale (Q * 2^gamma) S_in + A_qk V_new
    S_out     = diag(2^gamma_last) S_in + Kbar^T V_new

Every gate factor is evaluated directly as 2^(difference) in fp64, with no
factorisation.  The triangular inverse uses numpy's solver.  Nothing here is
blocked, fused or reordered beyond these formulas; it exists to pin that the
chunk decomposition equals the token recurrence (:func:`oracle.kda_recurrence`).
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
CHUNK = 64


def _l2n(x: np.ndarray, use_l2norm: bool, eps: float) -> np.ndarray:
    if not use_l2norm:
        return x
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def chunk_ranges(cu_seqlens, chunk: int = CHUNK):
    """(sequence, start, length) of every chunk, aligned to each sequence start."""
    out = []
    cu = [int(c) for c in cu_seqlens]
    for n in range(len(cu) - 1):
        for s in range(cu[n], cu[n + 1], chunk):
            out.append((n, s, min(chunk, cu[n + 1] - s)))
    return out


def kda_chunked(q, k, v, g, beta, cu_seqlens, initial=None, scale=None, use_l2norm=True, eps=1e-6,
                chunk: int = CHUNK):
    """Return (out [T,H,V], final [N,H,V,K]) computed chunk by chunk in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, H, K = q.shape
    V = v.shape[2]
    N = len(cu_seqlens) - 1
    if scale is None:
        scale = K ** -0.5
    qn = _l2n(q, use_l2norm, eps)
    kn = _l2n(k, use_l2norm, eps)
    out = np.zeros((T, H, V))
    # state per (n, h) as K x V matrices
    S = np.zeros((N, H, K, V))
    if initial is not None:
        S[:] = np.transpose(np.asarray(initial, np.float64), (0, 1, 3, 2))
    for (n, s, L) in chunk_ranges(cu_seqlens, chunk):
        for h in range(H):
            Q = qn[s:s + L, h]          # L x K
            Kc = kn[s:s + L, h]         # L x K
            Vc = v[s:s + L, h]          # L x V
            b = beta[s:s + L, h]        # L
            gam = np.cumsum(g[s:s + L, h], axis=0) * LOG2E   # L x K, inclusive
            diff = gam[:, None, :] - gam[None, :, :]          # [i, j, c]
            fac = np.exp2(np.where(np.tril(np.ones((L, L), bool))[:, :, None], diff, 0.0))
            A_kk = b[:, None] * np.einsum("ic,jc,ijc->ij", Kc, Kc, fac)
            A_kk = np.tril(A_kk, -1)
            A_qk = scale * np.einsum("ic,jc,ijc->ij", Q, Kc, fac)
            A_qk = np.tril(A_qk, 0)
            Tm = np.linalg.solve(np.eye(L) + A_kk, np.eye(L))
            W = Tm @ (b[:, None] * (Kc * np.exp2(gam)))
            U = Tm @ (b[:, None] * Vc)
            Kbar = Kc * np.exp2(gam[-1][None, :] - gam)
            Sin = S[n, h]
            Vnew = U - W @ Sin
            out[s:s + L, h] = scale * (Q * np.exp2(gam)) @ Sin + A_qk @ Vnew
            S[n, h] = np.exp2(gam[-1])[:, None] * Sin + Kbar.T @ Vnew
    final = np.transpose(S, (0, 1, 3, 2)).copy()
    return out, final
