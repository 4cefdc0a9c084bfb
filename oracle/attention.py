"""Attention shard of the Domino layer (forward and backward), numpy float64 (oracle;
tests only).

For attention the layer X·A·B = Y has A = multi-head self-attention on the rank's
head slice and B = the output projection ([Domino] "TP 的数据依赖：通信为何难以隐藏");
the attention is causal self-attention only ([Domino] "如何尝试 DeepSpeed-Domino").
Reading: scale 1/√d, mask k > i within each sequence, no bias / dropout / rotary
embedding. Layout: X is [batch·seq, h], token = b·seq + i; QKV columns are
[Q | K | V], each H·d wide, head j at columns j·d .. j·d+d−1 within each block.

Backward: the out-projection and the QKV product are linear layers whose input
gradient and weight gradient are independent products, the input gradient of the
first one being the partial that is all-reduced ([Overlap] §1); the attention's own
backward follows from the softmax and product rules (written out below).
"""
from __future__ import annotations

import math

import numpy as np

from .mlp import row_chunk_ranges, shard_sum


def attn_shard_weights(Aqkv, Bo, heads_full, head_dim, P, s):
    """Rank s's QKV columns (its head block of each of Q, K, V) and Bo rows."""
    if heads_full % P:
        raise ValueError("heads must divide evenly into P shards")
    hs = heads_full // P
    Hd = heads_full * head_dim
    c0, c1 = s * hs * head_dim, (s + 1) * hs * head_dim
    A_s = np.concatenate([Aqkv[:, blk * Hd + c0: blk * Hd + c1] for blk in range(3)], axis=1)
    return A_s, Bo[c0:c1, :]


def causal_attention(Q, K, V, scale):
    """softmax(Q·Kᵀ·scale with k > i masked)·V for one sequence and one head.

    Q, K, V: [n, d]. The softmax subtracts each row's maximum before exponentiating.
    """
    n = Q.shape[0]
    S = (Q @ K.T) * scale
    mask = np.triu(np.ones((n, n), dtype=bool), k=1)
    S = np.where(mask, -np.inf, S)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    Pm = E / E.sum(axis=1, keepdims=True)
    return Pm @ V


def _mha(QKV, batch, seq, heads, head_dim, scale):
    """O [T, heads·d] from QKV [T, 3·heads·d], head-concatenated."""
    Hd = heads * head_dim
    O = np.zeros((batch * seq, Hd))
    for b in range(batch):
        r = slice(b * seq, (b + 1) * seq)
        for j in range(heads):
            c = slice(j * head_dim, (j + 1) * head_dim)
            Q = QKV[r, 0 * Hd:1 * Hd][:, c]
            K = QKV[r, 1 * Hd:2 * Hd][:, c]
            V = QKV[r, 2 * Hd:3 * Hd][:, c]
            O[r, c] = causal_attention(Q, K, V, scale)
    return O


def attn_shard_forward(X, A_s, Bo_s, batch, seq, heads_shard, head_dim, scale=None):
    """One rank's forward: QKV = X·Aqkv_s, O = MHA(QKV) on its heads, Y_s = O·Bo_s."""
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    QKV = X @ A_s
    O = _mha(QKV, batch, seq, heads_shard, head_dim, scale)
    return QKV, O, O @ Bo_s


def attn_forward_unsharded(X, Aqkv, Bo, batch, seq, heads_full, head_dim, scale=None):
    """Full multi-head attention with all heads and the full output projection."""
    return attn_shard_forward(X, Aqkv, Bo, batch, seq, heads_full, head_dim, scale)[2]


def domino_attn_forward(X, Aqkv, Bo, batch, seq, heads_full, head_dim, P, row_chunks, scale=None):
    """Y by row chunks (whole sequences), each chunk the sum of the P head-slice partials."""
    T, h = X.shape
    Y = np.full((T, h), np.nan)
    hs = heads_full // P
    for r0, r1 in row_chunk_ranges(batch, seq, row_chunks):
        nb = (r1 - r0) // seq
        parts = []
        for s in range(P):
            A_s, Bo_s = attn_shard_weights(Aqkv, Bo, heads_full, head_dim, P, s)
            parts.append(attn_shard_forward(X[r0:r1], A_s, Bo_s, nb, seq, hs, head_dim, scale)[2])
        Y[r0:r1] = shard_sum(parts)
    return Y


def attn_y_rows(X_seq, Aqkv, Bo, heads_full, head_dim, rows, scale=None):
    """Rows `rows` (positions within one sequence) of the reduced Y, given that
    sequence's X [seq, h]. Only the prefix up to max(rows) is needed for K and V."""
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    rows = np.asarray(rows)
    n = int(rows.max()) + 1
    Hd = heads_full * head_dim
    Xp = X_seq[:n]
    K = Xp @ Aqkv[:, Hd:2 * Hd]
    V = Xp @ Aqkv[:, 2 * Hd:3 * Hd]
    Q = X_seq[rows] @ Aqkv[:, :Hd]
    O = np.zeros((len(rows), Hd))
    for j in range(heads_full):
        c = slice(j * head_dim, (j + 1) * head_dim)
        for t, i in enumerate(rows):
            s = (K[: i + 1, c] @ Q[t, c]) * scale
            s = s - s.max()
            e = np.exp(s)
            O[t, c] = (e / e.sum()) @ V[: i + 1, c]
    return O @ Bo


def causal_attention_lse(Q, K, scale):
    """Per row i, the natural log of Σ_{k ≤ i} exp(scale·q_i·k_k): what the forward keeps
    so the backward can rebuild the probabilities without renormalising."""
    n = Q.shape[0]
    S = (Q @ K.T) * scale
    S = np.where(np.triu(np.ones((n, n), dtype=bool), k=1), -np.inf, S)
    m = S.max(axis=1)
    return m + np.log(np.exp(S - m[:, None]).sum(axis=1))


def causal_attention_backward(Q, K, V, dO, scale):
    """dQ, dK, dV of O = P·V with P = softmax(Q·Kᵀ·scale, k > i masked), given dO.

    Product rule on O = P·V: dV = Pᵀ·dO and dP = dO·Vᵀ. Softmax rule, row by row:
    dS_ik = P_ik·(dP_ik − Σ_k' P_ik'·dP_ik') (masked entries have P = 0, so dS = 0).
    Product rule on S = scale·Q·Kᵀ: dQ = scale·dS·K, dK = scale·dSᵀ·Q.
    """
    n = Q.shape[0]
    S = (Q @ K.T) * scale
    S = np.where(np.triu(np.ones((n, n), dtype=bool), k=1), -np.inf, S)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    Pm = E / E.sum(axis=1, keepdims=True)
    dV = Pm.T @ dO
    dP = dO @ V.T
    dS = Pm * (dP - np.sum(Pm * dP, axis=1, keepdims=True))
    return scale * (dS @ K), scale * (dS.T @ Q), dV


def _mha_backward(QKV, dO, batch, seq, heads, head_dim, scale):
    """dQKV [T, 3·heads·d] from QKV and dO [T, heads·d], head by head per sequence."""
    Hd = heads * head_dim
    dQKV = np.zeros((batch * seq, 3 * Hd))
    for b in range(batch):
        r = slice(b * seq, (b + 1) * seq)
        for j in range(heads):
            c = slice(j * head_dim, (j + 1) * head_dim)
            Q = QKV[r, 0 * Hd:1 * Hd][:, c]
            K = QKV[r, 1 * Hd:2 * Hd][:, c]
            V = QKV[r, 2 * Hd:3 * Hd][:, c]
            dQ, dK, dV = causal_attention_backward(Q, K, V, dO[r, c], scale)
            dQKV[r, 0 * Hd:1 * Hd][:, c] = dQ
            dQKV[r, 1 * Hd:2 * Hd][:, c] = dK
            dQKV[r, 2 * Hd:3 * Hd][:, c] = dV
    return dQKV


def attn_lse(QKV, batch, seq, heads, head_dim, scale=None):
    """LSE [T, heads]: causal_attention_lse of every (sequence, head)."""
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    Hd = heads * head_dim
    L = np.zeros((batch * seq, heads))
    for b in range(batch):
        r = slice(b * seq, (b + 1) * seq)
        for j in range(heads):
            c = slice(j * head_dim, (j + 1) * head_dim)
            L[r, j] = causal_attention_lse(QKV[r, 0 * Hd:1 * Hd][:, c], QKV[r, 1 * Hd:2 * Hd][:, c], scale)
    return L


def attn_shard_backward(X, A_s, Bo_s, dY, batch, seq, heads_shard, head_dim, scale=None):
    """One rank's backward, given dY (identical on all ranks because Y was all-reduced).

    Out-projection: dO = dY·Bo_sᵀ, dBo_s = Oᵀ·dY. Attention: dQKV from dO. QKV product:
    dX_s = dQKV·A_sᵀ (this rank's partial, the tensor that is all-reduced),
    dA_s = Xᵀ·dQKV. Returns dO, dQKV, dX_s, dA_s, dBo_s.
    """
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    QKV, O, _ = attn_shard_forward(X, A_s, Bo_s, batch, seq, heads_shard, head_dim, scale)
    dO = dY @ Bo_s.T
    dBo_s = O.T @ dY
    dQKV = _mha_backward(QKV, dO, batch, seq, heads_shard, head_dim, scale)
    return dO, dQKV, dQKV @ A_s.T, X.T @ dQKV, dBo_s


def attn_backward_unsharded(X, Aqkv, Bo, dY, batch, seq, heads_full, head_dim, scale=None):
    """dX of the whole attention layer with all heads (what Σ_s dX_s must equal)."""
    return attn_shard_backward(X, Aqkv, Bo, dY, batch, seq, heads_full, head_dim, scale)[2]


def domino_attn_backward(X, Aqkv, Bo, dY, batch, seq, heads_full, head_dim, P, s, row_chunks, scale=None):
    """Rank s's backward by Domino row chunks (whole sequences), plus the reduced dX.

    Each dX chunk is Σ_p dX_p[chunk]; rank s's weight gradients accumulate over the row
    chunks (each contributes the K-slice of its tokens). Returns dX, dA_s, dBo_s.
    """
    T, h = X.shape
    hs = heads_full // P
    dX = np.full((T, h), np.nan)
    A_s, Bo_s = attn_shard_weights(Aqkv, Bo, heads_full, head_dim, P, s)
    dA_s = np.zeros(A_s.shape)
    dBo_s = np.zeros(Bo_s.shape)
    for r0, r1 in row_chunk_ranges(batch, seq, row_chunks):
        nb = (r1 - r0) // seq
        parts = []
        for p in range(P):
            A_p, Bo_p = attn_shard_weights(Aqkv, Bo, heads_full, head_dim, P, p)
            parts.append(attn_shard_backward(X[r0:r1], A_p, Bo_p, dY[r0:r1], nb, seq, hs, head_dim, scale)[2])
        dX[r0:r1] = shard_sum(parts)
        _, _, _, dA_c, dBo_c = attn_shard_backward(X[r0:r1], A_s, Bo_s, dY[r0:r1], nb, seq, hs, head_dim, scale)
        dA_s = dA_s + dA_c
        dBo_s = dBo_s + dBo_c
    return dX, dA_s, dBo_s
