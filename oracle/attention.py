"""Attention shard of the Domino layer (forward), numpy float64 (oracle; tests only).

For attention the layer X·A·B = Y has A = multi-head self-attention on the rank's
head slice and B = the output projection ([Domino] "TP 的数据依赖：通信为何难以隐藏");
the attention is causal self-attention only ([Domino] "如何尝试 DeepSpeed-Domino").
Reading: scale 1/√d, mask k > i within each sequence, no bias / dropout / rotary
embedding. Layout: X is [batch·seq, h], token = b·seq + i; QKV columns are
[Q | K | V], each H·d wide, head j at columns j·d .. j·d+d−1 within each block.
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
