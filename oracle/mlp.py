"""MLP shard of the Domino layer, forward and backward, in numpy float64 (oracle; tests only).

Notation follows the pages: the layer is X·A·B = Y, A column-parallel and B
row-parallel, each rank s of P holding A_s (columns S_s of A) and B_s (rows S_s
of B), its partial Y_s = act(X·A_s)·B_s, and the AllReduce summing the partials
([Domino] "TP 的数据依赖：通信为何难以隐藏"; [Primer] §3.1).
"""
from __future__ import annotations

import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715


def to_f64(t) -> np.ndarray:
    """Exact upcast of a CPU torch tensor (bf16 or fp32) or array to float64."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    import torch  # local: keeps the oracle importable for numpy-only use

    return t.detach().to(torch.float64).cpu().numpy()


# ----------------------------------------------------------------------------------------
# Activations. GeLU in its tanh form; SwiGLU = silu(gate) * up.
# ----------------------------------------------------------------------------------------
def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """0.5·x·(1 + tanh(√(2/π)·(x + 0.044715·x³)))."""
    return 0.5 * x * (1.0 + np.tanh(SQRT_2_OVER_PI * (x + GELU_CUBIC * x ** 3)))


def gelu_tanh_grad(x: np.ndarray) -> np.ndarray:
    """d/dx of gelu_tanh, by the product and chain rules on the expression above."""
    u = SQRT_2_OVER_PI * (x + GELU_CUBIC * x ** 3)
    t = np.tanh(u)
    du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * x ** 2)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def act_forward(Hpre: np.ndarray, act: str) -> np.ndarray:
    """H from the first GEMM's output. SwiGLU: Hpre = [gate | up], each f_s columns."""
    if act == "gelu_tanh":
        return gelu_tanh(Hpre)
    if act == "swiglu":
        f = Hpre.shape[1] // 2
        g, u = Hpre[:, :f], Hpre[:, f:]
        return silu(g) * u
    raise ValueError(act)


def act_backward(Hpre: np.ndarray, dH: np.ndarray, act: str) -> np.ndarray:
    """dHpre = (∂H/∂Hpre)ᵀ·dH, elementwise."""
    if act == "gelu_tanh":
        return dH * gelu_tanh_grad(Hpre)
    if act == "swiglu":
        f = Hpre.shape[1] // 2
        g, u = Hpre[:, :f], Hpre[:, f:]
        s = sigmoid(g)
        dg = dH * u * s * (1.0 + g * (1.0 - s))   # d silu(g)/dg = σ(g)(1 + g(1 − σ(g)))
        du = dH * g * s                            # = dH · silu(g)
        return np.concatenate([dg, du], axis=1)
    raise ValueError(act)


# ----------------------------------------------------------------------------------------
# Sharding: A column-parallel, B row-parallel ([Primer] §3.1, FFN = column then row).
# ----------------------------------------------------------------------------------------
def shard_slice(F: int, P: int, s: int) -> slice:
    """Rank s's contiguous block of the F FFN columns (equal blocks; F % P == 0)."""
    if F % P:
        raise ValueError("F must divide evenly into P shards")
    f = F // P
    return slice(s * f, (s + 1) * f)


def mlp_shard_weights(A: np.ndarray, B: np.ndarray, act: str, P: int, s: int):
    """A_s, B_s for rank s from the full weights A [h, n_a·F] and B [F, h]."""
    F = B.shape[0]
    S = shard_slice(F, P, s)
    if act == "swiglu":
        A_s = np.concatenate([A[:, :F][:, S], A[:, F:][:, S]], axis=1)
    else:
        A_s = A[:, S]
    return A_s, B[S, :]


def mlp_shard_forward(X: np.ndarray, A_s: np.ndarray, B_s: np.ndarray, act: str):
    """One rank's forward: Hpre = X·A_s, H = act(Hpre), Y_s = H·B_s (no reduce)."""
    Hpre = X @ A_s
    H = act_forward(Hpre, act)
    return Hpre, H, H @ B_s


def mlp_shard_backward(X, A_s, B_s, dY, act):
    """One rank's backward, given dY (identical on all ranks because Y was all-reduced).

    dgrad and wgrad of each linear layer are independent products
    ([Overlap] §1): dH = dY·B_sᵀ, dB_s = Hᵀ·dY; dHpre = act'(Hpre)⊙dH;
    dX_s = dHpre·A_sᵀ (this rank's partial, the tensor that is all-reduced),
    dA_s = Xᵀ·dHpre.
    """
    Hpre = X @ A_s
    H = act_forward(Hpre, act)
    dH = dY @ B_s.T
    dB_s = H.T @ dY
    dHpre = act_backward(Hpre, dH, act)
    dX_s = dHpre @ A_s.T
    dA_s = X.T @ dHpre
    return dHpre, dX_s, dA_s, dB_s


def shard_sum(partials) -> np.ndarray:
    """Σ_p partials[p] in the order p = 0..P−1: what the AllReduce of Y (or dX) produces."""
    out = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        out = out + np.asarray(p, dtype=np.float64)
    return out


def mlp_forward_unsharded(X, A, B, act):
    """The whole layer with full weights: act(X·A)·B (SwiGLU: silu(X·A_gate)⊙(X·A_up)·B)."""
    return act_forward(X @ A, act) @ B


def mlp_backward_unsharded(X, A, B, dY, act):
    """dX of the whole layer with full weights (what Σ_s dX_s must equal)."""
    Hpre = X @ A
    dHpre = act_backward(Hpre, dY @ B.T, act)
    return dHpre @ A.T


# ----------------------------------------------------------------------------------------
# Domino chunks: row split of X along batch, column split of B, and 2D
# ([Domino] "按行切分输入 X", "按列切分权重 B", "2D 切分（同时切 X 与 B）").
# ----------------------------------------------------------------------------------------
def _chunk_sizes(n: int, chunks: int):
    """torch.chunk sizes: ceil(n/chunks) each, the last one smaller, empty ones dropped."""
    if chunks < 1:
        raise ValueError("chunks must be >= 1")
    size = -(-n // chunks) if n else 0
    out, start = [], 0
    while start < n:
        stop = min(n, start + size)
        out.append((start, stop))
        start = stop
    return out


def row_chunk_ranges(batch: int, seq: int, chunks: int):
    """Token ranges of the row chunks: whole sequences, split along batch."""
    return [(b0 * seq, b1 * seq) for b0, b1 in _chunk_sizes(batch, chunks)]


def col_chunk_ranges(h: int, chunks: int):
    """Column ranges of the column chunks of B_s (its last dimension)."""
    return _chunk_sizes(h, chunks)


def domino_mlp_forward(X, A, B, act, P, batch, seq, row_chunks, col_chunks):
    """Y of the layer computed chunk by chunk, each chunk the sum of all P shard partials.

    Y[R_i, C_j] = Σ_s act(X[R_i]·A_s)·B_s[:, C_j]. Chunks are independent, so the
    result equals the unsplit layer; the chunk order is r0c0, r0c1, r1c0, r1c1.
    """
    T, h = X.shape
    Y = np.full((T, h), np.nan)
    for r0, r1 in row_chunk_ranges(batch, seq, row_chunks):
        for c0, c1 in col_chunk_ranges(h, col_chunks):
            parts = []
            for s in range(P):
                A_s, B_s = mlp_shard_weights(A, B, act, P, s)
                H = act_forward(X[r0:r1] @ A_s, act)
                parts.append(H @ B_s[:, c0:c1])
            Y[r0:r1, c0:c1] = shard_sum(parts)
    return Y


def domino_mlp_backward(X, A, B, dY, act, P, s, batch, seq, row_chunks, col_chunks):
    """Rank s's backward computed by Domino chunks, plus the reduced dX.

    dX is split like the forward's output where only one axis is split (row chunks
    of tokens, or column chunks of h, the mirror of the column split); the 2D split
    reduces dX by row chunks. Each dX chunk is Σ_p dX_p[chunk]. Weight gradients of
    rank s accumulate over row chunks (each contributes the K-slice of its tokens).
    Returns dX (reduced), dA_s, dB_s.
    """
    T, h = X.shape
    rows = row_chunk_ranges(batch, seq, row_chunks)
    cols = col_chunk_ranges(h, col_chunks if row_chunks == 1 else 1)
    dX = np.full((T, h), np.nan)
    for r0, r1 in rows:
        for c0, c1 in cols:
            parts = []
            for p in range(P):
                A_p, B_p = mlp_shard_weights(A, B, act, P, p)
                Hpre = X[r0:r1] @ A_p
                dHpre = act_backward(Hpre, dY[r0:r1] @ B_p.T, act)
                parts.append(dHpre @ A_p[c0:c1, :].T)
            dX[r0:r1, c0:c1] = shard_sum(parts)
    A_s, B_s = mlp_shard_weights(A, B, act, P, s)
    dA_s = np.zeros(A_s.shape)
    dB_s = np.zeros(B_s.shape)
    for r0, r1 in rows:
        Hpre = X[r0:r1] @ A_s
        H = act_forward(Hpre, act)
        dHpre = act_backward(Hpre, dY[r0:r1] @ B_s.T, act)
        dA_s = dA_s + X[r0:r1].T @ dHpre
        dB_s = dB_s + H.T @ dY[r0:r1]
    return dX, dA_s, dB_s


# ----------------------------------------------------------------------------------------
# Sampled evaluation for full-size workloads: rows of Y and dX depend only on the
# same rows of X and dY, and a column of dA_s (a row of dB_s) only on the matching
# FFN column(s) over all tokens, so a sample is computed exactly.
# ----------------------------------------------------------------------------------------
def mlp_y_rows(X_rows, A, B, act):
    """Rows of the reduced Y = Σ_s Y_s for the given rows of X (the unsharded layer)."""
    return mlp_forward_unsharded(X_rows, A, B, act)


def mlp_dx_rows(X_rows, dY_rows, A, B, act):
    """Rows of the reduced dX = Σ_s dX_s."""
    return mlp_backward_unsharded(X_rows, A, B, dY_rows, act)


def mlp_wgrad_slices(X, dY, A_s, B_s, act, ffn_cols):
    """Exact dA_s[:, cols] and dB_s[cols, :] for FFN columns `ffn_cols` of rank s.

    For SwiGLU the FFN column j has a gate column j and an up column f_s + j in A_s;
    both are returned (dA columns ordered [gate cols | up cols]).
    """
    ffn_cols = np.asarray(ffn_cols)
    f = B_s.shape[0]
    if act == "swiglu":
        a_cols = np.concatenate([ffn_cols, f + ffn_cols])
    else:
        a_cols = ffn_cols
    Hpre_c = X @ A_s[:, a_cols]                      # [T, n_a·k]
    dH_c = dY @ B_s[ffn_cols, :].T                   # [T, k]
    H_c = act_forward(Hpre_c, act)
    dHpre_c = act_backward(Hpre_c, dH_c, act)
    return X.T @ dHpre_c, H_c.T @ dY
