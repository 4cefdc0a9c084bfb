"""A tensor-parallel group simulated on one GPU.

Every rank's shard lives in the same HBM: rank r holds A's FFN columns
[r·f_s, (r+1)·f_s) (for SwiGLU, those columns of both the gate and the up block) and
the matching rows of B (primer "从单卡到集群…" §3.1: column-parallel first layer,
row-parallel second layer); for attention rank r holds heads [r·H_s, (r+1)·H_s) of each
of Q, K, V and the matching rows of the output projection. Peer ranks' partials are
computed with the same library calls (no reduction), then the measured rank's call sums
them with its own partial — the reduction an AllReduce would do.

Only data placement happens here (slicing, device copies, buffer allocation); all
arithmetic runs in the HIP library.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import _lib as L


def _tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _ldtype(dtype: str) -> int:
    return L.DOMINO_BF16 if dtype == "bf16" else L.DOMINO_F32


def mlp_shard_weights(A: torch.Tensor, B: torch.Tensor, act: str, P: int, r: int):
    F = B.shape[0]
    f = F // P
    cols = slice(r * f, (r + 1) * f)
    if act == "swiglu":
        A_s = torch.cat([A[:, :F][:, cols], A[:, F:][:, cols]], dim=1)
    else:
        A_s = A[:, cols]
    return A_s.contiguous(), B[cols, :].contiguous()


def attn_shard_weights(Aqkv: torch.Tensor, Bo: torch.Tensor, heads_full: int, head_dim: int, P: int, r: int):
    hs = heads_full // P
    Hd = heads_full * head_dim
    c0, c1 = r * hs * head_dim, (r + 1) * hs * head_dim
    A_s = torch.cat([Aqkv[:, k * Hd + c0:k * Hd + c1] for k in range(3)], dim=1)
    return A_s.contiguous(), Bo[c0:c1, :].contiguous()


class MlpGroup:
    """P ranks of an MLP layer on one device; rank 0 is the measured rank."""

    def __init__(self, *, batch, seq, hidden, ffn_shard, act, dtype, row_chunks, col_chunks, n_partials,
                 X, A, B, dY=None, device="cuda", ranks: Optional[List[int]] = None):
        self.batch, self.seq, self.hidden, self.f = batch, seq, hidden, ffn_shard
        self.act, self.dtype, self.P = act, dtype, n_partials
        self.row_chunks, self.col_chunks = row_chunks, col_chunks
        self.T = batch * seq
        self.n1 = 2 * ffn_shard if act == "swiglu" else ffn_shard
        td = _tdtype(dtype)
        self.device = device
        self.X = X.to(device=device, dtype=td).contiguous()
        self.dY = None if dY is None else dY.to(device=device, dtype=td).contiguous()
        self.ranks = list(range(n_partials)) if ranks is None else ranks
        self.A_s, self.B_s = {}, {}
        for r in self.ranks:
            a, b = mlp_shard_weights(A, B, act, n_partials, r)
            self.A_s[r] = a.to(device=device, dtype=td)
            self.B_s[r] = b.to(device=device, dtype=td)
        T, h, n1, f = self.T, hidden, self.n1, ffn_shard
        e = dict(device=device, dtype=td)
        self.Hpre = {r: torch.empty(T, n1, **e) for r in self.ranks}
        self.H = {r: torch.empty(T, f, **e) for r in self.ranks}
        self.Y_own = {r: torch.empty(T, h, **e) for r in self.ranks}
        self.Y = torch.empty(T, h, **e)
        if self.dY is not None:
            self.dHpre = {r: torch.empty(T, n1, **e) for r in self.ranks}
            self.dX_own = {r: torch.empty(T, h, **e) for r in self.ranks}
            self.dX = torch.empty(T, h, **e)
            self.dA = torch.zeros(h, n1, device=device, dtype=torch.float32)
            self.dB = torch.zeros(f, h, device=device, dtype=torch.float32)
        # One workspace for every call this group makes: the split as configured and the
        # unsplit (peer and comparison) calls.
        descs = [self.desc(), self.desc(rank_alone=True, row_chunks=1, col_chunks=1)]
        nbytes = max(max(L.domino_block_fwd_workspace_size(d), L.domino_block_bwd_workspace_size(d)) for d in descs)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        self.ws_bytes = nbytes

    def desc(self, *, rank_alone=False, row_chunks=None, col_chunks=None, no_join=0) -> L.MlpDesc:
        return L.MlpDesc(batch=self.batch, seq=self.seq, hidden=self.hidden, ffn_shard=self.f,
                         act=L.DOMINO_ACT_SWIGLU if self.act == "swiglu" else L.DOMINO_ACT_GELU_TANH,
                         dtype=_ldtype(self.dtype),
                         row_chunks=self.row_chunks if row_chunks is None else row_chunks,
                         col_chunks=self.col_chunks if col_chunks is None else col_chunks,
                         n_partials=1 if rank_alone else self.P, no_join=no_join)

    # -- peers: their partials, computed alone (no reduction) -------------------------------
    def peer_forward(self, stream=None):
        for r in self.ranks[1:]:
            L.domino_block_fwd(self.desc(rank_alone=True, row_chunks=1, col_chunks=1), self.X, self.A_s[r],
                               self.B_s[r], self.Hpre[r], self.H[r], self.Y_own[r], None, None, self.ws,
                               self.ws_bytes, stream, None)

    def peer_backward(self, stream=None):
        dA = torch.empty_like(self.dA)
        dB = torch.empty_like(self.dB)
        for r in self.ranks[1:]:
            L.domino_block_bwd(self.desc(rank_alone=True, row_chunks=1, col_chunks=1), self.X, self.A_s[r],
                               self.B_s[r], self.Hpre[r], self.H[r], self.dY, self.dHpre[r], self.dX_own[r], None,
                               None, dA, dB, 0, self.ws, self.ws_bytes, stream, None)

    def peers(self, bufs):
        return [bufs[r] for r in self.ranks[1:]] if self.P > 1 else None

    # -- the measured rank -----------------------------------------------------------------
    def forward(self, compute=None, comm=None, **desc_kw):
        r = self.ranks[0]
        L.domino_block_fwd(self.desc(**desc_kw), self.X, self.A_s[r], self.B_s[r], self.Hpre[r], self.H[r],
                           self.Y_own[r], self.peers(self.Y_own), self.Y, self.ws, self.ws_bytes, compute, comm)

    def backward(self, compute=None, comm=None, accumulate=0, **desc_kw):
        r = self.ranks[0]
        L.domino_block_bwd(self.desc(**desc_kw), self.X, self.A_s[r], self.B_s[r], self.Hpre[r], self.H[r], self.dY,
                           self.dHpre[r], self.dX_own[r], self.peers(self.dX_own), self.dX, self.dA, self.dB,
                           accumulate, self.ws, self.ws_bytes, compute, comm)


class AttnGroup:
    """P ranks of an attention layer (head slices) on one device; rank 0 is measured."""

    def __init__(self, *, batch, seq, hidden, heads_shard, head_dim, row_chunks, n_partials, X, Aqkv, Bo,
                 device="cuda", scale=0.0, dY=None):
        self.batch, self.seq, self.hidden = batch, seq, hidden
        self.hs, self.d, self.P, self.row_chunks, self.scale = heads_shard, head_dim, n_partials, row_chunks, scale
        self.T = batch * seq
        td = torch.bfloat16
        self.X = X.to(device=device, dtype=td).contiguous()
        self.A_s, self.B_s = {}, {}
        for r in range(n_partials):
            a, b = attn_shard_weights(Aqkv, Bo, heads_shard * n_partials, head_dim, n_partials, r)
            self.A_s[r] = a.to(device=device, dtype=td)
            self.B_s[r] = b.to(device=device, dtype=td)
        hd = heads_shard * head_dim
        e = dict(device=device, dtype=td)
        self.QKV = {r: torch.empty(self.T, 3 * hd, **e) for r in range(n_partials)}
        self.O = {r: torch.empty(self.T, hd, **e) for r in range(n_partials)}
        self.Y_own = {r: torch.empty(self.T, hidden, **e) for r in range(n_partials)}
        self.Y = torch.empty(self.T, hidden, **e)
        self.lse = {r: torch.empty(self.T, heads_shard, device=device, dtype=torch.float32) for r in range(n_partials)}
        if dY is not None:
            # Backward buffers: dY is the same on every rank (Y was all-reduced).
            self.dY = dY.to(device=device, dtype=td).contiguous()
            self.dO = {r: torch.empty(self.T, hd, **e) for r in range(n_partials)}
            self.dQKV = {r: torch.empty(self.T, 3 * hd, **e) for r in range(n_partials)}
            self.dX_own = {r: torch.empty(self.T, hidden, **e) for r in range(n_partials)}
            self.dX = torch.empty(self.T, hidden, **e)
            self.dA = torch.zeros(hidden, 3 * hd, device=device, dtype=torch.float32)
            self.dB = torch.zeros(hd, hidden, device=device, dtype=torch.float32)
        descs = (self.desc(), self.desc(rank_alone=True, row_chunks=1))
        nbytes = max(max(L.domino_attn_block_fwd_workspace_size(d), L.domino_attn_block_bwd_workspace_size(d))
                     for d in descs)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        self.ws_bytes = nbytes

    def desc(self, *, rank_alone=False, row_chunks=None, no_join=0) -> L.AttnDesc:
        return L.AttnDesc(batch=self.batch, seq=self.seq, hidden=self.hidden, heads=self.hs, head_dim=self.d,
                          scale=self.scale, dtype=L.DOMINO_BF16,
                          row_chunks=self.row_chunks if row_chunks is None else row_chunks,
                          n_partials=1 if rank_alone else self.P, no_join=no_join)

    def peer_forward(self, stream=None):
        for r in range(1, self.P):
            L.domino_attn_block_fwd(self.desc(rank_alone=True, row_chunks=1), self.X, self.A_s[r], self.B_s[r],
                                    self.QKV[r], self.O[r], self.Y_own[r], None, None, self.ws, self.ws_bytes,
                                    stream, None, lse=self.lse[r])

    def forward(self, compute=None, comm=None, **desc_kw):
        peers = [self.Y_own[r] for r in range(1, self.P)] if self.P > 1 else None
        L.domino_attn_block_fwd(self.desc(**desc_kw), self.X, self.A_s[0], self.B_s[0], self.QKV[0], self.O[0],
                                self.Y_own[0], peers, self.Y, self.ws, self.ws_bytes, compute, comm, lse=self.lse[0])

    def peer_backward(self, stream=None):
        dA, dB = torch.empty_like(self.dA), torch.empty_like(self.dB)
        for r in range(1, self.P):
            L.domino_attn_block_bwd(self.desc(rank_alone=True, row_chunks=1), self.X, self.A_s[r], self.B_s[r],
                                    self.QKV[r], self.O[r], self.lse[r], self.dY, self.dO[r], self.dQKV[r],
                                    self.dX_own[r], None, None, dA, dB, 0, self.ws, self.ws_bytes, stream, None)

    def backward(self, compute=None, comm=None, accumulate=0, **desc_kw):
        peers = [self.dX_own[r] for r in range(1, self.P)] if self.P > 1 else None
        L.domino_attn_block_bwd(self.desc(**desc_kw), self.X, self.A_s[0], self.B_s[0], self.QKV[0], self.O[0],
                                self.lse[0], self.dY, self.dO[0], self.dQKV[0], self.dX_own[0], peers, self.dX,
                                self.dA, self.dB, accumulate, self.ws, self.ws_bytes, compute, comm)
