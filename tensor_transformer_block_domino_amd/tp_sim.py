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


def mlp_shard_bias(b1: torch.Tensor, act: str, P: int, r: int):
    """Rank r's slice of the first MLP product's bias ([gate | up] for SwiGLU)."""
    F = b1.numel() // (2 if act == "swiglu" else 1)
    f = F // P
    if act == "swiglu":
        return torch.cat([b1[r * f:(r + 1) * f], b1[F + r * f:F + (r + 1) * f]]).contiguous()
    return b1[r * f:(r + 1) * f].contiguous()


def attn_shard_bias(bqkv: torch.Tensor, heads_full: int, head_dim: int, P: int, r: int):
    """Rank r's slice of the QKV bias: its heads' columns of each of Q, K, V."""
    Hd = heads_full * head_dim
    c0, c1 = r * (Hd // P), (r + 1) * (Hd // P)
    return torch.cat([bqkv[k * Hd + c0:k * Hd + c1] for k in range(3)]).contiguous()


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
        """Rank 0's forward. With rank_alone=True the call reduces nothing: Y_own is the
        output (tensor-parallel communication disabled)."""
        alone = desc_kw.get("rank_alone", False)
        peers = [self.Y_own[r] for r in range(1, self.P)] if self.P > 1 and not alone else None
        L.domino_attn_block_fwd(self.desc(**desc_kw), self.X, self.A_s[0], self.B_s[0], self.QKV[0], self.O[0],
                                self.Y_own[0], peers, None if alone else self.Y, self.ws, self.ws_bytes, compute,
                                comm, lse=self.lse[0])

    def peer_backward(self, stream=None):
        dA, dB = torch.empty_like(self.dA), torch.empty_like(self.dB)
        for r in range(1, self.P):
            L.domino_attn_block_bwd(self.desc(rank_alone=True, row_chunks=1), self.X, self.A_s[r], self.B_s[r],
                                    self.QKV[r], self.O[r], self.lse[r], self.dY, self.dO[r], self.dQKV[r],
                                    self.dX_own[r], None, None, dA, dB, 0, self.ws, self.ws_bytes, stream, None)

    def backward(self, compute=None, comm=None, accumulate=0, **desc_kw):
        """Rank 0's backward; rank_alone=True reduces nothing (dX_own is the output)."""
        alone = desc_kw.get("rank_alone", False)
        peers = [self.dX_own[r] for r in range(1, self.P)] if self.P > 1 and not alone else None
        L.domino_attn_block_bwd(self.desc(**desc_kw), self.X, self.A_s[0], self.B_s[0], self.QKV[0], self.O[0],
                                self.lse[0], self.dY, self.dO[0], self.dQKV[0], self.dX_own[0], peers,
                                None if alone else self.dX, self.dA, self.dB, accumulate, self.ws, self.ws_bytes,
                                compute, comm)


_ACTS = {"gelu_tanh": L.DOMINO_ACT_GELU_TANH, "swiglu": L.DOMINO_ACT_SWIGLU}


class LayerGroup:
    """P ranks of a stack of Domino transformer layers on one device; rank 0 is measured.

    `layers` is a list of per-layer dicts of full (unsharded) CPU tensors: ln1_g, ln1_b, Aqkv,
    Bo, ln2_g, ln2_b, A, B, keep1, keep2 (and optionally bo, b2). peer_forward() runs the
    stack once rank by rank with the plain library calls (each rank's attention and MLP
    partials, their sums, the groups) so every layer's peer partials are those the other GPUs
    would hold for the true layer inputs; forward() then runs rank 0's Domino schedule.
    """

    def __init__(self, *, batch, seq, hidden, heads_shard, head_dim, ffn_shard, act, row_chunks, n_partials, p_drop,
                 X, layers, device="cuda", eps=1e-5):
        self.batch, self.seq, self.hidden, self.hs, self.d = batch, seq, hidden, heads_shard, head_dim
        self.f, self.act, self.rc, self.P, self.p, self.eps = ffn_shard, act, row_chunks, n_partials, p_drop, eps
        self.T = T = batch * seq
        self.L = len(layers)
        P, h, hd = n_partials, hidden, heads_shard * head_dim
        n1 = 2 * ffn_shard if act == "swiglu" else ffn_shard
        bf = dict(device=device, dtype=torch.bfloat16)
        f32 = dict(device=device, dtype=torch.float32)
        self.X = X.to(**bf).contiguous()
        self.out = torch.empty(T, h, **bf)
        self.rank_prm = []   # [layer][rank] dict of device tensors
        self.params = []     # rank 0's domino_layer_params per layer
        self.acts = []       # rank 0's domino_layer_acts per layer
        self.peer = []       # [layer] dict of peer partial lists
        for l, lay in enumerate(layers):
            ranks = []
            for r in range(P):
                Aq, Bo = attn_shard_weights(lay["Aqkv"], lay["Bo"], heads_shard * P, head_dim, P, r)
                A_s, B_s = mlp_shard_weights(lay["A"], lay["B"], act, P, r)
                rk = dict(A_qkv_s=Aq.to(**bf), B_o_s=Bo.to(**bf), A_s=A_s.to(**bf), B_s=B_s.to(**bf), b_qkv_s=None,
                          b_1_s=None)
                if lay.get("bqkv") is not None:
                    rk["b_qkv_s"] = attn_shard_bias(lay["bqkv"], heads_shard * P, head_dim, P, r).to(**bf)
                if lay.get("b1") is not None:
                    rk["b_1_s"] = mlp_shard_bias(lay["b1"], act, P, r).to(**bf)
                ranks.append(rk)
            self.rank_prm.append(ranks)
            dev_or_none = lambda k: None if lay.get(k) is None else lay[k].to(device).contiguous()  # noqa: E731
            self.params.append(dict(ln1_gamma=dev_or_none("ln1_g"), ln1_beta=dev_or_none("ln1_b"),
                                    A_qkv_s=ranks[0]["A_qkv_s"], B_o_s=ranks[0]["B_o_s"], b_o=dev_or_none("bo"),
                                    ln2_gamma=dev_or_none("ln2_g"), ln2_beta=dev_or_none("ln2_b"),
                                    A_s=ranks[0]["A_s"], B_s=ranks[0]["B_s"], b_2=dev_or_none("b2"),
                                    keep_attn=dev_or_none("keep1"), keep_mlp=dev_or_none("keep2"),
                                    b_qkv=ranks[0]["b_qkv_s"], b_1=ranks[0]["b_1_s"]))
            peer = dict(y_attn=[torch.empty(T, h, **bf) for _ in range(P - 1)],
                        y_mlp=[torch.empty(T, h, **bf) for _ in range(P - 1)])
            self.peer.append(peer)
            self.acts.append(dict(
                x_in=None if l == 0 else torch.empty(T, h, **bf), ln1=torch.empty(T, h, **bf),
                mean1=torch.empty(T, **f32), rstd1=torch.empty(T, **f32), QKV=torch.empty(T, 3 * hd, **bf),
                O=torch.empty(T, hd, **bf), lse=torch.empty(T, heads_shard, **f32), y_attn_own=torch.empty(T, h, **bf),
                peer_y_attn=peer["y_attn"] if P > 1 else None, y_attn=torch.empty(T, h, **bf),
                h=torch.empty(T, h, **bf), ln2=torch.empty(T, h, **bf), mean2=torch.empty(T, **f32),
                rstd2=torch.empty(T, **f32), Hpre=torch.empty(T, n1, **bf), H=torch.empty(T, ffn_shard, **bf),
                y_mlp_own=torch.empty(T, h, **bf), peer_y_mlp=peer["y_mlp"] if P > 1 else None,
                y_mlp=torch.empty(T, h, **bf)))
        ws_attn = L.domino_attn_block_fwd_workspace_size(self._attn_desc())
        ws_mlp = L.domino_block_fwd_workspace_size(self._mlp_desc())
        self.ws_bytes = max(ws_attn, ws_mlp)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)

    def desc(self, *, row_chunks=None, rank_alone=False) -> L.LayerDesc:
        return L.LayerDesc(batch=self.batch, seq=self.seq, hidden=self.hidden, heads=self.hs, head_dim=self.d,
                           ffn_shard=self.f, act=_ACTS[self.act], eps=self.eps, p_drop=self.p, scale=0.0,
                           row_chunks=self.rc if row_chunks is None else row_chunks,
                           n_partials=1 if rank_alone else self.P, layers=self.L, reserved=0)

    def _attn_desc(self):
        return L.AttnDesc(batch=self.batch, seq=self.seq, hidden=self.hidden, heads=self.hs, head_dim=self.d, scale=0.0,
                          dtype=L.DOMINO_BF16, row_chunks=1, n_partials=1, no_join=0)

    def _mlp_desc(self):
        return L.MlpDesc(batch=self.batch, seq=self.seq, hidden=self.hidden, ffn_shard=self.f, act=_ACTS[self.act],
                         dtype=L.DOMINO_BF16, row_chunks=1, col_chunks=1, n_partials=1, no_join=0)

    def peer_forward(self, stream=None):
        """Every rank's partials of every layer, from the true layer inputs, by plain calls."""
        T, h, hd, P = self.T, self.hidden, self.hs * self.d, self.P
        n1 = 2 * self.f if self.act == "swiglu" else self.f
        bf = dict(device=self.X.device, dtype=torch.bfloat16)
        f32 = dict(device=self.X.device, dtype=torch.float32)
        gd = L.GroupDesc(rows=T, hidden=h, eps=self.eps, p_drop=self.p)
        x, a, hh, m = self.X, torch.empty(T, h, **bf), torch.empty(T, h, **bf), torch.empty(T, h, **bf)
        mean, rstd = torch.empty(T, **f32), torch.empty(T, **f32)
        qkv, o = torch.empty(T, 3 * hd, **bf), torch.empty(T, hd, **bf)
        hpre, hmid = torch.empty(T, n1, **bf), torch.empty(T, self.f, **bf)
        own, y = torch.empty(T, h, **bf), torch.empty(T, h, **bf)
        nxt = [torch.empty(T, h, **bf), torch.empty(T, h, **bf)]
        ad, md = self._attn_desc(), self._mlp_desc()
        for l in range(self.L):
            prm, ranks, peer = self.params[l], self.rank_prm[l], self.peer[l]
            L.domino_resid_ln_fwd(gd, x, None, None, None, x, prm["ln1_gamma"], prm["ln1_beta"], a, mean, rstd, stream)
            for r in range(P):
                dst = own if r == 0 else peer["y_attn"][r - 1]
                L.domino_attn_block_fwd(ad, a, ranks[r]["A_qkv_s"], ranks[r]["B_o_s"], qkv, o, dst, None, None,
                                        self.ws, self.ws_bytes, stream, None, b_qkv_s=ranks[r]["b_qkv_s"])
            L.shard_reduce(y, h, [own] + peer["y_attn"], h, T, h, L.DOMINO_BF16, stream)
            L.domino_resid_ln_fwd(gd, x, y, prm["b_o"], prm["keep_attn"], hh, prm["ln2_gamma"], prm["ln2_beta"], m,
                                  mean, rstd, stream)
            for r in range(P):
                dst = own if r == 0 else peer["y_mlp"][r - 1]
                L.domino_block_fwd(md, m, ranks[r]["A_s"], ranks[r]["B_s"], hpre, hmid, dst, None, None, self.ws,
                                   self.ws_bytes, stream, None, b1_s=ranks[r]["b_1_s"])
            L.shard_reduce(y, h, [own] + peer["y_mlp"], h, T, h, L.DOMINO_BF16, stream)
            x = nxt[l % 2]
            L.domino_resid_ln_fwd(gd, hh, y, prm["b_2"], prm["keep_mlp"], x, None, None, None, None, None, stream)

    def forward(self, compute=None, comm=None, **desc_kw):
        L.domino_stack_fwd(self.desc(**desc_kw), self.X, self.params, self.acts, self.out, self.ws, self.ws_bytes,
                           compute, comm)

    # ------------------------------------------------------------------------------------
    # Backward
    # ------------------------------------------------------------------------------------
    def alloc_backward(self, d_out: torch.Tensor):
        T, h, hd, P = self.T, self.hidden, self.hs * self.d, self.P
        n1 = 2 * self.f if self.act == "swiglu" else self.f
        dev = self.X.device
        bf = dict(device=dev, dtype=torch.bfloat16)
        f32 = dict(device=dev, dtype=torch.float32)
        self.d_out = d_out.to(**bf).contiguous()
        self.dX = torch.empty(T, h, **bf)
        self.grads, self.peer_grad = [], []
        for l in range(self.L):
            pg = dict(dx_mlp=[torch.empty(T, h, **bf) for _ in range(P - 1)],
                      dx_attn=[torch.empty(T, h, **bf) for _ in range(P - 1)])
            self.peer_grad.append(pg)
            has_bo, has_b2 = self.params[l]["b_o"] is not None, self.params[l]["b_2"] is not None
            self.grads.append(dict(
                d_ln1_gamma=torch.zeros(h, **f32), d_ln1_beta=torch.zeros(h, **f32),
                dA_qkv_s=torch.zeros(h, 3 * hd, **f32), dB_o_s=torch.zeros(hd, h, **f32),
                d_b_o=torch.zeros(h, **f32) if has_bo else None,
                d_ln2_gamma=torch.zeros(h, **f32), d_ln2_beta=torch.zeros(h, **f32),
                dA_s=torch.zeros(h, n1, **f32), dB_s=torch.zeros(self.f, h, **f32),
                d_b_2=torch.zeros(h, **f32) if has_b2 else None,
                d_x_in=None if l == 0 else torch.empty(T, h, **bf), d_ym=torch.empty(T, h, **bf),
                dHpre=torch.empty(T, n1, **bf), dx_mlp_own=torch.empty(T, h, **bf),
                peer_dx_mlp=pg["dx_mlp"] if P > 1 else None, dx_mlp=torch.empty(T, h, **bf),
                d_h=torch.empty(T, h, **bf), d_ya=torch.empty(T, h, **bf), dO=torch.empty(T, hd, **bf),
                dQKV=torch.empty(T, 3 * hd, **bf), dx_attn_own=torch.empty(T, h, **bf),
                peer_dx_attn=pg["dx_attn"] if P > 1 else None, dx_attn=torch.empty(T, h, **bf),
                d_b_qkv=torch.zeros(3 * hd, **f32) if self.params[l]["b_qkv"] is not None else None,
                d_b_1=torch.zeros(n1, **f32) if self.params[l]["b_1"] is not None else None))
        self.bws_bytes = max(L.domino_stack_bwd_workspace_size(self.desc()),
                             L.domino_stack_bwd_workspace_size(self.desc(row_chunks=1)),
                             L.domino_attn_block_bwd_workspace_size(self._attn_desc()),
                             L.domino_block_bwd_workspace_size(self._mlp_desc()),
                             L.domino_resid_ln_bwd_workspace_size(L.GroupDesc(rows=T, hidden=h, eps=self.eps,
                                                                              p_drop=self.p)))
        self.bws = torch.empty(max(self.bws_bytes, 16), dtype=torch.uint8, device=dev)

    def peer_backward(self, stream=None):
        """Every rank's input-gradient partials of every layer, from the true layer gradients,
        by plain calls: a reference forward keeps each layer's LayerNorm inputs and outputs,
        then the backward runs top down, each rank recomputing its own forward activations."""
        T, h, hd, P, f = self.T, self.hidden, self.hs * self.d, self.P, self.f
        n1 = 2 * f if self.act == "swiglu" else f
        bf = dict(device=self.X.device, dtype=torch.bfloat16)
        f32 = dict(device=self.X.device, dtype=torch.float32)
        gd = L.GroupDesc(rows=T, hidden=h, eps=self.eps, p_drop=self.p)
        ad, md = self._attn_desc(), self._mlp_desc()
        qkv, o, lse = torch.empty(T, 3 * hd, **bf), torch.empty(T, hd, **bf), torch.empty(T, self.hs, **f32)
        hpre, hmid = torch.empty(T, n1, **bf), torch.empty(T, f, **bf)
        own, y = torch.empty(T, h, **bf), torch.empty(T, h, **bf)
        # Reference forward, keeping what the backward needs.
        ref = []
        x = self.X
        for l in range(self.L):
            prm, ranks = self.params[l], self.rank_prm[l]
            r = dict(x=x, a=torch.empty(T, h, **bf), m1=torch.empty(T, **f32), s1=torch.empty(T, **f32),
                     hh=torch.empty(T, h, **bf), m=torch.empty(T, h, **bf), m2=torch.empty(T, **f32),
                     s2=torch.empty(T, **f32))
            L.domino_resid_ln_fwd(gd, x, None, None, None, x, prm["ln1_gamma"], prm["ln1_beta"], r["a"], r["m1"],
                                  r["s1"], stream)
            parts = []
            for k in range(P):
                dst = own if k == 0 else torch.empty(T, h, **bf)
                L.domino_attn_block_fwd(ad, r["a"], ranks[k]["A_qkv_s"], ranks[k]["B_o_s"], qkv, o, dst, None, None,
                                        self.ws, self.ws_bytes, stream, None, b_qkv_s=ranks[k]["b_qkv_s"])
                parts.append(dst)
            L.shard_reduce(y, h, parts, h, T, h, L.DOMINO_BF16, stream)
            L.domino_resid_ln_fwd(gd, x, y, prm["b_o"], prm["keep_attn"], r["hh"], prm["ln2_gamma"], prm["ln2_beta"],
                                  r["m"], r["m2"], r["s2"], stream)
            parts = []
            for k in range(P):
                dst = own if k == 0 else torch.empty(T, h, **bf)
                L.domino_block_fwd(md, r["m"], ranks[k]["A_s"], ranks[k]["B_s"], hpre, hmid, dst, None, None, self.ws,
                                   self.ws_bytes, stream, None, b1_s=ranks[k]["b_1_s"])
                parts.append(dst)
            L.shard_reduce(y, h, parts, h, T, h, L.DOMINO_BF16, stream)
            x = torch.empty(T, h, **bf)
            L.domino_resid_ln_fwd(gd, r["hh"], y, prm["b_2"], prm["keep_mlp"], x, None, None, None, None, None,
                                  stream)
            ref.append(r)
        # Reference backward.
        d_r = self.d_out
        d_ym, d_h, d_ya, scratch, y_fwd = (torch.empty(T, h, **bf) for _ in range(5))
        dHpre, dO, dQKV = torch.empty(T, n1, **bf), torch.empty(T, hd, **bf), torch.empty(T, 3 * hd, **bf)
        dA_m, dB_m = torch.empty(h, n1, **f32), torch.empty(f, h, **f32)
        dA_a, dB_a = torch.empty(h, 3 * hd, **f32), torch.empty(hd, h, **f32)
        for l in range(self.L - 1, -1, -1):
            prm, ranks, pg, r = self.params[l], self.rank_prm[l], self.peer_grad[l], ref[l]
            L.domino_resid_ln_bwd(gd, None, d_r, None, None, None, None, prm["keep_mlp"], scratch, d_ym, None, None,
                                  None, 0, self.bws, self.bws_bytes, stream)
            parts = []
            for k in range(P):
                L.domino_block_fwd(md, r["m"], ranks[k]["A_s"], ranks[k]["B_s"], hpre, hmid, y_fwd, None, None,
                                   self.ws, self.ws_bytes, stream, None, b1_s=ranks[k]["b_1_s"])
                dst = own if k == 0 else pg["dx_mlp"][k - 1]
                L.domino_block_bwd(md, r["m"], ranks[k]["A_s"], ranks[k]["B_s"], hpre, hmid, d_ym, dHpre, dst, None,
                                   None, dA_m, dB_m, 0, self.bws, self.bws_bytes, stream, None)
                parts.append(dst)
            L.shard_reduce(y, h, parts, h, T, h, L.DOMINO_BF16, stream)
            L.domino_resid_ln_bwd(gd, y, d_r, r["hh"], r["m2"], r["s2"], prm["ln2_gamma"], prm["keep_attn"], d_h, d_ya,
                                  None, None, None, 0, self.bws, self.bws_bytes, stream)
            parts = []
            for k in range(P):
                L.domino_attn_block_fwd(ad, r["a"], ranks[k]["A_qkv_s"], ranks[k]["B_o_s"], qkv, o, y_fwd, None, None,
                                        self.ws, self.ws_bytes, stream, None, lse=lse, b_qkv_s=ranks[k]["b_qkv_s"])
                dst = own if k == 0 else pg["dx_attn"][k - 1]
                L.domino_attn_block_bwd(ad, r["a"], ranks[k]["A_qkv_s"], ranks[k]["B_o_s"], qkv, o, lse, d_ya, dO, dQKV,
                                        dst, None, None, dA_a, dB_a, 0, self.bws, self.bws_bytes, stream, None)
                parts.append(dst)
            L.shard_reduce(y, h, parts, h, T, h, L.DOMINO_BF16, stream)
            d_x = torch.empty(T, h, **bf)
            L.domino_resid_ln_bwd(gd, y, d_h, r["x"], r["m1"], r["s1"], prm["ln1_gamma"], None, d_x, None, None, None,
                                  None, 0, self.bws, self.bws_bytes, stream)
            d_r = d_x

    def backward(self, compute=None, comm=None, accumulate=0, **desc_kw):
        L.domino_stack_bwd(self.desc(**desc_kw), self.X, self.params, self.acts, self.grads, self.d_out, self.dX,
                           accumulate, self.bws, self.bws_bytes, compute, comm)
