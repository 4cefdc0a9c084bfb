"""Seeded synthetic inputs shared by the oracle tests, the GPU tests, smoke() and bench.py.

This module draws random numbers and nothing else: it holds none of the layer's
arithmetic (no slicing into shards, no products, no activations). Both sides of a
parity check read the same full tensors from here and each derives what it needs
on its own.

Recipe (one CPU generator per workload, seeded; draws in this fixed order):
  MLP:        X ~ N(0,1) [T, h];  A ~ N(0,1)*0.02 [h, n_a*F];  B ~ N(0,1)*0.02 [F, h];
              dY ~ N(0,1) [T, h]
              with F = P * f_s (the full FFN width) and n_a = 2 for SwiGLU
              (columns [gate | up], gate first), 1 for GeLU.
  attention:  X ~ N(0,1) [T, h];  Aqkv ~ N(0,1)*0.02 [h, 3*H*d] (columns [Q | K | V]);
              Bo ~ N(0,1)*0.02 [H*d, h]
Draws are fp32 (torch.randn on a CPU torch.Generator); bf16 workloads then round
each tensor to nearest-even bf16, and consumers read those exact values.
The 0.02 scale is a standard deviation (the plain reading of the N(0, 0.02)
initialiser named by the config object in the DeepSpeed-Domino 深度解析 page,
section "如何尝试 DeepSpeed-Domino").
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = ["MlpWorkload", "AttnWorkload", "WORKLOADS", "mlp_inputs", "attn_inputs", "workload"]


@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    name: str
    batch: int
    seq: int
    hidden: int
    ffn_shard: int          # f_s, the FFN width one tensor-parallel rank holds
    act: str                # "gelu_tanh" | "swiglu"
    dtype: str              # "bf16" | "f32"
    row_chunks: int         # Domino row split of X along batch
    col_chunks: int         # Domino column split of B (last dim)
    n_partials: int         # P, the tensor-parallel degree whose partials are summed
    backward: bool
    seed: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def n1(self) -> int:
        return (2 if self.act == "swiglu" else 1) * self.ffn_shard

    @property
    def ffn_full(self) -> int:
        return self.n_partials * self.ffn_shard


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    batch: int
    seq: int
    hidden: int
    heads_shard: int        # heads one rank holds
    head_dim: int
    dtype: str
    row_chunks: int
    n_partials: int
    seed: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def heads_full(self) -> int:
        return self.n_partials * self.heads_shard


# The five workloads: a tiny fp32 MLP simulating TP=2, and layers shaped like
# GPT-3 2.7B / 6.7B and Llama-2 7B / 13B at TP=8.
WORKLOADS = {
    "tiny_fp32_mlp_tp2_row": MlpWorkload(
        "tiny_fp32_mlp_tp2_row", batch=2, seq=16, hidden=64, ffn_shard=128, act="gelu_tanh",
        dtype="f32", row_chunks=2, col_chunks=1, n_partials=2, backward=False, seed=0),
    "gpt3_2p7b_mlp_tp8_row": MlpWorkload(
        "gpt3_2p7b_mlp_tp8_row", batch=4, seq=2048, hidden=2560, ffn_shard=1280, act="gelu_tanh",
        dtype="bf16", row_chunks=2, col_chunks=1, n_partials=8, backward=True, seed=1),
    "llama2_7b_swiglu_tp8_col": MlpWorkload(
        "llama2_7b_swiglu_tp8_col", batch=4, seq=4096, hidden=4096, ffn_shard=1376, act="swiglu",
        dtype="bf16", row_chunks=1, col_chunks=2, n_partials=8, backward=True, seed=2),
    "gpt3_6p7b_attn_tp8_row": AttnWorkload(
        "gpt3_6p7b_attn_tp8_row", batch=8, seq=2048, hidden=4096, heads_shard=4, head_dim=128,
        dtype="bf16", row_chunks=2, n_partials=8, seed=3),
    "llama2_13b_swiglu_tp8_2d": MlpWorkload(
        "llama2_13b_swiglu_tp8_2d", batch=8, seq=4096, hidden=5120, ffn_shard=1728, act="swiglu",
        dtype="bf16", row_chunks=2, col_chunks=2, n_partials=8, backward=True, seed=4),
}


def workload(name: str):
    return WORKLOADS[name]


def _cast(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def mlp_inputs(w: MlpWorkload, *, seed: Optional[int] = None, tokens: Optional[int] = None):
    """Full (unsharded) MLP tensors on the CPU, in the workload's storage dtype.

    Returns dict with X [T,h], A [h, n_a*F], B [F,h], dY [T,h]. `tokens` overrides T
    (used by small parity cases); `seed` overrides the workload's seed.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    T = w.tokens if tokens is None else tokens
    h, F = w.hidden, w.ffn_full
    n_a = 2 if w.act == "swiglu" else 1
    X = torch.randn(T, h, generator=g, dtype=torch.float32)
    A = torch.randn(h, n_a * F, generator=g, dtype=torch.float32) * 0.02
    B = torch.randn(F, h, generator=g, dtype=torch.float32) * 0.02
    dY = torch.randn(T, h, generator=g, dtype=torch.float32)
    return {k: _cast(v, w.dtype) for k, v in dict(X=X, A=A, B=B, dY=dY).items()}


def attn_inputs(w: AttnWorkload, *, seed: Optional[int] = None, tokens: Optional[int] = None):
    """Full attention tensors: X [T,h], Aqkv [h, 3*H*d] ([Q|K|V]), Bo [H*d, h], and the
    output gradient dY [T,h] for the backward (drawn last, so the forward tensors do not
    depend on it)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    T = w.tokens if tokens is None else tokens
    h, Hd = w.hidden, w.heads_full * w.head_dim
    X = torch.randn(T, h, generator=g, dtype=torch.float32)
    Aqkv = torch.randn(h, 3 * Hd, generator=g, dtype=torch.float32) * 0.02
    Bo = torch.randn(Hd, h, generator=g, dtype=torch.float32) * 0.02
    dY = torch.randn(T, h, generator=g, dtype=torch.float32)
    return {k: _cast(v, w.dtype) for k, v in dict(X=X, Aqkv=Aqkv, Bo=Bo, dY=dY).items()}


def randn(shape, *, seed: int, dtype: str = "bf16", scale: float = 1.0) -> torch.Tensor:
    """A standalone seeded N(0, scale^2) draw (for reduce-only and edge-case tests)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return _cast(torch.randn(*shape, generator=g, dtype=torch.float32) * scale, dtype)
