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
  group:      resid ~ N(0,1) [T, h];  y ~ N(0,1) [T, h];  bias ~ N(0,1)*0.02 [h];
              gamma ~ 1 + N(0,1)*0.1 [h];  beta ~ N(0,1)*0.1 [h];  keep: uniform u [T, h],
              kept where u >= p;  d_ln ~ N(0,1) [T, h];  d_res ~ N(0,1) [T, h]
  layer:      X ~ N(0,1) [T, h]; then per layer: ln1 gamma, beta; Aqkv; Bo; ln2 gamma, beta;
              A; B (as above); keep1, keep2; finally dY ~ N(0,1) [T, h]
Keep masks are bit-packed: element j of a row is bit j % 32 of int32 word j // 32.
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

__all__ = ["MlpWorkload", "AttnWorkload", "LayerWorkload", "WORKLOADS", "mlp_inputs", "attn_inputs",
           "group_inputs", "layer_inputs", "pack_keep", "workload"]


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


@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    """A stack of pre-LayerNorm transformer layers (attention + MLP) on one rank."""
    name: str
    batch: int
    seq: int
    hidden: int
    heads_shard: int
    head_dim: int
    ffn_shard: int
    act: str
    row_chunks: int         # μ-batches (whole sequences)
    n_partials: int
    layers: int
    p_drop: float
    seed: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def heads_full(self) -> int:
        return self.n_partials * self.heads_shard

    @property
    def ffn_full(self) -> int:
        return self.n_partials * self.ffn_shard


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
    # Whole layers of the GPT-3 6.7B shape (the attention workload's shard plus its MLP,
    # 4·h / 8 FFN columns per rank), two μ-batches, hidden dropout 0.1.
    "gpt3_6p7b_layer_tp8_row": LayerWorkload(
        "gpt3_6p7b_layer_tp8_row", batch=8, seq=2048, hidden=4096, heads_shard=4, head_dim=128, ffn_shard=2048,
        act="gelu_tanh", row_chunks=2, n_partials=8, layers=2, p_drop=0.1, seed=5),
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


def pack_keep(keep: torch.Tensor) -> torch.Tensor:
    """Bool [rows, h] -> int32 words [rows, ceil(h/32)]: element j is bit j % 32 of word j // 32."""
    import numpy as np

    rows, h = keep.shape
    words = (h + 31) // 32
    b = np.packbits(keep.numpy().astype(np.uint8), axis=1, bitorder="little")
    b = np.pad(b, ((0, 0), (0, 4 * words - b.shape[1])))
    return torch.from_numpy(np.ascontiguousarray(b).view("<i4").copy())


def _keep(g: torch.Generator, rows: int, h: int, p: float) -> torch.Tensor:
    return pack_keep(torch.rand(rows, h, generator=g, dtype=torch.float32) >= p)


def group_inputs(rows: int, hidden: int, *, seed: int, p: float = 0.1):
    """Inputs of the residual/LayerNorm group and of its backward (bf16, keep mask int32)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = dict(resid=torch.randn(rows, hidden, generator=g), y=torch.randn(rows, hidden, generator=g),
               bias=torch.randn(hidden, generator=g) * 0.02,
               gamma=1.0 + torch.randn(hidden, generator=g) * 0.1, beta=torch.randn(hidden, generator=g) * 0.1)
    keep = _keep(g, rows, hidden, p)
    out.update(d_ln=torch.randn(rows, hidden, generator=g), d_res=torch.randn(rows, hidden, generator=g))
    out = {k: v.to(torch.bfloat16) for k, v in out.items()}
    out["keep"] = keep
    return out


def layer_inputs(w: LayerWorkload, *, layers: Optional[int] = None):
    """X, per-layer parameters and keep masks, and dY of a stack (bf16; masks int32)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    T, h, Hd, F = w.tokens, w.hidden, w.heads_full * w.head_dim, w.ffn_full
    n_a = 2 if w.act == "swiglu" else 1
    bf = lambda t: t.to(torch.bfloat16)  # noqa: E731
    X = bf(torch.randn(T, h, generator=g))
    per = []
    for _ in range(w.layers if layers is None else layers):
        prm = dict(ln1_g=bf(1.0 + torch.randn(h, generator=g) * 0.1), ln1_b=bf(torch.randn(h, generator=g) * 0.1),
                   Aqkv=bf(torch.randn(h, 3 * Hd, generator=g) * 0.02), Bo=bf(torch.randn(Hd, h, generator=g) * 0.02),
                   ln2_g=bf(1.0 + torch.randn(h, generator=g) * 0.1), ln2_b=bf(torch.randn(h, generator=g) * 0.1),
                   A=bf(torch.randn(h, n_a * F, generator=g) * 0.02), B=bf(torch.randn(F, h, generator=g) * 0.02))
        prm["keep1"] = _keep(g, T, h, w.p_drop)
        prm["keep2"] = _keep(g, T, h, w.p_drop)
        per.append(prm)
    dY = bf(torch.randn(T, h, generator=g))
    return dict(X=X, layers=per, dY=dY)


def randn(shape, *, seed: int, dtype: str = "bf16", scale: float = 1.0) -> torch.Tensor:
    """A standalone seeded N(0, scale^2) draw (for reduce-only and edge-case tests)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return _cast(torch.randn(*shape, generator=g, dtype=torch.float32) * scale, dtype)
