"""CPU fp64 oracle of one tensor-parallel rank's share of a transformer layer, Y = X·A·B.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The HIP library never calls it and
shares no code, header, table or helper with it; the two meet only in the seeded
draws of `synth`.

Everything here is plain numpy in float64: bf16/fp32 inputs are upcast exactly,
and no intermediate result is rounded. Library matmuls are used as steps; there is
no blocking, fusion or reordering beyond what the definitions state, so each
function can be checked against its source by eye.

Sources (web pages, by title and section):
  [Domino]  "DeepSpeed-Domino 深度解析：通过通用张量切分与计算通信重叠实现单机与多节点统一的
            LLM 张量并行训练" — sections "TP 的数据依赖：通信为何难以隐藏" (the layer as
            X·A·B = Y followed by an AllReduce of Y), "按行切分输入 X", "按列切分权重 B",
            "2D 切分（同时切 X 与 B）", "反向：扩展与权重梯度计算的重叠",
            "μ-batch 流水：DominoTransformer 与 DominoTransformerLayer".
  [Primer]  "从单卡到集群…" (parallel-training primer), §3.1 "TP的切分方式与计算模式"
            (column-parallel and row-parallel linear layers; FFN = column then row).
  [Overlap] "04 · TP/SP 的通信-计算 overlap 与工程优化", §1 "粗粒度：dgrad 通信 ∥ wgrad 计算"
            (grad_input = grad_output·Wᵀ needs the reduce; grad_weight is local).
  The layer (layer.py) follows [Domino] "前向：多个计算片段轮转重叠 AllReduce" (attention,
  then the small kernels Dropout, Residual, LayerNorm, then the MLP) and the
  DominoTransformerLayer excerpt under "μ-batch 流水" (pre-LayerNorm block).

Readings where the pages are silent (the plainest reading the rest of the pages supports):
  GeLU is the tanh form; SwiGLU is silu(gate)*up with A's columns [gate | up];
  shards are contiguous equal column blocks of A and the matching row blocks of B
  (contiguous head blocks for attention); the row split is along batch with
  torch.chunk sizes; attention is causal self-attention with scale 1/sqrt(d) and
  no bias, dropout or rotary embedding; LayerNorm uses the biased variance and eps 1e-5
  inside the root; dropout is inverted dropout with a given keep mask.

Every function below is pinned by tests/test_oracle_pins.py and tests/test_oracle_layer_pins.py (brute-force scalar
loops, the split and shard-sum identities, finite differences, closed forms and
library cross-checks); none is "parity unpinned".
"""
from .mlp import (  # noqa: F401
    to_f64, gelu_tanh, gelu_tanh_grad, sigmoid, silu, act_forward, act_backward,
    shard_slice, mlp_shard_weights, mlp_shard_forward, mlp_shard_backward,
    mlp_forward_unsharded, mlp_backward_unsharded, shard_sum,
    row_chunk_ranges, col_chunk_ranges, domino_mlp_forward, domino_mlp_backward,
    mlp_dx_rows, mlp_y_rows, mlp_wgrad_slices,
)
from .attention import (  # noqa: F401
    attn_shard_weights, causal_attention, attn_shard_forward, attn_forward_unsharded,
    attn_y_rows, domino_attn_forward, causal_attention_lse, causal_attention_backward,
    attn_lse, attn_shard_backward, attn_backward_unsharded, domino_attn_backward,
)
from .layer import (  # noqa: F401
    LN_EPS, unpack_keep, dropout, layer_norm, layer_norm_backward, resid_group_forward,
    resid_group_backward, layer_forward, layer_backward, stack_forward, stack_backward,
)
