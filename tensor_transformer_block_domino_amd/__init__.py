"""MI355X-native Domino tensor-parallel shard: one rank's share of a transformer layer,
X·A·B = Y, in Domino's independent row / column / 2D chunks, with the partials' sum done
on the GPU. The compute is in the HIP library (libdomino_mi355x.so); this package is its
thin Python binding plus a driver that simulates a tensor-parallel group on one GPU.
"""
from ._lib import (  # noqa: F401
    DOMINO_ACT_GELU_TANH, DOMINO_ACT_SWIGLU, DOMINO_BF16, DOMINO_F32, DOMINO_MAX_PARTIALS, EXPORTED, KERNEL_KINDS,
    LIB_PATH, AttnDesc, DominoError, MlpDesc, domino_attn_block_fwd, domino_attn_block_bwd, domino_block_bwd,
    domino_attn_block_fwd_workspace_size, domino_attn_block_bwd_workspace_size, domino_block_bwd_workspace_size,
    domino_block_fwd, domino_block_bwd_noalloc, NOALLOC_SCRATCH_BYTES,
    domino_block_fwd_workspace_size, domino_status_string, domino_timing_enable, GroupDesc, domino_resid_ln_fwd,
    domino_resid_ln_bwd, domino_resid_ln_bwd_workspace_size, LayerDesc, LayerParams, LayerActs, domino_stack_fwd,
    LayerGrads, domino_stack_bwd, domino_stack_bwd_workspace_size,
    domino_timing_kernel, domino_timing_read, load, shard_reduce,
)
