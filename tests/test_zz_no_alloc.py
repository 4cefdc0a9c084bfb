"""domino_block_bwd_noalloc (the backward whose k-split workspace is the library's static
device scratch) against domino_block_bwd with a caller workspace, through the C ABI: the
same kernels and plan, so every output must be bit-identical. Two call pairs in a row, the
second on a smaller input, so the scratch holds the first call's contents when the second
runs."""
import pytest

import synth
from gpu_util import D, torch, dev, sync, poison
from tensor_transformer_block_domino_amd.tp_sim import MlpGroup

pytestmark = pytest.mark.gpu


def group(batch, seq, hidden, ffn, act, rc, seed):
    w = synth.MlpWorkload("noalloc", batch=batch, seq=seq, hidden=hidden, ffn_shard=ffn, act=act, dtype="bf16",
                          row_chunks=rc, col_chunks=1, n_partials=3, backward=True, seed=seed)
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=batch, seq=seq, hidden=hidden, ffn_shard=ffn, act=act, dtype="bf16", row_chunks=rc,
                 col_chunks=1, n_partials=3, X=inp["X"], A=inp["A"], B=inp["B"], dY=inp["dY"], device=dev())
    g.peer_forward()
    g.forward()
    g.peer_backward()
    sync()
    return g


def outputs(g):
    return [g.dHpre[0].clone(), g.dX_own[0].clone(), g.dX.clone(), g.dA.clone(), g.dB.clone()]


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_noalloc_backward_equals_workspace_backward(act):
    comm = torch.cuda.Stream()
    # Shapes whose weight gradients split along k (few output tiles, long k = tokens), so the
    # workspace (and the static scratch) is used; the second call is smaller.
    for batch, seq, hidden, ffn, rc, seed in [(4, 1024, 512, 192, 2, 41), (2, 640, 256, 96, 2, 42)]:
        g = group(batch, seq, hidden, ffn, act, rc, seed)
        need = D.domino_block_bwd_workspace_size(g.desc())
        print(f"no-alloc backward: act={act} T={batch * seq} h={hidden} f_s={ffn} workspace {need} bytes",
              flush=True)
        assert 0 < need <= D.NOALLOC_SCRATCH_BYTES
        poison(g.dHpre[0], g.dX_own[0], g.dX)
        g.dA.fill_(0.5)
        g.dB.fill_(-0.25)
        g.backward(comm=comm, accumulate=1)
        sync()
        ref = outputs(g)
        poison(g.dHpre[0], g.dX_own[0], g.dX)
        g.dA.fill_(0.5)
        g.dB.fill_(-0.25)
        D.domino_block_bwd_noalloc(g.desc(), g.X, g.A_s[0], g.B_s[0], g.Hpre[0], g.H[0], g.dY, g.dHpre[0],
                                   g.dX_own[0], g.peers(g.dX_own), g.dX, g.dA, g.dB, 1, None, comm)
        sync()
        for name, a, b in zip(("dHpre", "dX_own", "dX", "dA_s", "dB_s"), ref, outputs(g)):
            assert torch.equal(bits(a), bits(b)), name
        del g
        torch.cuda.empty_cache()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # T·h large enough that the k-split slices exceed the static scratch: rejected before
    # anything runs (no pointers are dereferenced on that path).
    import tensor_transformer_block_domino_amd._lib as L

    dev()
    big = L.MlpDesc(batch=64, seq=4096, hidden=8192, ffn_shard=8192, act=1, dtype=1, row_chunks=1, col_chunks=1,
                    n_partials=1, no_join=0)
    need = D.domino_block_bwd_workspace_size(big)
    if need <= D.NOALLOC_SCRATCH_BYTES:
        pytest.skip(f"this shape needs only {need} bytes")
    with pytest.raises(D.DominoError, match="static scratch"):
        F = 1 << 20  # a 16-byte-aligned address that is never dereferenced (validation fails first)
        D.domino_block_bwd_noalloc(big, F, F, F, F, F, F, F, F, None, F, F, F, 0, None, None)
