"""Products whose last round of tiles is split along k (fp32 slices in the workspace,
finished by a fixed-order sum with the epilogue), against the fp64 oracle: the epilogues
of the products that split (the GeLU and SwiGLU gradients, plain stores, fp32 weight
gradients with and without accumulation), ragged M, N and K, and the same call without a
workspace. Forward products never split."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL
from tensor_transformer_block_domino_amd.tp_sim import AttnGroup, MlpGroup

pytestmark = pytest.mark.gpu


def workload(act, split=(2, 1)):
    # hidden 2048 gives dgrad-B k = 2048 on a grid of few tiles (split in two), SwiGLU's
    # dgrad-A k = 2·1040, and T = 1200 gives the weight gradients k = 1200 (split in two);
    # 1200 rows and ffn_shard 1040 leave ragged tiles in m, n and k.
    return synth.MlpWorkload("ksplit", batch=2, seq=600, hidden=2048, ffn_shard=1040, act=act, dtype="bf16",
                             row_chunks=split[0], col_chunks=split[1], n_partials=2, backward=True, seed=31)


def group(w, inp, with_ws=True):
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn_shard=w.ffn_shard, act=w.act, dtype=w.dtype,
                 row_chunks=w.row_chunks, col_chunks=w.col_chunks, n_partials=w.n_partials, X=inp["X"], A=inp["A"],
                 B=inp["B"], dY=inp["dY"], device=dev())
    if not with_ws:
        g.ws, g.ws_bytes = None, 0
    return g


def fwd_bwd(g, accumulate=0):
    poison(g.Y, *g.Hpre.values(), *g.H.values(), *g.Y_own.values(), g.dX, *g.dHpre.values(), *g.dX_own.values())
    if not accumulate:
        poison(g.dA, g.dB)
    g.peer_forward()
    g.forward(comm=torch.cuda.Stream())
    g.peer_backward()
    g.backward(comm=torch.cuda.Stream(), accumulate=accumulate)
    sync()
    return [t.detach().clone() for t in (g.Y, g.Hpre[0], g.H[0], g.dX, g.dHpre[0], g.dA, g.dB)]


NAMES = ["Y", "Hpre", "H", "dX", "dHpre", "dA_s", "dB_s"]


def references(w, inp):
    X, A, B, dY = (oracle.to_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    P, act = w.n_partials, w.act
    A0, B0 = oracle.mlp_shard_weights(A, B, act, P, 0)
    Hpre, H, _ = oracle.mlp_shard_forward(X, A0, B0, act)
    Y = oracle.domino_mlp_forward(X, A, B, act, P, w.batch, w.seq, w.row_chunks, w.col_chunks)
    dX, dA, dB = oracle.domino_mlp_backward(X, A, B, dY, act, P, 0, w.batch, w.seq, w.row_chunks, w.col_chunks)
    dHpre = oracle.mlp_shard_backward(X, A0, B0, dY, act)[0]
    return [Y, Hpre, H, dX, dHpre, dA, dB]


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_ksplit_mlp_matches_oracle_and_is_deterministic(act):
    w = workload(act)
    d = D.MlpDesc(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn_shard=w.ffn_shard,
                  act=D.DOMINO_ACT_SWIGLU if act == "swiglu" else D.DOMINO_ACT_GELU_TANH, dtype=D.DOMINO_BF16,
                  row_chunks=2, col_chunks=1, n_partials=2, no_join=0)
    assert D.domino_block_fwd_workspace_size(d) == 0 and D.domino_block_bwd_workspace_size(d) > 0
    print(f"k-split mlp act={act} T={w.tokens} h={w.hidden} f_s={w.ffn_shard} ws fwd "
          f"{D.domino_block_fwd_workspace_size(d)} bwd {D.domino_block_bwd_workspace_size(d)}", flush=True)
    inp = synth.mlp_inputs(w)
    g = group(w, inp)
    D.domino_timing_enable(True)
    outs = fwd_bwd(g)
    assert D.domino_timing_kernel("aux").startswith("gemm_fixup_kernel<")
    n_aux, _ = D.domino_timing_read("aux")
    D.domino_timing_enable(False)
    assert n_aux > 0
    for name, got, ref in zip(NAMES, outs, references(w, inp)):
        check(name, f64(got), ref, BF16_TOL)
    again = fwd_bwd(g)
    for name, a, b in zip(NAMES, outs, again):
        assert torch.equal(a, b), f"{name} differs between two identical calls"


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_ksplit_against_whole_tiles_and_accumulate(act):
    w = workload(act)
    inp = synth.mlp_inputs(w)
    whole = fwd_bwd(group(w, inp, with_ws=False))
    g = group(w, inp)
    split = fwd_bwd(g)
    for name, a, b in zip(NAMES, split, whole):
        check(f"{name} split vs whole", f64(a), f64(b), 2e-3)
    # accumulate: the split weight gradients add to what is there.
    dA1, dB1 = g.dA.clone(), g.dB.clone()
    fwd_bwd(g, accumulate=1)
    check("dA accumulated", f64(g.dA), 2 * f64(dA1), 1e-6)
    check("dB accumulated", f64(g.dB), 2 * f64(dB1), 1e-6)


def test_ksplit_too_small_workspace_runs_whole_tiles():
    w = workload("gelu_tanh")
    inp = synth.mlp_inputs(w)
    g = group(w, inp)
    g.ws_bytes = 64  # smaller than any split needs: every tile runs whole
    D.domino_timing_enable(True)
    outs = fwd_bwd(g)
    n_aux, _ = D.domino_timing_read("aux")
    D.domino_timing_enable(False)
    assert n_aux == 0
    for name, got, ref in zip(NAMES, outs, references(w, inp)):
        check(name, f64(got), ref, BF16_TOL)


def test_attention_products_do_not_split():
    batch, seq, hidden, hs, P = 2, 256, 1024, 2, 2
    w = synth.AttnWorkload("ksplit_attn", batch=batch, seq=seq, hidden=hidden, heads_shard=hs, head_dim=128,
                           dtype="bf16", row_chunks=2, n_partials=P, seed=41)
    inp = synth.attn_inputs(w)
    g = AttnGroup(batch=batch, seq=seq, hidden=hidden, heads_shard=hs, head_dim=128, row_chunks=2, n_partials=P,
                  X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"], device=dev())
    assert D.domino_attn_block_fwd_workspace_size(g.desc()) == 0  # the forward products never split
    poison(g.Y, *g.QKV.values(), *g.O.values(), *g.Y_own.values())
    g.peer_forward()
    g.forward(comm=torch.cuda.Stream())
    sync()
    X, Aqkv, Bo = (oracle.to_f64(inp[k]) for k in ("X", "Aqkv", "Bo"))
    A0, B0 = oracle.attn_shard_weights(Aqkv, Bo, hs * P, 128, P, 0)
    QKV_ref, O_ref, _ = oracle.attn_shard_forward(X, A0, B0, batch, seq, hs, 128)
    check("QKV", f64(g.QKV[0]), QKV_ref, BF16_TOL)
    check("Y", f64(g.Y), oracle.domino_attn_forward(X, Aqkv, Bo, batch, seq, hs * P, 128, P, 2), BF16_TOL)
