"""A stack of Domino transformer layers (LayerNorm, attention, dropout + residual, LayerNorm,
MLP, dropout + residual) on rank 0 of a simulated tensor-parallel group, against the fp64
oracle of the unsharded stack: the output, and rank 0's saved activations (the residual
stream entering each layer, LN1's output, the middle residual). The peer partials come from
a plain rank-by-rank run of the library over the true layer inputs."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL
from tensor_transformer_block_domino_amd.tp_sim import LayerGroup

pytestmark = pytest.mark.gpu


def small_workload(act="gelu_tanh", row_chunks=2, P=3, layers=2, batch=4, seq=72, p=0.1):
    return synth.LayerWorkload("small_layer", batch=batch, seq=seq, hidden=264, heads_shard=2, head_dim=128,
                               ffn_shard=136, act=act, row_chunks=row_chunks, n_partials=P, layers=layers, p_drop=p,
                               seed=29)


def make_group(w, with_bias=False):
    inp = synth.layer_inputs(w)
    if with_bias:
        gen = torch.Generator().manual_seed(99)
        for lay in inp["layers"]:
            lay["bo"] = (torch.randn(w.hidden, generator=gen) * 0.1).to(torch.bfloat16)
            lay["b2"] = (torch.randn(w.hidden, generator=gen) * 0.1).to(torch.bfloat16)
    g = LayerGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                   ffn_shard=w.ffn_shard, act=w.act, row_chunks=w.row_chunks, n_partials=w.n_partials,
                   p_drop=w.p_drop, X=inp["X"], layers=inp["layers"], device=dev())
    return g, inp


def oracle_stack(w, inp, rows=None):
    """The unsharded stack in fp64 over all rows (or the given whole sequences)."""
    X = oracle.to_f64(inp["X"])
    layers, keeps = [], []
    for lay in inp["layers"]:
        prm = {k: oracle.to_f64(lay[k]) for k in ("ln1_g", "ln1_b", "Aqkv", "Bo", "ln2_g", "ln2_b", "A", "B")}
        prm["bo"] = oracle.to_f64(lay["bo"]) if "bo" in lay else None
        prm["b2"] = oracle.to_f64(lay["b2"]) if "b2" in lay else None
        k1 = oracle.unpack_keep(lay["keep1"].numpy(), w.hidden)
        k2 = oracle.unpack_keep(lay["keep2"].numpy(), w.hidden)
        layers.append(prm)
        keeps.append((k1, k2))
    batch = w.batch
    if rows is not None:
        X = X[rows]
        keeps = [(k1[rows], k2[rows]) for k1, k2 in keeps]
        batch = (rows.stop - rows.start) // w.seq
    out, inputs = oracle.stack_forward(X, layers, keeps, w.p_drop, batch, w.seq, w.heads_full, w.head_dim, w.act)
    saved = []
    for l, prm in enumerate(layers):
        saved.append(oracle.layer_forward(inputs[l], prm, keeps[l][0], keeps[l][1], w.p_drop, batch, w.seq,
                                          w.heads_full, w.head_dim, w.act)[1])
    return out, inputs, saved


def check_stack(g, w, inp):
    out, inputs, saved = oracle_stack(w, inp)
    check("out", f64(g.out), out, BF16_TOL)
    for l in range(w.layers):
        a = g.acts[l]
        if l > 0:
            check(f"x_in[{l}]", f64(a["x_in"]), inputs[l], BF16_TOL)
        check(f"ln1[{l}]", f64(a["ln1"]), saved[l]["a"], BF16_TOL)
        check(f"h[{l}]", f64(a["h"]), saved[l]["h"], BF16_TOL)
        check(f"ln2[{l}]", f64(a["ln2"]), saved[l]["m"], BF16_TOL)


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_stack_forward_matches_oracle(act):
    w = small_workload(act)
    print(f"layer stack fwd act={act} T={w.tokens} h={w.hidden} layers={w.layers} P={w.n_partials} "
          f"mu-batches={w.row_chunks}", flush=True)
    g, inp = make_group(w)
    g.peer_forward()
    poison(g.out, *[a["h"] for a in g.acts], *[a["ln1"] for a in g.acts])
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    sync()
    check_stack(g, w, inp)


def test_stack_forward_with_biases_three_layers_four_chunks():
    w = small_workload("gelu_tanh", row_chunks=4, layers=3)
    print(f"layer stack fwd with biases, layers=3, mu-batches=4", flush=True)
    g, inp = make_group(w, with_bias=True)
    g.peer_forward()
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    sync()
    check_stack(g, w, inp)


def test_stack_forward_schedule_does_not_change_results():
    """The second stream changes no bit; one μ-batch (different launch shapes) also matches
    the oracle."""
    w = small_workload("gelu_tanh")
    print("layer stack fwd: serial vs two streams vs unsplit", flush=True)
    g, inp = make_group(w)
    g.peer_forward()
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    sync()
    two = g.out.clone()
    g.forward(compute=torch.cuda.current_stream(), comm=None)
    sync()
    assert torch.equal(two, g.out)
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream(), row_chunks=1)
    sync()
    check_stack(g, w, inp)


def test_stack_forward_one_rank_no_dropout():
    w = small_workload("swiglu", P=1, p=0.0, layers=1, batch=2, seq=130)
    print("layer stack fwd P=1, p=0, seq=130", flush=True)
    g, inp = make_group(w)
    for lay in g.params:
        lay["keep_attn"] = lay["keep_mlp"] = None
    for a in g.acts:
        a["y_attn"] = a["y_attn_own"]
        a["y_mlp"] = a["y_mlp_own"]
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    sync()
    check_stack(g, w, inp)
