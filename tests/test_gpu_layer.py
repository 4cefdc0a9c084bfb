"""A stack of Domino transformer layers (LayerNorm, attention, dropout + residual, LayerNorm,
MLP, dropout + residual) on rank 0 of a simulated tensor-parallel group, against the fp64
oracle of the unsharded stack: the output, and rank 0's saved activations (the residual
stream entering each layer, LN1's output, the middle residual). The peer partials come from
a plain rank-by-rank run of the library over the true layer inputs."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL, ATTN_BWD_ROW_TOL
from gpu_util import check as _check
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


def oracle_stack_backward(w, inp):
    X = oracle.to_f64(inp["X"])
    layers, keeps = [], []
    for lay in inp["layers"]:
        prm = {k: oracle.to_f64(lay[k]) for k in ("ln1_g", "ln1_b", "Aqkv", "Bo", "ln2_g", "ln2_b", "A", "B")}
        prm["bo"] = oracle.to_f64(lay["bo"]) if "bo" in lay else None
        prm["b2"] = oracle.to_f64(lay["b2"]) if "b2" in lay else None
        layers.append(prm)
        keeps.append((oracle.unpack_keep(lay["keep1"].numpy(), w.hidden),
                      oracle.unpack_keep(lay["keep2"].numpy(), w.hidden)))
    d_out = oracle.to_f64(inp["dY"])
    dx, per = oracle.stack_backward(X, layers, keeps, w.p_drop, d_out, w.batch, w.seq, w.heads_full, w.head_dim, w.act)
    return dx, per, layers, keeps


def check_stack_backward(g, w, inp, with_bias=False):
    dx, per, layers, keeps = oracle_stack_backward(w, inp)
    errors = []

    def check(name, got, ref, tol, row_tol=None):  # every tensor's error is printed before the first failure
        try:
            _check(name, got, ref, tol, row_tol)
        except AssertionError as e:
            errors.append(str(e))

    check("dX", f64(g.dX), dx, BF16_TOL, ATTN_BWD_ROW_TOL)
    _, inputs = oracle.stack_forward(oracle.to_f64(inp["X"]), layers, keeps, w.p_drop, w.batch, w.seq, w.heads_full,
                                     w.head_dim, w.act)
    for l in range(w.layers):
        gr, sv = per[l]
        G = g.grads[l]
        for k_gpu, k_ref in (("d_ln1_gamma", "ln1_g"), ("d_ln1_beta", "ln1_b"), ("d_ln2_gamma", "ln2_g"),
                             ("d_ln2_beta", "ln2_b")):
            check(f"{k_gpu}[{l}]", f64(G[k_gpu]), gr[k_ref], BF16_TOL)
        if with_bias:
            check(f"d_b_o[{l}]", f64(G["d_b_o"]), gr["bo"], BF16_TOL)
            check(f"d_b_2[{l}]", f64(G["d_b_2"]), gr["b2"], BF16_TOL)
        check(f"d_ym[{l}]", f64(G["d_ym"]), gr["d_ym"], BF16_TOL)
        check(f"d_ya[{l}]", f64(G["d_ya"]), gr["d_ya"], BF16_TOL)
        A0, B0 = oracle.mlp_shard_weights(layers[l]["A"], layers[l]["B"], w.act, w.n_partials, 0)
        _, _, dA, dB = oracle.mlp_shard_backward(sv["m"], A0, B0, gr["d_ym"], w.act)
        check(f"dA_s[{l}]", f64(G["dA_s"]), dA, BF16_TOL)
        check(f"dB_s[{l}]", f64(G["dB_s"]), dB, BF16_TOL)
        Aq0, Bo0 = oracle.attn_shard_weights(layers[l]["Aqkv"], layers[l]["Bo"], w.heads_full, w.head_dim,
                                             w.n_partials, 0)
        _, _, _, dAq, dBo = oracle.attn_shard_backward(sv["a"], Aq0, Bo0, gr["d_ya"], w.batch, w.seq, w.heads_shard,
                                                       w.head_dim)
        check(f"dA_qkv_s[{l}]", f64(G["dA_qkv_s"]), dAq, BF16_TOL, ATTN_BWD_ROW_TOL)
        check(f"dB_o_s[{l}]", f64(G["dB_o_s"]), dBo, BF16_TOL)
        if l > 0:
            d_in = oracle.stack_backward(inputs[l], layers[l:], keeps[l:], w.p_drop, oracle.to_f64(inp["dY"]),
                                         w.batch, w.seq, w.heads_full, w.head_dim, w.act)[0]
            check(f"d_x_in[{l}]", f64(G["d_x_in"]), d_in, BF16_TOL, ATTN_BWD_ROW_TOL)
    assert not errors, errors


def run_backward(w, with_bias=False, comm=True):
    g, inp = make_group(w, with_bias=with_bias)
    g.alloc_backward(inp["dY"])
    g.peer_forward()
    g.peer_backward()
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    poison(g.dX, *[G["d_h"] for G in g.grads])
    g.backward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream() if comm else None)
    sync()
    return g, inp


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_stack_backward_matches_oracle(act):
    w = small_workload(act)
    print(f"layer stack bwd act={act} T={w.tokens} layers={w.layers} P={w.n_partials} mu-batches={w.row_chunks}",
          flush=True)
    g, inp = run_backward(w)
    check_stack_backward(g, w, inp)


def test_stack_backward_with_biases_three_layers_four_chunks():
    w = small_workload("gelu_tanh", row_chunks=4, layers=3)
    print("layer stack bwd with biases, layers=3, mu-batches=4", flush=True)
    g, inp = run_backward(w, with_bias=True)
    check_stack_backward(g, w, inp, with_bias=True)


def test_stack_backward_schedule_and_accumulate():
    """The second stream changes no bit; accumulate adds to every parameter gradient."""
    w = small_workload("gelu_tanh")
    print("layer stack bwd: two streams vs serial, accumulate", flush=True)
    g, inp = run_backward(w)
    first = {k: [G[k].clone() for G in g.grads] for k in ("d_ln1_gamma", "dA_s", "dB_o_s", "d_ln2_beta")}
    dX = g.dX.clone()
    g.backward(compute=torch.cuda.current_stream(), comm=None)
    sync()
    assert torch.equal(dX, g.dX)
    for k, v in first.items():
        for a, G in zip(v, g.grads):
            assert torch.equal(a, G[k]), k
    g.backward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream(), accumulate=1)
    sync()
    for k, v in first.items():
        for a, G in zip(v, g.grads):
            torch.testing.assert_close(G[k], 2 * a, rtol=1e-5, atol=1e-5)


def add_column_biases(inp, w, seed=7):
    gen = torch.Generator().manual_seed(seed)
    n_a = 2 if w.act == "swiglu" else 1
    for lay in inp["layers"]:
        lay["bqkv"] = (torch.randn(3 * w.heads_full * w.head_dim, generator=gen) * 0.1).to(torch.bfloat16)
        lay["b1"] = (torch.randn(n_a * w.ffn_full, generator=gen) * 0.1).to(torch.bfloat16)
        lay["bo"] = (torch.randn(w.hidden, generator=gen) * 0.1).to(torch.bfloat16)
        lay["b2"] = (torch.randn(w.hidden, generator=gen) * 0.1).to(torch.bfloat16)


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_stack_with_all_biases(act):
    """The column-parallel biases (QKV, first MLP product: in the GEMM epilogue, before the
    attention / activation) and the row-parallel ones (after the sum); every bias gradient."""
    from tensor_transformer_block_domino_amd.tp_sim import attn_shard_bias, mlp_shard_bias

    w = small_workload(act)
    print(f"layer stack with all biases act={act}", flush=True)
    inp = synth.layer_inputs(w)
    add_column_biases(inp, w)
    g = LayerGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                   ffn_shard=w.ffn_shard, act=w.act, row_chunks=w.row_chunks, n_partials=w.n_partials,
                   p_drop=w.p_drop, X=inp["X"], layers=inp["layers"], device=dev())
    g.alloc_backward(inp["dY"])
    g.peer_forward()
    g.peer_backward()
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    g.backward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    sync()
    X = oracle.to_f64(inp["X"])
    layers, keeps = [], []
    for lay in inp["layers"]:
        layers.append({k: oracle.to_f64(lay[k]) for k in ("ln1_g", "ln1_b", "Aqkv", "bqkv", "Bo", "bo", "ln2_g",
                                                          "ln2_b", "A", "b1", "B", "b2")})
        keeps.append((oracle.unpack_keep(lay["keep1"].numpy(), w.hidden),
                      oracle.unpack_keep(lay["keep2"].numpy(), w.hidden)))
    out, _ = oracle.stack_forward(X, layers, keeps, w.p_drop, w.batch, w.seq, w.heads_full, w.head_dim, w.act)
    check("out", f64(g.out), out, BF16_TOL)
    dx, per = oracle.stack_backward(X, layers, keeps, w.p_drop, oracle.to_f64(inp["dY"]), w.batch, w.seq,
                                    w.heads_full, w.head_dim, w.act)
    check("dX", f64(g.dX), dx, BF16_TOL)
    for l in range(w.layers):
        gr = per[l][0]
        G = g.grads[l]
        ref_bqkv = attn_shard_bias(torch.from_numpy(gr["bqkv"]), w.heads_full, w.head_dim, w.n_partials, 0).numpy()
        ref_b1 = mlp_shard_bias(torch.from_numpy(gr["b1"]), w.act, w.n_partials, 0).numpy()
        check(f"d_b_qkv[{l}]", f64(G["d_b_qkv"]), ref_bqkv, BF16_TOL)
        check(f"d_b_1[{l}]", f64(G["d_b_1"]), ref_b1, BF16_TOL)
        check(f"d_b_o[{l}]", f64(G["d_b_o"]), gr["bo"], BF16_TOL)
        check(f"d_b_2[{l}]", f64(G["d_b_2"]), gr["b2"], BF16_TOL)


def test_stack_many_mu_batches_most_partials():
    """Sixteen μ-batches of one sequence each and the largest group (16 partials): every
    μ-batch's events and reductions in both directions, forward and backward."""
    w = small_workload("swiglu", row_chunks=16, P=16, layers=2, batch=16, seq=40)
    print(f"layer stack mu-batches=16 P=16 T={w.tokens}", flush=True)
    g, inp = run_backward(w)
    check_stack(g, w, inp)
    check_stack_backward(g, w, inp)
