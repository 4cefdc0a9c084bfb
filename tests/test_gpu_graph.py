"""The Domino schedules captured into a HIP graph (torch.cuda.graph on the compute stream;
the reduction stream joins the capture through the library's own events) and replayed:
every replay, with eager work and synchronisation between replays, must equal the eager
run bit for bit. The library records no memset and allocates nothing in these calls, so
the whole step can be captured."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL
from tensor_transformer_block_domino_amd.tp_sim import LayerGroup, MlpGroup

pytestmark = pytest.mark.gpu


def replay_and_compare(graph, outputs, ref, replays=3):
    for i in range(replays):
        poison(*outputs)          # eager work on the current stream between replays
        sync()
        graph.replay()
        sync()
        diffs = []
        for name, t, r in zip(range(len(outputs)), outputs, ref):
            if not torch.equal(t, r):
                bad = (t != r) & ~(torch.isnan(t) & torch.isnan(r))
                rows = torch.nonzero(bad.reshape(bad.shape[0], -1).any(1)).flatten().tolist()
                d = (t.float() - r.float()).abs().nan_to_num(float("inf"))
                diffs.append(f"output {name}: {int(bad.sum())} elements differ (max |diff| {d.max().item():.3e}, "
                             f"nan {int(torch.isnan(t).sum())}) in rows {rows[:8]}{'...' if len(rows) > 8 else ''}")
        for msg in diffs:
            print(f"  replay {i}: {msg}", flush=True)
        assert not diffs, f"replay {i} differs from the eager run: {diffs}"


def test_mlp_block_step_as_graph():
    w = synth.MlpWorkload("graph_mlp", batch=4, seq=96, hidden=264, ffn_shard=136, act="gelu_tanh", dtype="bf16",
                          row_chunks=2, col_chunks=1, n_partials=3, backward=True, seed=41)
    print(f"graph: MLP block fwd+bwd T={w.tokens} split rows x2 P=3", flush=True)
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn_shard=w.ffn_shard, act=w.act, dtype=w.dtype,
                 row_chunks=w.row_chunks, col_chunks=w.col_chunks, n_partials=w.n_partials, X=inp["X"], A=inp["A"],
                 B=inp["B"], dY=inp["dY"], device=dev())
    g.peer_forward()
    g.peer_backward()
    compute, comm = torch.cuda.Stream(), torch.cuda.Stream()

    def step():
        g.forward(compute, comm, no_join=1)
        g.backward(compute, comm)

    step()
    sync()
    outputs = [g.Y, g.dX, g.dA, g.dB]
    ref = [t.clone() for t in outputs]
    X, A, B, dY = (oracle.to_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    check("Y (eager)", f64(g.Y), oracle.domino_mlp_forward(X, A, B, w.act, 3, w.batch, w.seq, 2, 1), BF16_TOL)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=compute):
        step()
    sync()
    replay_and_compare(graph, outputs, ref)


def test_layer_stack_step_as_graph():
    w = synth.LayerWorkload("graph_layer", batch=4, seq=72, hidden=264, heads_shard=2, head_dim=128, ffn_shard=136,
                            act="swiglu", row_chunks=2, n_partials=3, layers=2, p_drop=0.1, seed=43)
    print(f"graph: layer stack fwd+bwd T={w.tokens} layers=2 mu-batches=2 P=3", flush=True)
    inp = synth.layer_inputs(w)
    g = LayerGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                   ffn_shard=w.ffn_shard, act=w.act, row_chunks=w.row_chunks, n_partials=w.n_partials,
                   p_drop=w.p_drop, X=inp["X"], layers=inp["layers"], device=dev())
    g.alloc_backward(inp["dY"])
    g.peer_forward()
    g.peer_backward()
    compute, comm = torch.cuda.Stream(), torch.cuda.Stream()

    def step():
        g.forward(compute, comm)
        g.backward(compute, comm)

    step()
    sync()
    outputs = [g.out, g.dX] + [G[k] for G in g.grads for k in ("d_ln1_gamma", "dA_qkv_s", "dA_s", "d_ln2_beta")]
    ref = [t.clone() for t in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=compute):
        step()
    sync()
    replay_and_compare(graph, outputs, ref)
