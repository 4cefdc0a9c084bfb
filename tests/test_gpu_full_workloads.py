"""The four full-size bf16 workloads, in the launch configuration bench.py times (the
workload's Domino split, reductions on a second stream), against the fp64 oracle on
sampled rows and columns (rows of Y and dX and columns of the weight gradients are
exact functions of the same rows / columns of the inputs)."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, sync, oracle, BF16_TOL, ATTN_BWD_ROW_TOL
from tensor_transformer_block_domino_amd.tp_sim import AttnGroup, MlpGroup

pytestmark = pytest.mark.gpu


def sample_rows(T, chunk_rows, n, seed):
    rng = np.random.default_rng(seed)
    edges = set()
    for c0 in range(0, T, chunk_rows):
        edges |= {c0, c0 + 1, c0 + chunk_rows - 1}
    rows = set(rng.choice(T, size=n, replace=False).tolist()) | {r for r in edges if r < T}
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["gpt3_2p7b_mlp_tp8_row", "llama2_7b_swiglu_tp8_col", "llama2_13b_swiglu_tp8_2d"])
def test_full_mlp_workload(name):
    w = synth.WORKLOADS[name]
    print(f"full workload {name}: generating inputs", flush=True)
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn_shard=w.ffn_shard, act=w.act, dtype=w.dtype,
                 row_chunks=w.row_chunks, col_chunks=w.col_chunks, n_partials=w.n_partials, X=inp["X"], A=inp["A"],
                 B=inp["B"], dY=inp["dY"], device=dev())
    print("  running the 8 ranks on the GPU", flush=True)
    g.peer_forward()
    g.forward(comm=torch.cuda.Stream())
    g.peer_backward()
    g.backward(comm=torch.cuda.Stream())
    sync()
    T = w.tokens
    rows = sample_rows(T, T // w.row_chunks, 128, seed=w.seed)
    print(f"  oracle on {len(rows)} sampled rows", flush=True)
    rt = torch.from_numpy(rows)
    X = oracle.to_f64(inp["X"][rt])
    dY = oracle.to_f64(inp["dY"][rt])
    A, B = oracle.to_f64(inp["A"]), oracle.to_f64(inp["B"])
    check("Y rows", f64(g.Y[rt.to(g.Y.device)]), oracle.mlp_y_rows(X, A, B, w.act), BF16_TOL)
    check("dX rows", f64(g.dX[rt.to(g.dX.device)]), oracle.mlp_dx_rows(X, dY, A, B, w.act), BF16_TOL)
    # Weight gradients of rank 0 on sampled FFN columns (incl. the first and last).
    A0, B0 = oracle.mlp_shard_weights(A, B, w.act, w.n_partials, 0)
    rng = np.random.default_rng(w.seed + 1)
    f = w.ffn_shard
    cols = np.array(sorted(set(rng.choice(f, size=24, replace=False).tolist()) | {0, f - 1}))
    print(f"  oracle on {len(cols)} sampled FFN columns of the weight gradients", flush=True)
    Xf, dYf = oracle.to_f64(inp["X"]), oracle.to_f64(inp["dY"])
    dA_ref, dB_ref = oracle.mlp_wgrad_slices(Xf, dYf, A0, B0, w.act, cols)
    a_cols = np.concatenate([cols, f + cols]) if w.act == "swiglu" else cols
    check("dA_s cols", f64(g.dA)[:, a_cols], dA_ref, BF16_TOL)
    check("dB_s rows", f64(g.dB)[cols], dB_ref, BF16_TOL)


def test_full_attention_workload():
    w = synth.WORKLOADS["gpt3_6p7b_attn_tp8_row"]
    print("full attention workload: generating inputs", flush=True)
    inp = synth.attn_inputs(w)
    g = AttnGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                  row_chunks=w.row_chunks, n_partials=w.n_partials, X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"],
                  device=dev())
    g.peer_forward()
    g.forward(comm=torch.cuda.Stream())
    sync()
    # Causal row 0 of every sequence equals V_0 exactly, at full size.
    O, QKV = f64(g.O[0]), f64(g.QKV[0])
    hd = w.heads_shard * w.head_dim
    for b in range(w.batch):
        assert np.array_equal(O[b * w.seq], QKV[b * w.seq, 2 * hd:3 * hd]), b
    Aqkv, Bo = oracle.to_f64(inp["Aqkv"]), oracle.to_f64(inp["Bo"])
    rng = np.random.default_rng(7)
    for b in (0, w.batch // w.row_chunks, w.batch - 1):   # first sequence of each chunk and the last
        pos = np.array(sorted(set(rng.choice(w.seq, size=10, replace=False).tolist()) | {0, 1, 127, 128, w.seq - 1}))
        print(f"  oracle on sequence {b}, {len(pos)} positions", flush=True)
        X_seq = oracle.to_f64(inp["X"][b * w.seq:(b + 1) * w.seq])
        ref = oracle.attn_y_rows(X_seq, Aqkv, Bo, w.heads_full, w.head_dim, pos)
        check(f"Y rows (seq {b})", f64(g.Y)[b * w.seq + pos], ref, BF16_TOL)


def test_full_attention_backward_workload():
    """The attention workload's backward at full size (8 ranks of 4 heads, row split x2):
    rank 0's dO, dQKV and weight gradients in full, and the reduced dX on the first sequence
    of each row chunk (a sequence's dX depends only on that sequence)."""
    w = synth.WORKLOADS["gpt3_6p7b_attn_tp8_row"]
    print("full attention backward: generating inputs", flush=True)
    inp = synth.attn_inputs(w)
    g = AttnGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                  row_chunks=w.row_chunks, n_partials=w.n_partials, X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"],
                  dY=inp["dY"], device=dev())
    print("  running the 8 ranks' forward and backward on the GPU", flush=True)
    g.peer_forward()
    g.forward(comm=torch.cuda.Stream())
    g.peer_backward()
    g.backward(comm=torch.cuda.Stream())
    sync()
    X, Aqkv, Bo, dY = (oracle.to_f64(inp[k]) for k in ("X", "Aqkv", "Bo", "dY"))
    print("  oracle: rank 0's backward over all sequences", flush=True)
    A0, B0 = oracle.attn_shard_weights(Aqkv, Bo, w.heads_full, w.head_dim, w.n_partials, 0)
    dO, dQKV, _, dA, dB = oracle.attn_shard_backward(X, A0, B0, dY, w.batch, w.seq, w.heads_shard, w.head_dim)
    check("dO", f64(g.dO[0]), dO, BF16_TOL)
    check("dQKV", f64(g.dQKV[0]), dQKV, BF16_TOL, ATTN_BWD_ROW_TOL)
    check("dA_qkv_s", f64(g.dA), dA, BF16_TOL, ATTN_BWD_ROW_TOL)
    check("dB_o_s", f64(g.dB), dB, BF16_TOL)
    dX = f64(g.dX)
    for b in (0, w.batch // w.row_chunks):
        print(f"  oracle: reduced dX of sequence {b} (all {w.heads_full} heads)", flush=True)
        r = slice(b * w.seq, (b + 1) * w.seq)
        ref = oracle.attn_backward_unsharded(X[r], Aqkv, Bo, dY[r], 1, w.seq, w.heads_full, w.head_dim)
        check(f"dX seq {b}", dX[r], ref, BF16_TOL, ATTN_BWD_ROW_TOL)


def test_full_layer_stack_workload():
    """The two-layer GPT-3 6.7B-shaped stack (8 ranks, two μ-batches, dropout 0.1) forward and
    backward in the bench's schedule; the output and dX of the first sequence of the second
    μ-batch against the oracle's unsharded stack run over that sequence alone (a sequence's
    rows depend on that sequence only)."""
    from tensor_transformer_block_domino_amd.tp_sim import LayerGroup

    w = synth.WORKLOADS["gpt3_6p7b_layer_tp8_row"]
    print("full layer stack: generating inputs", flush=True)
    inp = synth.layer_inputs(w)
    g = LayerGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                   ffn_shard=w.ffn_shard, act=w.act, row_chunks=w.row_chunks, n_partials=w.n_partials,
                   p_drop=w.p_drop, X=inp["X"], layers=inp["layers"], device=dev())
    g.alloc_backward(inp["dY"])
    print("  peer partials, then rank 0's forward and backward on the GPU", flush=True)
    g.peer_forward()
    g.peer_backward()
    g.forward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    g.backward(compute=torch.cuda.current_stream(), comm=torch.cuda.Stream())
    sync()
    b = w.batch // w.row_chunks
    rows = slice(b * w.seq, (b + 1) * w.seq)
    print(f"  oracle: the unsharded stack over sequence {b}", flush=True)
    X = oracle.to_f64(inp["X"][rows])
    dY = oracle.to_f64(inp["dY"][rows])
    layers, keeps = [], []
    for lay in inp["layers"]:
        layers.append({k: oracle.to_f64(lay[k]) for k in ("ln1_g", "ln1_b", "Aqkv", "Bo", "ln2_g", "ln2_b", "A", "B")})
        keeps.append((oracle.unpack_keep(lay["keep1"][rows].numpy(), w.hidden),
                      oracle.unpack_keep(lay["keep2"][rows].numpy(), w.hidden)))
    out, _ = oracle.stack_forward(X, layers, keeps, w.p_drop, 1, w.seq, w.heads_full, w.head_dim, w.act)
    check(f"out (sequence {b})", f64(g.out[rows]), out, BF16_TOL)
    dx, _ = oracle.stack_backward(X, layers, keeps, w.p_drop, dY, 1, w.seq, w.heads_full, w.head_dim, w.act)
    check(f"dX (sequence {b})", f64(g.dX[rows]), dx, BF16_TOL, ATTN_BWD_ROW_TOL)
