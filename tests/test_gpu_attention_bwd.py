"""Attention shard backward on the GPU against the fp64 oracle: dO, dQKV = [dQ | dK | dV]
of the causal attention, the reduced dX (by row chunks), and the rank's fp32 weight
gradients, on ragged sequence lengths (1, 64, 130, 200, 333), one and two heads per
rank, one and two row chunks; determinism and accumulation."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL, ATTN_BWD_ROW_TOL
from tensor_transformer_block_domino_amd.tp_sim import AttnGroup

pytestmark = pytest.mark.gpu


def run(batch, seq, hidden, hs, P, row_chunks, seed=23, accumulate=0, group=None):
    w = synth.AttnWorkload("small_attn_bwd", batch=batch, seq=seq, hidden=hidden, heads_shard=hs, head_dim=128,
                           dtype="bf16", row_chunks=row_chunks, n_partials=P, seed=seed)
    inp = synth.attn_inputs(w)
    g = group or AttnGroup(batch=batch, seq=seq, hidden=hidden, heads_shard=hs, head_dim=128, row_chunks=row_chunks,
                           n_partials=P, X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"], dY=inp["dY"], device=dev())
    poison(g.dX, *g.dO.values(), *g.dQKV.values(), *g.dX_own.values())
    if not accumulate:
        poison(g.dA, g.dB)
    g.peer_forward()
    g.forward(comm=torch.cuda.Stream())
    g.peer_backward()
    g.backward(comm=torch.cuda.Stream(), accumulate=accumulate)
    sync()
    return g, inp, w


def references(inp, batch, seq, hs, P, row_chunks):
    X, Aqkv, Bo, dY = (oracle.to_f64(inp[k]) for k in ("X", "Aqkv", "Bo", "dY"))
    A0, B0 = oracle.attn_shard_weights(Aqkv, Bo, hs * P, 128, P, 0)
    dO, dQKV, _, _, _ = oracle.attn_shard_backward(X, A0, B0, dY, batch, seq, hs, 128)
    dX, dA, dB = oracle.domino_attn_backward(X, Aqkv, Bo, dY, batch, seq, hs * P, 128, P, 0, row_chunks)
    return dO, dQKV, dX, dA, dB


@pytest.mark.parametrize("batch,seq,hs,row_chunks", [(2, 200, 2, 2), (2, 64, 1, 1), (1, 333, 1, 1), (2, 1, 2, 2),
                                                      (4, 130, 2, 2)])
def test_attention_backward_small(batch, seq, hs, row_chunks):
    hidden, P = 256, 2
    print(f"attention backward batch={batch} seq={seq} heads/rank={hs} P={P} chunks={row_chunks}", flush=True)
    g, inp, w = run(batch, seq, hidden, hs, P, row_chunks)
    dO, dQKV, dX, dA, dB = references(inp, batch, seq, hs, P, row_chunks)
    hd = hs * 128
    got = f64(g.dQKV[0])
    check("dO", f64(g.dO[0]), dO, BF16_TOL)
    check("dV", got[:, 2 * hd:], dQKV[:, 2 * hd:], BF16_TOL)
    if seq == 1:
        # One token: O = V whatever Q and K, so dQ = dK = 0 exactly; the GPU's differ from 0
        # only by the rounding of dP − Δ (two fp32 sums of the same products).
        bound = 1e-3 * float(np.max(np.abs(dQKV[:, 2 * hd:])))
        for name, blk in (("dQ", got[:, :hd]), ("dK", got[:, hd:2 * hd])):
            print(f"  {name}: max abs {np.max(np.abs(blk)):.3e} (exact 0, bound {bound:.3e})", flush=True)
            assert np.max(np.abs(blk)) <= bound, name
    else:
        check("dQ", got[:, :hd], dQKV[:, :hd], BF16_TOL, ATTN_BWD_ROW_TOL)
        check("dK", got[:, hd:2 * hd], dQKV[:, hd:2 * hd], BF16_TOL, ATTN_BWD_ROW_TOL)
    check("dX", f64(g.dX), dX, BF16_TOL, ATTN_BWD_ROW_TOL)
    check("dA_qkv_s", f64(g.dA), dA, BF16_TOL, ATTN_BWD_ROW_TOL)
    check("dB_o_s", f64(g.dB), dB, BF16_TOL)


def test_attention_backward_deterministic_and_accumulates():
    batch, seq, hidden, hs, P = 2, 200, 256, 2, 2
    g, inp, w = run(batch, seq, hidden, hs, P, 2)
    first = [t.detach().clone() for t in (g.dQKV[0], g.dX, g.dA, g.dB)]
    g, _, _ = run(batch, seq, hidden, hs, P, 2, group=g)
    for name, a, b in zip(("dQKV", "dX", "dA", "dB"), first, (g.dQKV[0], g.dX, g.dA, g.dB)):
        assert torch.equal(a, b), f"{name} differs between two identical calls"
    g, _, _ = run(batch, seq, hidden, hs, P, 2, group=g, accumulate=1)
    check("dA accumulated", f64(g.dA), 2 * f64(first[2]), 1e-6)
    check("dB accumulated", f64(g.dB), 2 * f64(first[3]), 1e-6)


def test_attention_backward_workspace_required():
    batch, seq, hidden, hs = 1, 64, 128, 1
    w = synth.AttnWorkload("s", batch=batch, seq=seq, hidden=hidden, heads_shard=hs, head_dim=128, dtype="bf16",
                           row_chunks=1, n_partials=1, seed=5)
    inp = synth.attn_inputs(w)
    g = AttnGroup(batch=batch, seq=seq, hidden=hidden, heads_shard=hs, head_dim=128, row_chunks=1, n_partials=1,
                  X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"], dY=inp["dY"], device=dev())
    g.forward()
    sync()
    g.ws_bytes = 64
    with pytest.raises(D.DominoError) as e:
        g.backward()
    assert e.value.status == 1  # DOMINO_ERR_INVALID_ARG, before anything is enqueued
