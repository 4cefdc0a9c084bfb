"""Products that run the 256×160 tile (four waves stacked along M, one workgroup per CU),
against the fp64 oracle, whole-tensor and row by row (normwise). Two shapes make it the tile of different
products: a wide FFN shard (forward GEMM1 and the activation-gradient product dY·B_sᵀ)
and a wide hidden size (GEMM2 per row chunk and dHpre·A_sᵀ). Both leave ragged tiles in
m (2000 rows), n (3904 columns: 24 tiles of 160 and one of 64) and k (200, or 400 for
SwiGLU's dgrad-A)."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL
from tensor_transformer_block_domino_amd.tp_sim import MlpGroup

pytestmark = pytest.mark.gpu

SHAPES = {
    # (hidden, ffn_shard, row_chunks): products expected on the 256×160 tile
    "wide_ffn": (200, 3904, 2),
    "wide_hidden": (3904, 200, 1),
}


def expected_roles(shape, act):
    if shape == "wide_ffn":
        # SwiGLU's forward pairs gate and up columns across two N-waves: other tiles.
        return ["dgrad_b"] if act == "swiglu" else ["fwd_gemm1", "dgrad_b"]
    return ["fwd_gemm2", "dgrad_a"]


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_256x160_tile_matches_oracle(shape, act):
    h, f, rc = SHAPES[shape]
    w = synth.MlpWorkload("tile160", batch=2, seq=1000, hidden=h, ffn_shard=f, act=act, dtype="bf16",
                          row_chunks=rc, col_chunks=1, n_partials=2, backward=True, seed=53)
    print(f"256x160 tile: {shape} act={act} T={w.tokens} h={h} f_s={f} row_chunks={rc}", flush=True)
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=h, ffn_shard=f, act=act, dtype="bf16", row_chunks=rc,
                 col_chunks=1, n_partials=2, X=inp["X"], A=inp["A"], B=inp["B"], dY=inp["dY"], device=dev())
    poison(g.Y, *g.Hpre.values(), *g.H.values(), *g.Y_own.values(), g.dX, *g.dHpre.values(),
           *g.dX_own.values(), g.dA, g.dB)
    g.peer_forward()
    g.peer_backward()
    D.domino_timing_enable(True)
    g.forward(comm=torch.cuda.Stream())
    g.backward(comm=torch.cuda.Stream())
    sync()
    kernels = {r: D.domino_timing_kernel(r) for r in ("fwd_gemm1", "fwd_gemm2", "dgrad_b", "dgrad_a")}
    D.domino_timing_enable(False)
    for role in expected_roles(shape, act):
        assert kernels[role].startswith("gemm_bf16_kernel<256, 160, "), (role, kernels[role])

    X, A, B, dY = (oracle.to_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    A0, B0 = oracle.mlp_shard_weights(A, B, act, 2, 0)
    Hpre, H, _ = oracle.mlp_shard_forward(X, A0, B0, act)
    check("Hpre", f64(g.Hpre[0]), Hpre, BF16_TOL)
    check("H", f64(g.H[0]), H, BF16_TOL)
    check("Y", f64(g.Y), oracle.domino_mlp_forward(X, A, B, act, 2, w.batch, w.seq, rc, 1), BF16_TOL)
    dX, dA, dB = oracle.domino_mlp_backward(X, A, B, dY, act, 2, 0, w.batch, w.seq, rc, 1)
    check("dHpre", f64(g.dHpre[0]), oracle.mlp_shard_backward(X, A0, B0, dY, act)[0], BF16_TOL)
    check("dX", f64(g.dX), dX, BF16_TOL)
    check("dA_s", f64(g.dA), dA, BF16_TOL)
    check("dB_s", f64(g.dB), dB, BF16_TOL)


# Products on the eight-wave 256×256 kernel (gemm8_kernel: two ping-pong wave groups, one
# workgroup per CU). Sizes leave ragged tiles in m (8200 rows: 32 tiles and 8 rows), n
# (4104 hidden columns, 2056 FFN columns) and k, with at least one full round of tiles.
# With the column split, the first chunk's reduction runs on the second stream while the
# second chunk's input gradient runs on the eight-wave kernel: its memory traffic slows the
# kernel's copies, which is when a copy landing late in LDS would show (it did, before the
# kernel drained every wave's copies ahead of its epilogue).
@pytest.mark.parametrize("act,col_chunks", [("gelu_tanh", 1), ("swiglu", 1), ("swiglu", 2)])
def test_8wave_tile_matches_oracle(act, col_chunks):
    h, f = 4104 if col_chunks == 1 else 4112, 2056
    w = synth.MlpWorkload("tile8w", batch=2, seq=4100, hidden=h, ffn_shard=f, act=act, dtype="bf16",
                          row_chunks=1, col_chunks=col_chunks, n_partials=2, backward=True, seed=57)
    print(f"8-wave tile: act={act} T={w.tokens} h={h} f_s={f} col_chunks={col_chunks}", flush=True)
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=h, ffn_shard=f, act=act, dtype="bf16", row_chunks=1,
                 col_chunks=col_chunks, n_partials=2, X=inp["X"], A=inp["A"], B=inp["B"], dY=inp["dY"],
                 device=dev())
    poison(g.Y, *g.Hpre.values(), *g.H.values(), *g.Y_own.values(), g.dX, *g.dHpre.values(),
           *g.dX_own.values(), g.dA, g.dB)
    g.peer_forward()
    g.peer_backward()
    D.domino_timing_enable(True)
    g.forward(comm=torch.cuda.Stream())
    g.backward(comm=torch.cuda.Stream())
    sync()
    kernels = {r: D.domino_timing_kernel(r) for r in ("fwd_gemm1", "dgrad_b", "dgrad_a")}
    D.domino_timing_enable(False)
    for role, k in kernels.items():
        assert k.startswith("gemm8_kernel<"), (role, k)

    X, A, B, dY = (oracle.to_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    A0, B0 = oracle.mlp_shard_weights(A, B, act, 2, 0)
    Hpre, H, Y0 = oracle.mlp_shard_forward(X, A0, B0, act)
    check("Hpre", f64(g.Hpre[0]), Hpre, BF16_TOL)
    check("H", f64(g.H[0]), H, BF16_TOL)
    check("Y_own", f64(g.Y_own[0]), Y0, BF16_TOL)
    check("Y", f64(g.Y), oracle.mlp_forward_unsharded(X, A, B, act), BF16_TOL)
    dHpre, dX0, dA, dB = oracle.mlp_shard_backward(X, A0, B0, dY, act)
    check("dHpre", f64(g.dHpre[0]), dHpre, BF16_TOL)
    check("dX_own", f64(g.dX_own[0]), dX0, BF16_TOL)
    check("dA_s", f64(g.dA), dA, BF16_TOL)
    check("dB_s", f64(g.dB), dB, BF16_TOL)
    check("dX", f64(g.dX), oracle.mlp_backward_unsharded(X, A, B, dY, act), BF16_TOL)
    check("Y (chunks)", f64(g.Y), oracle.domino_mlp_forward(X, A, B, act, 2, w.batch, w.seq, 1, col_chunks), BF16_TOL)
    # With its workspace the forward read the weights through transposed copies (contiguous
    # along k); without one it reads them as given. Same values in the same order: the
    # outputs agree bit for bit.
    Hp, Hh, Yo = (torch.empty_like(t) for t in (g.Hpre[0], g.H[0], g.Y_own[0]))
    d = g.desc(rank_alone=True)
    assert D.domino_block_fwd_workspace_size(d) <= g.ws_bytes
    D.domino_block_fwd(d, g.X, g.A_s[0], g.B_s[0], Hp, Hh, Yo, None, None)
    sync()
    for name, a, b in (("Hpre", Hp, g.Hpre[0]), ("H", Hh, g.H[0]), ("Y_own", Yo, g.Y_own[0])):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
