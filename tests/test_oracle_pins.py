"""Pins of the CPU oracle against things other than itself (CPU only).

The pages print no tensor values, so the oracle is pinned by:
  * brute-force scalar loops on tiny shapes (an independent evaluation route);
  * the identities the pages fix: row-chunk, column-chunk and 2D-chunk outputs equal
    the unsplit Y; the sum of shard partials equals the unsharded layer (for attention,
    the sum over head-slice shards equals full multi-head attention);
  * central finite differences and the adjoint identity for the backward (MLP and
    attention), torch autograd through scaled-dot-product attention for the attention
    backward, and its closed forms (one token: dV = dO, dQ = dK = 0; Q = 0: dV_k =
    Σ_{i≥k} dO_i/(i+1); V = ones: dQ = dK = 0), scipy's logsumexp for the LSE;
  * closed forms and special cases (gelu(0)=0, gelu'(0)=1/2, first causal row = V_0,
    Q = 0 gives prefix means, softmax rows sum to 1);
  * library routines for special cases (torch's tanh-GeLU and SiLU, torch autograd,
    torch's causal scaled-dot-product attention, scipy's exact erf GeLU within the
    tanh form's approximation error).
A final test plants plausible mistakes in the oracle and checks that a pin fails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mlp as omlp
from oracle import attention as oattn

RNG = np.random.default_rng(12345)


def rnd(*shape, scale=1.0, rng=None):
    return (rng or RNG).standard_normal(shape) * scale


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


# ------------------------------------------------------------------------------------------
# Brute force: scalar loops in pure Python.
# ------------------------------------------------------------------------------------------
def bf_matmul(A, B):
    n, k = len(A), len(A[0])
    m = len(B[0])
    return [[sum(A[i][t] * B[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def bf_gelu(x):
    return 0.5 * x * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def bf_silu(x):
    return x / (1.0 + math.exp(-x))


def bf_mlp_shard_forward(X, A_s, B_s, act):
    Hpre = bf_matmul(X, A_s)
    if act == "gelu_tanh":
        H = [[bf_gelu(v) for v in row] for row in Hpre]
    else:
        f = len(Hpre[0]) // 2
        H = [[bf_silu(row[j]) * row[f + j] for j in range(f)] for row in Hpre]
    return Hpre, H, bf_matmul(H, B_s)


def bf_causal_attention(Q, K, V, scale):
    n, d = len(Q), len(Q[0])
    out = []
    for i in range(n):
        s = [scale * sum(Q[i][t] * K[k][t] for t in range(d)) for k in range(i + 1)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        out.append([sum(e[k] / z * V[k][t] for k in range(i + 1)) for t in range(d)])
    return out


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_mlp_forward_vs_brute_force(act):
    T, h, f = 4, 8, 16
    n_a = 2 if act == "swiglu" else 1
    X, A_s, B_s = rnd(T, h), rnd(h, n_a * f, scale=0.3), rnd(f, h, scale=0.3)
    Hpre, H, Y = omlp.mlp_shard_forward(X, A_s, B_s, act)
    bHpre, bH, bY = bf_mlp_shard_forward(X.tolist(), A_s.tolist(), B_s.tolist(), act)
    assert np.max(np.abs(Hpre - np.array(bHpre))) < 1e-12
    assert np.max(np.abs(H - np.array(bH))) < 1e-12
    assert np.max(np.abs(Y - np.array(bY))) < 1e-12


def test_attention_vs_brute_force():
    batch, seq, heads, d = 2, 5, 2, 4
    h = 6
    X = rnd(batch * seq, h)
    A_s = rnd(h, 3 * heads * d, scale=0.5)
    Bo_s = rnd(heads * d, h, scale=0.5)
    QKV, O, Y = oattn.attn_shard_forward(X, A_s, Bo_s, batch, seq, heads, d)
    bQKV = np.array(bf_matmul(X.tolist(), A_s.tolist()))
    assert np.max(np.abs(QKV - bQKV)) < 1e-12
    Hd = heads * d
    bO = np.zeros((batch * seq, Hd))
    for b in range(batch):
        for j in range(heads):
            rows = range(b * seq, (b + 1) * seq)
            Q = [[bQKV[r][j * d + t] for t in range(d)] for r in rows]
            K = [[bQKV[r][Hd + j * d + t] for t in range(d)] for r in rows]
            V = [[bQKV[r][2 * Hd + j * d + t] for t in range(d)] for r in rows]
            o = bf_causal_attention(Q, K, V, 1.0 / math.sqrt(d))
            for i, r in enumerate(rows):
                bO[r, j * d:(j + 1) * d] = o[i]
    assert np.max(np.abs(O - bO)) < 1e-12
    assert np.max(np.abs(Y - np.array(bf_matmul(bO.tolist(), Bo_s.tolist())))) < 1e-12


# ------------------------------------------------------------------------------------------
# Activations: closed forms and library routines.
# ------------------------------------------------------------------------------------------
def test_activation_closed_forms():
    z = np.zeros(3)
    assert np.all(omlp.gelu_tanh(z) == 0.0)
    assert np.allclose(omlp.gelu_tanh_grad(z), 0.5, atol=0, rtol=0)
    assert np.all(omlp.silu(z) == 0.0)
    # Large |x|: gelu -> x for x >> 0 and -> 0 for x << 0.
    assert abs(omlp.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(omlp.gelu_tanh(np.array([-30.0]))[0]) < 1e-12


def test_gelu_tanh_matches_torch_and_erf_form():
    x = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(omlp.gelu_tanh(x) - ref)) < 1e-13
    from scipy.special import erf

    exact = 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))
    # The tanh form approximates the erf form to well under 1e-3 everywhere.
    assert np.max(np.abs(omlp.gelu_tanh(x) - exact)) < 1e-3


def test_act_grads_match_torch_autograd():
    x = torch.linspace(-6, 6, 1201, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(x, approximate="tanh").sum().backward()
    assert np.max(np.abs(omlp.gelu_tanh_grad(x.detach().numpy()) - x.grad.numpy())) < 1e-12
    g = torch.randn(7, 5, dtype=torch.float64, generator=torch.Generator().manual_seed(3), requires_grad=True)
    u = torch.randn(7, 5, dtype=torch.float64, generator=torch.Generator().manual_seed(4), requires_grad=True)
    dH = torch.randn(7, 5, dtype=torch.float64, generator=torch.Generator().manual_seed(5))
    (torch.nn.functional.silu(g) * u * dH).sum().backward()
    Hpre = np.concatenate([g.detach().numpy(), u.detach().numpy()], axis=1)
    dHpre = omlp.act_backward(Hpre, dH.numpy(), "swiglu")
    assert np.max(np.abs(dHpre[:, :5] - g.grad.numpy())) < 1e-12
    assert np.max(np.abs(dHpre[:, 5:] - u.grad.numpy())) < 1e-12
    assert np.max(np.abs(omlp.act_forward(Hpre, "swiglu")
                         - (torch.nn.functional.silu(g) * u).detach().numpy())) < 1e-12


# ------------------------------------------------------------------------------------------
# Split identities and the shard-sum identity.
# ------------------------------------------------------------------------------------------
SPLITS = [(1, 1), (2, 1), (1, 2), (2, 2), (3, 1), (1, 3), (4, 2), (2, 4)]


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("split", SPLITS)
def test_domino_forward_chunks_equal_unsharded_layer(act, split):
    batch, seq, h, f_s, P = 4, 3, 10, 6, 3
    n_a = 2 if act == "swiglu" else 1
    X = rnd(batch * seq, h)
    A = rnd(h, n_a * P * f_s, scale=0.3)
    B = rnd(P * f_s, h, scale=0.3)
    Y = omlp.domino_mlp_forward(X, A, B, act, P, batch, seq, *split)
    ref = omlp.mlp_forward_unsharded(X, A, B, act)
    assert not np.isnan(Y).any()
    assert np.max(np.abs(Y - ref)) < 1e-12
    # Σ of the per-rank partials computed whole equals the unsharded layer too.
    parts = [omlp.mlp_shard_forward(X, *omlp.mlp_shard_weights(A, B, act, P, s), act)[2] for s in range(P)]
    assert np.max(np.abs(omlp.shard_sum(parts) - ref)) < 1e-12


def test_shard_weights_partition_full_weights():
    h, f_s, P = 5, 4, 3
    A = rnd(h, 2 * P * f_s)
    B = rnd(P * f_s, h)
    gate_cols, up_cols, b_rows = [], [], []
    for s in range(P):
        A_s, B_s = omlp.mlp_shard_weights(A, B, "swiglu", P, s)
        assert A_s.shape == (h, 2 * f_s) and B_s.shape == (f_s, h)
        gate_cols.append(A_s[:, :f_s])
        up_cols.append(A_s[:, f_s:])
        b_rows.append(B_s)
    assert np.array_equal(np.concatenate(gate_cols, 1), A[:, :P * f_s])
    assert np.array_equal(np.concatenate(up_cols, 1), A[:, P * f_s:])
    assert np.array_equal(np.concatenate(b_rows, 0), B)


def test_chunk_ranges_follow_torch_chunk():
    for n, c in [(4, 2), (5, 2), (7, 3), (1, 2), (8, 8), (3, 5)]:
        ours = [b - a for a, b in omlp._chunk_sizes(n, c)]
        theirs = [t.numel() for t in torch.arange(n).chunk(c)]
        assert ours == theirs
    assert omlp.row_chunk_ranges(4, 2048, 2) == [(0, 4096), (4096, 8192)]
    assert omlp.col_chunk_ranges(4096, 2) == [(0, 2048), (2048, 4096)]


def test_shard_sum_order_and_value():
    parts = [np.full((2, 3), float(p)) for p in range(5)]
    assert np.array_equal(omlp.shard_sum(parts), np.full((2, 3), 10.0))


# ------------------------------------------------------------------------------------------
# Backward: finite differences, adjoint identity, chunked == unsplit, torch autograd.
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_backward_finite_differences(act):
    T, h, f = 3, 4, 5
    n_a = 2 if act == "swiglu" else 1
    rng = np.random.default_rng(7)
    X, A_s, B_s = rnd(T, h, rng=rng), rnd(h, n_a * f, scale=0.5, rng=rng), rnd(f, h, scale=0.5, rng=rng)
    dY = rnd(T, h, rng=rng)
    _, dX, dA, dB = omlp.mlp_shard_backward(X, A_s, B_s, dY, act)

    def loss(X_, A_, B_):
        return float(np.sum(dY * omlp.mlp_shard_forward(X_, A_, B_, act)[2]))

    eps = 1e-6
    for M, G, which in [(X, dX, 0), (A_s, dA, 1), (B_s, dB, 2)]:
        num = np.zeros_like(M)
        for idx in np.ndindex(M.shape):
            args_p = [X.copy(), A_s.copy(), B_s.copy()]
            args_m = [X.copy(), A_s.copy(), B_s.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - G)) < 1e-7, which


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_backward_adjoint_identity(act):
    """⟨dY, J·V⟩ = ⟨Jᵀ·dY, V⟩ for a random direction V in X (J = ∂Y_s/∂X)."""
    T, h, f = 6, 5, 7
    n_a = 2 if act == "swiglu" else 1
    X, A_s, B_s = rnd(T, h), rnd(h, n_a * f, scale=0.5), rnd(f, h, scale=0.5)
    dY, V = rnd(T, h), rnd(T, h)
    _, dX, _, _ = omlp.mlp_shard_backward(X, A_s, B_s, dY, act)
    eps = 1e-5
    JV = (omlp.mlp_shard_forward(X + eps * V, A_s, B_s, act)[2]
          - omlp.mlp_shard_forward(X - eps * V, A_s, B_s, act)[2]) / (2 * eps)
    assert abs(np.sum(dY * JV) - np.sum(dX * V)) < 1e-7 * max(1.0, abs(np.sum(dX * V)))


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_backward_matches_torch_autograd(act):
    T, h, f = 5, 6, 4
    n_a = 2 if act == "swiglu" else 1
    X, A_s, B_s, dY = rnd(T, h), rnd(h, n_a * f, scale=0.5), rnd(f, h, scale=0.5), rnd(T, h)
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A_s, B_s))
    Hpre = tX @ tA
    if act == "gelu_tanh":
        H = torch.nn.functional.gelu(Hpre, approximate="tanh")
    else:
        H = torch.nn.functional.silu(Hpre[:, :f]) * Hpre[:, f:]
    Y = H @ tB
    (Y * torch.tensor(dY)).sum().backward()
    _, dX, dA, dB = omlp.mlp_shard_backward(X, A_s, B_s, dY, act)
    assert np.max(np.abs(omlp.mlp_shard_forward(X, A_s, B_s, act)[2] - Y.detach().numpy())) < 1e-12
    assert np.max(np.abs(dX - tX.grad.numpy())) < 1e-12
    assert np.max(np.abs(dA - tA.grad.numpy())) < 1e-12
    assert np.max(np.abs(dB - tB.grad.numpy())) < 1e-12


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("split", SPLITS)
def test_domino_backward_chunks_equal_unsplit(act, split):
    batch, seq, h, f_s, P = 4, 2, 6, 5, 2
    n_a = 2 if act == "swiglu" else 1
    X, dY = rnd(batch * seq, h), rnd(batch * seq, h)
    A, B = rnd(h, n_a * P * f_s, scale=0.4), rnd(P * f_s, h, scale=0.4)
    s = 1
    dX, dA, dB = omlp.domino_mlp_backward(X, A, B, dY, act, P, s, batch, seq, *split)
    assert not np.isnan(dX).any()
    assert np.max(np.abs(dX - omlp.mlp_backward_unsharded(X, A, B, dY, act))) < 1e-12
    parts = [omlp.mlp_shard_backward(X, *omlp.mlp_shard_weights(A, B, act, P, p), dY, act)[1] for p in range(P)]
    assert np.max(np.abs(dX - omlp.shard_sum(parts))) < 1e-12
    _, _, rA, rB = omlp.mlp_shard_backward(X, *omlp.mlp_shard_weights(A, B, act, P, s), dY, act)
    assert np.max(np.abs(dA - rA)) < 1e-12
    assert np.max(np.abs(dB - rB)) < 1e-12


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_sampled_helpers_equal_full(act):
    T, h, f_s, P = 9, 6, 4, 2
    n_a = 2 if act == "swiglu" else 1
    X, dY = rnd(T, h), rnd(T, h)
    A, B = rnd(h, n_a * P * f_s, scale=0.4), rnd(P * f_s, h, scale=0.4)
    rows = np.array([0, 4, 8])
    assert np.max(np.abs(omlp.mlp_y_rows(X[rows], A, B, act) - omlp.mlp_forward_unsharded(X, A, B, act)[rows])) < 1e-12
    assert np.max(np.abs(omlp.mlp_dx_rows(X[rows], dY[rows], A, B, act)
                         - omlp.mlp_backward_unsharded(X, A, B, dY, act)[rows])) < 1e-12
    A_s, B_s = omlp.mlp_shard_weights(A, B, act, P, 0)
    _, _, dA, dB = omlp.mlp_shard_backward(X, A_s, B_s, dY, act)
    cols = np.array([1, 3])
    sA, sB = omlp.mlp_wgrad_slices(X, dY, A_s, B_s, act, cols)
    a_cols = np.concatenate([cols, f_s + cols]) if act == "swiglu" else cols
    assert np.max(np.abs(sA - dA[:, a_cols])) < 1e-12
    assert np.max(np.abs(sB - dB[cols, :])) < 1e-12


# ------------------------------------------------------------------------------------------
# Attention: special cases, library cross-check, head-shard sum.
# ------------------------------------------------------------------------------------------
def test_attention_first_row_and_prefix_means():
    n, d = 9, 4
    Q, K, V = rnd(n, d), rnd(n, d), rnd(n, d)
    O = oattn.causal_attention(Q, K, V, 1 / math.sqrt(d))
    assert np.max(np.abs(O[0] - V[0])) < 1e-15
    O0 = oattn.causal_attention(np.zeros((n, d)), K, V, 1 / math.sqrt(d))
    means = np.cumsum(V, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(O0 - means)) < 1e-13
    # Softmax rows sum to 1: with V = ones the output is all ones.
    O1 = oattn.causal_attention(Q, K, np.ones((n, d)), 0.7)
    assert np.max(np.abs(O1 - 1.0)) < 1e-13


def test_attention_matches_torch_sdpa():
    batch, seq, heads, d, h = 2, 7, 3, 8, 10
    X = rnd(batch * seq, h)
    A = rnd(h, 3 * heads * d, scale=0.4)
    Bo = rnd(heads * d, h, scale=0.4)
    QKV, O, Y = oattn.attn_shard_forward(X, A, Bo, batch, seq, heads, d)
    q, k, v = (torch.from_numpy(QKV[:, i * heads * d:(i + 1) * heads * d]).view(batch, seq, heads, d).transpose(1, 2)
               for i in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    ref = ref.transpose(1, 2).reshape(batch * seq, heads * d).numpy()
    assert np.max(np.abs(O - ref)) < 1e-12


@pytest.mark.parametrize("row_chunks", [1, 2, 4])
def test_attention_head_shards_sum_to_full_mha(row_chunks):
    batch, seq, heads, d, h, P = 4, 5, 4, 3, 7, 2
    X = rnd(batch * seq, h)
    Aqkv = rnd(h, 3 * heads * d, scale=0.4)
    Bo = rnd(heads * d, h, scale=0.4)
    Y = oattn.domino_attn_forward(X, Aqkv, Bo, batch, seq, heads, d, P, row_chunks)
    ref = oattn.attn_forward_unsharded(X, Aqkv, Bo, batch, seq, heads, d)
    assert not np.isnan(Y).any()
    assert np.max(np.abs(Y - ref)) < 1e-12
    # Sampled-row helper equals the full computation.
    b = 2
    rows = np.array([0, 3, 4])
    got = oattn.attn_y_rows(X[b * seq:(b + 1) * seq], Aqkv, Bo, heads, d, rows)
    assert np.max(np.abs(got - ref[b * seq + rows])) < 1e-12


# ------------------------------------------------------------------------------------------
# Attention backward: torch autograd (per head and through the whole shard), finite
# differences, closed forms, the log-sum-exp, chunked == unsplit.
# ------------------------------------------------------------------------------------------
def test_attention_backward_matches_torch_autograd():
    batch, seq, heads, d, h = 2, 6, 2, 4, 5
    scale = 0.37
    X, A, Bo, dY = rnd(batch * seq, h), rnd(h, 3 * heads * d, scale=0.5), rnd(heads * d, h, scale=0.5), rnd(batch * seq, h)
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A, Bo))
    QKV = tX @ tA
    q, k, v = (QKV[:, i * heads * d:(i + 1) * heads * d].reshape(batch, seq, heads, d).transpose(1, 2) for i in range(3))
    q.retain_grad()
    O = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    O2 = O.transpose(1, 2).reshape(batch * seq, heads * d)
    O2.retain_grad()
    Y = O2 @ tB
    (Y * torch.tensor(dY)).sum().backward()
    dO, dQKV, dX, dA, dBo = oattn.attn_shard_backward(X, A, Bo, dY, batch, seq, heads, d, scale)
    assert np.max(np.abs(dO - O2.grad.numpy())) < 1e-12
    assert np.max(np.abs(dX - tX.grad.numpy())) < 1e-12
    assert np.max(np.abs(dA - tA.grad.numpy())) < 1e-12
    assert np.max(np.abs(dBo - tB.grad.numpy())) < 1e-12
    dq = q.grad.transpose(1, 2).reshape(batch * seq, heads * d).numpy()
    assert np.max(np.abs(dQKV[:, :heads * d] - dq)) < 1e-12


def test_attention_backward_finite_differences():
    batch, seq, heads, d, h = 1, 4, 2, 2, 3
    rng = np.random.default_rng(11)
    X, A, Bo, dY = rnd(batch * seq, h, rng=rng), rnd(h, 3 * heads * d, scale=0.7, rng=rng), \
        rnd(heads * d, h, scale=0.7, rng=rng), rnd(batch * seq, h, rng=rng)
    _, _, dX, dA, dBo = oattn.attn_shard_backward(X, A, Bo, dY, batch, seq, heads, d)

    def loss(X_, A_, B_):
        return float(np.sum(dY * oattn.attn_shard_forward(X_, A_, B_, batch, seq, heads, d)[2]))

    eps = 1e-6
    for M, G, which in [(X, dX, 0), (A, dA, 1), (Bo, dBo, 2)]:
        num = np.zeros_like(M)
        for idx in np.ndindex(M.shape):
            args_p = [X.copy(), A.copy(), Bo.copy()]
            args_m = [X.copy(), A.copy(), Bo.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - G)) < 1e-7, which


def test_attention_backward_closed_forms():
    d = 3
    # One token: O = V whatever Q and K, so dV = dO and dQ = dK = 0.
    Q, K, V, dO = rnd(1, d), rnd(1, d), rnd(1, d), rnd(1, d)
    dQ, dK, dV = oattn.causal_attention_backward(Q, K, V, dO, 0.9)
    assert np.max(np.abs(dV - dO)) < 1e-15 and np.max(np.abs(dQ)) < 1e-15 and np.max(np.abs(dK)) < 1e-15
    # Q = 0: row i averages V_0..V_i, so dV_k = Σ_{i ≥ k} dO_i / (i + 1).
    n = 7
    K, V, dO = rnd(n, d), rnd(n, d), rnd(n, d)
    _, _, dV = oattn.causal_attention_backward(np.zeros((n, d)), K, V, dO, 0.5)
    ref = np.array([sum(dO[i] / (i + 1) for i in range(k, n)) for k in range(n)])
    assert np.max(np.abs(dV - ref)) < 1e-13
    # V = ones: O is all ones whatever the scores, so dQ = dK = 0.
    Q = rnd(n, d)
    dQ, dK, _ = oattn.causal_attention_backward(Q, K, np.ones((n, d)), dO, 0.5)
    assert np.max(np.abs(dQ)) < 1e-13 and np.max(np.abs(dK)) < 1e-13


def test_attention_lse():
    from scipy.special import logsumexp
    n, d, scale = 9, 4, 0.6
    Q, K = rnd(n, d), rnd(n, d)
    L = oattn.causal_attention_lse(Q, K, scale)
    ref = np.array([logsumexp(scale * (K[: i + 1] @ Q[i])) for i in range(n)])
    assert np.max(np.abs(L - ref)) < 1e-13
    # exp(S − LSE) over the visible keys is the attention row: it reproduces O.
    V = rnd(n, d)
    O = np.array([np.exp(scale * (K[: i + 1] @ Q[i]) - L[i]) @ V[: i + 1] for i in range(n)])
    assert np.max(np.abs(O - oattn.causal_attention(Q, K, V, scale))) < 1e-13


def test_multi_head_lse_matches_logsumexp_and_sdpa():
    """attn_lse over a multi-head QKV: per (sequence, head), against scipy's logsumexp of
    the scores of the Q and K heads that torch's own head reshape picks out, and the
    softmax it implies against torch's causal scaled-dot-product attention (so the Q and
    K column blocks and every head offset are pinned by a route other than the oracle's
    slicing)."""
    from scipy.special import logsumexp
    batch, seq, heads, d = 3, 6, 3, 4
    scale = 1.0 / math.sqrt(d)
    rng = np.random.default_rng(77)
    QKV = rng.standard_normal((batch * seq, 3 * heads * d))
    # Distinct scales per block so a block mix-up moves the scores a lot.
    QKV[:, heads * d:2 * heads * d] *= 2.0
    QKV[:, 2 * heads * d:] *= 0.3
    L = oattn.attn_lse(QKV, batch, seq, heads, d)
    assert L.shape == (batch * seq, heads)
    q, k, v = (torch.from_numpy(QKV).view(batch, seq, 3, heads, d)[:, :, i].transpose(1, 2) for i in range(3))
    q, k, v = q.numpy(), k.numpy(), v.numpy()  # [batch, heads, seq, d]
    for b in range(batch):
        for j in range(heads):
            ref = np.array([logsumexp(scale * (k[b, j, : i + 1] @ q[b, j, i])) for i in range(seq)])
            assert np.max(np.abs(L[b * seq:(b + 1) * seq, j] - ref)) < 1e-12, (b, j)
    # exp(S − LSE) is the attention row: over the visible keys it sums to one and, applied
    # to V, gives torch's causal attention output.
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()
    for b in range(batch):
        for j in range(heads):
            S = scale * (q[b, j] @ k[b, j].T)
            Pm = np.where(np.tril(np.ones((seq, seq), dtype=bool)), np.exp(S - L[b * seq:(b + 1) * seq, j][:, None]), 0)
            assert np.max(np.abs(Pm.sum(axis=1) - 1.0)) < 1e-12
            assert np.max(np.abs(Pm @ v[b, j] - O[b, j])) < 1e-12


@pytest.mark.parametrize("row_chunks", [1, 2, 4])
def test_domino_attn_backward_chunks_equal_unsplit(row_chunks):
    batch, seq, heads, d, h, P = 4, 5, 4, 3, 7, 2
    X, dY = rnd(batch * seq, h), rnd(batch * seq, h)
    Aqkv, Bo = rnd(h, 3 * heads * d, scale=0.4), rnd(heads * d, h, scale=0.4)
    s = 1
    dX, dA, dBo = oattn.domino_attn_backward(X, Aqkv, Bo, dY, batch, seq, heads, d, P, s, row_chunks)
    assert not np.isnan(dX).any()
    assert np.max(np.abs(dX - oattn.attn_backward_unsharded(X, Aqkv, Bo, dY, batch, seq, heads, d))) < 1e-12
    A_s, Bo_s = oattn.attn_shard_weights(Aqkv, Bo, heads, d, P, s)
    _, _, _, rA, rB = oattn.attn_shard_backward(X, A_s, Bo_s, dY, batch, seq, heads // P, d)
    assert np.max(np.abs(dA - rA)) < 1e-12
    assert np.max(np.abs(dBo - rB)) < 1e-12


# ------------------------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle must make at least one pin fail.
# ------------------------------------------------------------------------------------------
def _pins():
    return [
        lambda: test_gelu_tanh_matches_torch_and_erf_form(),
        lambda: test_act_grads_match_torch_autograd(),
        lambda: test_backward_matches_torch_autograd("gelu_tanh"),
        lambda: test_backward_matches_torch_autograd("swiglu"),
        lambda: test_attention_matches_torch_sdpa(),
        lambda: test_attention_first_row_and_prefix_means(),
        lambda: test_domino_forward_chunks_equal_unsharded_layer("swiglu", (2, 2)),
        lambda: test_domino_backward_chunks_equal_unsplit("swiglu", (1, 2)),
        lambda: test_mlp_forward_vs_brute_force("swiglu"),
        lambda: test_attention_backward_matches_torch_autograd(),
        lambda: test_attention_backward_closed_forms(),
        lambda: test_attention_lse(),
        lambda: test_multi_head_lse_matches_logsumexp_and_sdpa(),
    ]


def _any_pin_fails():
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            return True
    return False


MUTATIONS = {
    "gelu_constant": ("GELU_CUBIC", 0.0447),
    "gelu_grad_dropped_cubic": ("gelu_tanh_grad", lambda x: 0.5 * (1 + np.tanh(omlp.SQRT_2_OVER_PI * (x + 0.044715 * x ** 3)))
                                 + 0.5 * x * (1 - np.tanh(omlp.SQRT_2_OVER_PI * (x + 0.044715 * x ** 3)) ** 2)
                                 * omlp.SQRT_2_OVER_PI),
    "swiglu_gate_up_swapped": ("act_forward", lambda Hpre, act: (
        omlp.silu(Hpre[:, Hpre.shape[1] // 2:]) * Hpre[:, :Hpre.shape[1] // 2]) if act == "swiglu"
        else omlp.gelu_tanh(Hpre)),
    "swiglu_grad_sign": ("act_backward", lambda Hpre, dH, act: np.concatenate([
        dH * Hpre[:, Hpre.shape[1] // 2:] * omlp.sigmoid(Hpre[:, :Hpre.shape[1] // 2])
        * (1 - Hpre[:, :Hpre.shape[1] // 2] * (1 - omlp.sigmoid(Hpre[:, :Hpre.shape[1] // 2]))),
        dH * omlp.silu(Hpre[:, :Hpre.shape[1] // 2])], axis=1) if act == "swiglu"
        else dH * omlp.gelu_tanh_grad(Hpre)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mlp_mistakes_are_caught(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(omlp, attr, value)
    assert _any_pin_fails(), name


def test_planted_attention_mistakes_are_caught(monkeypatch):
    orig = oattn.causal_attention

    def no_mask(Q, K, V, scale):  # mask off by one: the diagonal excluded is impossible for row 0,
        n = Q.shape[0]            # so plant "attends to one future token" instead
        S = (Q @ K.T) * scale
        S = np.where(np.triu(np.ones((n, n), dtype=bool), k=2), -np.inf, S)
        E = np.exp(S - S.max(1, keepdims=True))
        return (E / E.sum(1, keepdims=True)) @ V

    monkeypatch.setattr(oattn, "causal_attention", no_mask)
    assert _any_pin_fails()
    monkeypatch.setattr(oattn, "causal_attention", lambda Q, K, V, scale: orig(Q, K, V, 1.0))
    assert _any_pin_fails()


ATTN_BWD_MUTATIONS = {
    # the row term of the softmax rule dropped
    "no_row_term": lambda Q, K, V, dO, scale: _mut_attn_bwd(Q, K, V, dO, scale, row_term=False),
    # dK from dS instead of its transpose
    "dk_untransposed": lambda Q, K, V, dO, scale: _mut_attn_bwd(Q, K, V, dO, scale, transpose_dk=False),
    # the score scale left out of dQ and dK
    "scale_dropped": lambda Q, K, V, dO, scale: _mut_attn_bwd(Q, K, V, dO, scale, use_scale=False),
}


def _mut_attn_bwd(Q, K, V, dO, scale, row_term=True, transpose_dk=True, use_scale=True):
    n = Q.shape[0]
    S = (Q @ K.T) * scale
    S = np.where(np.triu(np.ones((n, n), dtype=bool), k=1), -np.inf, S)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    Pm = E / E.sum(axis=1, keepdims=True)
    dV = Pm.T @ dO
    dP = dO @ V.T
    dS = Pm * (dP - np.sum(Pm * dP, axis=1, keepdims=True)) if row_term else Pm * dP
    c = scale if use_scale else 1.0
    return c * (dS @ K), c * ((dS.T if transpose_dk else dS) @ Q), dV


@pytest.mark.parametrize("name", sorted(ATTN_BWD_MUTATIONS))
def test_planted_attention_backward_mistakes_are_caught(name, monkeypatch):
    monkeypatch.setattr(oattn, "causal_attention_backward", ATTN_BWD_MUTATIONS[name])
    assert _any_pin_fails(), name


def _mut_attn_lse(QKV, batch, seq, heads, head_dim, scale=None, k_block=1, head_shift=0):
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    Hd = heads * head_dim
    L = np.zeros((batch * seq, heads))
    for b in range(batch):
        r = slice(b * seq, (b + 1) * seq)
        for j in range(heads):
            jq = j
            jk = (j + head_shift) % heads
            Q = QKV[r, jq * head_dim:(jq + 1) * head_dim]
            K = QKV[r, k_block * Hd + jk * head_dim:k_block * Hd + (jk + 1) * head_dim]
            L[r, j] = oattn.causal_attention_lse(Q, K, scale)
    return L


LSE_MUTATIONS = {
    # K read from the V block
    "k_from_v_block": lambda *a, **kw: _mut_attn_lse(*a, k_block=2, **kw),
    # K of the neighbouring head (head offset off by one)
    "head_offset_off_by_one": lambda *a, **kw: _mut_attn_lse(*a, head_shift=1, **kw),
}


@pytest.mark.parametrize("name", sorted(LSE_MUTATIONS))
def test_planted_lse_mistakes_are_caught(name, monkeypatch):
    # The unmutated copy passes the pin; each mutation must fail it.
    monkeypatch.setattr(oattn, "attn_lse", lambda *a, **kw: _mut_attn_lse(*a, **kw))
    assert not _any_pin_fails()
    monkeypatch.setattr(oattn, "attn_lse", LSE_MUTATIONS[name])
    assert _any_pin_fails(), name
