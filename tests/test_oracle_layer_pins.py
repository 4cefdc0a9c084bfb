"""Pins of the oracle's small-kernel group and whole layer against things other than itself
(CPU only).

  * torch's fp64 LayerNorm (torch.nn.functional.layer_norm) and torch autograd through
    LayerNorm, dropout, the residual adds, causal scaled-dot-product attention and the MLP,
    for one layer and for a stack of two;
  * central finite differences of ⟨dY, out⟩ through the group;
  * closed forms: a constant row normalises to β; x̂ has mean 0 and variance σ²/(σ² + eps);
    keep-all dropout scales by 1/(1 − p), keep-none gives zero; hand-made bit words for
    the mask layout;
  * planted mistakes (unbiased variance, eps outside the root, dropout without its scale,
    dropped LayerNorm-backward terms, a lost residual gradient) each fail a pin.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import layer as olayer

RNG = np.random.default_rng(2024)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def t64(a):
    return torch.tensor(np.asarray(a), dtype=torch.float64)


def rand_keep(rows, h, p):
    return RNG.random((rows, h)) >= p


# ------------------------------------------------------------------------------------
# LayerNorm and dropout
# ------------------------------------------------------------------------------------
def test_layer_norm_matches_torch():
    x, g, b = rnd(7, 48) * 3 + 1.5, 1 + rnd(48, scale=0.2), rnd(48, scale=0.3)
    out, mean, rstd = oracle.layer_norm(x, g, b)
    ref = F.layer_norm(t64(x), (48,), t64(g), t64(b), eps=1e-5).numpy()
    assert rel(out, ref) < 1e-13
    assert np.allclose(mean, x.mean(axis=1)) and np.allclose(rstd, 1 / np.sqrt(x.var(axis=1) + 1e-5))


def test_layer_norm_closed_forms():
    g, b = 1 + rnd(16, scale=0.2), rnd(16)
    const = np.full((3, 16), 2.5)
    out, _, _ = oracle.layer_norm(const, g, b)
    assert np.allclose(out, np.broadcast_to(b, out.shape), atol=1e-12)
    x = rnd(5, 16) * 2
    xhat, _, _ = oracle.layer_norm(x, np.ones(16), np.zeros(16))
    var = x.var(axis=1)
    assert np.allclose(xhat.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(xhat.var(axis=1), var / (var + 1e-5), rtol=1e-12)


def test_layer_norm_backward_matches_torch_autograd():
    x, g, b, dy = rnd(6, 40) * 2 + 0.5, 1 + rnd(40, scale=0.2), rnd(40, scale=0.3), rnd(6, 40)
    xt, gt, bt = (t64(v).requires_grad_() for v in (x, g, b))
    F.layer_norm(xt, (40,), gt, bt, eps=1e-5).backward(t64(dy))
    dx, dg, db = oracle.layer_norm_backward(dy, x, g)
    assert rel(dx, xt.grad.numpy()) < 1e-12
    assert rel(dg, gt.grad.numpy()) < 1e-12 and rel(db, bt.grad.numpy()) < 1e-12


def test_keep_mask_bit_layout():
    # word 0 = 0b101: elements 0 and 2; word 1 = −2³¹ (sign bit only): element 63.
    words = np.array([[5, -(2 ** 31)]], dtype=np.int32)
    k = oracle.unpack_keep(words, 64)
    assert k.shape == (1, 64) and set(np.flatnonzero(k[0])) == {0, 2, 63}
    assert oracle.unpack_keep(words, 40).shape == (1, 40)


def test_dropout_special_cases():
    y = rnd(4, 10)
    assert np.allclose(oracle.dropout(y, np.ones((4, 10), bool), 0.3), y / 0.7)
    assert np.all(oracle.dropout(y, np.zeros((4, 10), bool), 0.3) == 0)
    assert np.array_equal(oracle.dropout(y, None, 0.3), y)


# ------------------------------------------------------------------------------------
# The group: r_out = resid + dropout(y + bias); LayerNorm(r_out)
# ------------------------------------------------------------------------------------
def _torch_group(resid, y, bias, keep, p, g, b):
    z = y + bias
    r = resid + torch.where(t64(keep).bool(), z / (1 - p), torch.zeros_like(z))
    return r, F.layer_norm(r, (r.shape[1],), g, b, eps=1e-5)


def test_group_forward_backward_match_torch_autograd():
    rows, h, p = 5, 24, 0.25
    resid, y, bias = rnd(rows, h), rnd(rows, h), rnd(h, scale=0.1)
    g, b, keep = 1 + rnd(h, scale=0.2), rnd(h, scale=0.2), rand_keep(rows, h, p)
    d_ln, d_res = rnd(rows, h), rnd(rows, h)
    r_o, ln_o, _, _ = oracle.resid_group_forward(resid, y, bias, keep, p, g, b)
    ts = [t64(v).requires_grad_() for v in (resid, y, bias, g, b)]
    r_t, ln_t = _torch_group(ts[0], ts[1], ts[2], keep, p, ts[3], ts[4])
    assert rel(r_o, r_t.detach().numpy()) < 1e-14 and rel(ln_o, ln_t.detach().numpy()) < 1e-13
    ((r_t * t64(d_res)).sum() + (ln_t * t64(d_ln)).sum()).backward()
    d_resid, d_y, dg, db, dbias = oracle.resid_group_backward(d_ln, d_res, r_o, keep, p, g)
    assert rel(d_resid, ts[0].grad.numpy()) < 1e-12
    assert rel(d_y, ts[1].grad.numpy()) < 1e-12 and rel(dbias, ts[2].grad.numpy()) < 1e-12
    assert rel(dg, ts[3].grad.numpy()) < 1e-12 and rel(db, ts[4].grad.numpy()) < 1e-12


def test_group_backward_finite_differences():
    rows, h, p, eps = 3, 12, 0.2, 1e-6
    resid, y, g, b = rnd(rows, h), rnd(rows, h), 1 + rnd(h, scale=0.2), rnd(h, scale=0.2)
    keep, d_ln, d_res = rand_keep(rows, h, p), rnd(rows, h), rnd(rows, h)

    def loss(rs, yy):
        r, ln, _, _ = oracle.resid_group_forward(rs, yy, None, keep, p, g, b)
        return float((r * d_res).sum() + (ln * d_ln).sum())

    r_o = oracle.resid_group_forward(resid, y, None, keep, p, g, b)[0]
    d_resid, d_y = oracle.resid_group_backward(d_ln, d_res, r_o, keep, p, g)[:2]
    for (i, j) in [(0, 0), (1, 5), (2, 11)]:
        e = np.zeros_like(resid)
        e[i, j] = eps
        fd_r = (loss(resid + e, y) - loss(resid - e, y)) / (2 * eps)
        fd_y = (loss(resid, y + e) - loss(resid, y - e)) / (2 * eps)
        assert abs(fd_r - d_resid[i, j]) < 1e-6 * max(1, abs(fd_r))
        assert abs(fd_y - d_y[i, j]) < 1e-6 * max(1, abs(fd_y))


# ------------------------------------------------------------------------------------
# The whole layer and a stack, against torch autograd of the same definitions
# ------------------------------------------------------------------------------------
def _params(h, heads, d, f, act):
    n_a = 2 if act == "swiglu" else 1
    return dict(ln1_g=1 + rnd(h, scale=0.2), ln1_b=rnd(h, scale=0.2), Aqkv=rnd(h, 3 * heads * d, scale=0.3),
                Bo=rnd(heads * d, h, scale=0.3), ln2_g=1 + rnd(h, scale=0.2), ln2_b=rnd(h, scale=0.2),
                A=rnd(h, n_a * f, scale=0.3), B=rnd(f, h, scale=0.3))


def _torch_layer(x, prm, k1, k2, p, batch, seq, heads, d, act):
    h = x.shape[1]
    a = F.layer_norm(x, (h,), prm["ln1_g"], prm["ln1_b"], eps=1e-5)
    qkv = a @ prm["Aqkv"] + (prm["bqkv"] if "bqkv" in prm else 0.0)
    hd = heads * d

    def split(t):
        return t.reshape(batch, seq, heads, d).permute(0, 2, 1, 3)

    q, k, v = split(qkv[:, :hd]), split(qkv[:, hd:2 * hd]), split(qkv[:, 2 * hd:])
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    ya = o.permute(0, 2, 1, 3).reshape(batch * seq, hd) @ prm["Bo"]
    ya = ya + (prm["bo"] if "bo" in prm else 0.0)
    hh = x + torch.where(t64(k1).bool(), ya / (1 - p), torch.zeros_like(ya))
    m = F.layer_norm(hh, (h,), prm["ln2_g"], prm["ln2_b"], eps=1e-5)
    hp = m @ prm["A"] + (prm["b1"] if "b1" in prm else 0.0)
    if act == "swiglu":
        f = hp.shape[1] // 2
        hmid = F.silu(hp[:, :f]) * hp[:, f:]
    else:
        hmid = F.gelu(hp, approximate="tanh")
    ym = hmid @ prm["B"] + (prm["b2"] if "b2" in prm else 0.0)
    return hh + torch.where(t64(k2).bool(), ym / (1 - p), torch.zeros_like(ym))


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_layer_matches_torch_autograd(act):
    batch, seq, heads, d, h, f, p = 2, 5, 2, 4, 16, 12, 0.2
    T = batch * seq
    x, dy = rnd(T, h), rnd(T, h)
    prm = _params(h, heads, d, f, act)
    k1, k2 = rand_keep(T, h, p), rand_keep(T, h, p)
    out, _ = oracle.layer_forward(x, prm, k1, k2, p, batch, seq, heads, d, act)
    tp = {k: t64(v).requires_grad_() for k, v in prm.items()}
    xt = t64(x).requires_grad_()
    ref = _torch_layer(xt, tp, k1, k2, p, batch, seq, heads, d, act)
    assert rel(out, ref.detach().numpy()) < 1e-12
    ref.backward(t64(dy))
    dx, grads, _ = oracle.layer_backward(x, prm, k1, k2, p, dy, batch, seq, heads, d, act)
    assert rel(dx, xt.grad.numpy()) < 1e-11
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        assert rel(grads[k], tp[k].grad.numpy()) < 1e-11, k


def test_layer_with_biases_matches_torch_autograd():
    batch, seq, heads, d, h, f, p, act = 2, 4, 2, 4, 16, 10, 0.2, "swiglu"
    T = batch * seq
    x, dy = rnd(T, h), rnd(T, h)
    prm = _params(h, heads, d, f, act)
    prm.update(bqkv=rnd(3 * heads * d, scale=0.3), bo=rnd(h, scale=0.3), b1=rnd(2 * f, scale=0.3),
               b2=rnd(h, scale=0.3))
    k1, k2 = rand_keep(T, h, p), rand_keep(T, h, p)
    out, _ = oracle.layer_forward(x, prm, k1, k2, p, batch, seq, heads, d, act)
    tp = {k: t64(v).requires_grad_() for k, v in prm.items()}
    xt = t64(x).requires_grad_()
    ref = _torch_layer(xt, tp, k1, k2, p, batch, seq, heads, d, act)
    assert rel(out, ref.detach().numpy()) < 1e-12
    ref.backward(t64(dy))
    dx, grads, _ = oracle.layer_backward(x, prm, k1, k2, p, dy, batch, seq, heads, d, act)
    assert rel(dx, xt.grad.numpy()) < 1e-11
    for k in ("bqkv", "bo", "b1", "b2", "ln1_g", "ln2_b"):
        assert rel(grads[k], tp[k].grad.numpy()) < 1e-11, k


def test_stack_matches_torch_autograd():
    batch, seq, heads, d, h, f, p, act = 1, 6, 2, 4, 16, 8, 0.1, "gelu_tanh"
    T = batch * seq
    x, dy = rnd(T, h), rnd(T, h)
    layers = [_params(h, heads, d, f, act) for _ in range(2)]
    keeps = [(rand_keep(T, h, p), rand_keep(T, h, p)) for _ in range(2)]
    out, inputs = oracle.stack_forward(x, layers, keeps, p, batch, seq, heads, d, act)
    xt = t64(x).requires_grad_()
    tps = [{k: t64(v).requires_grad_() for k, v in prm.items()} for prm in layers]
    y = xt
    for tp, (k1, k2) in zip(tps, keeps):
        y = _torch_layer(y, tp, k1, k2, p, batch, seq, heads, d, act)
    assert rel(out, y.detach().numpy()) < 1e-12 and rel(inputs[0], x) == 0
    y.backward(t64(dy))
    dx, per = oracle.stack_backward(x, layers, keeps, p, dy, batch, seq, heads, d, act)
    assert rel(dx, xt.grad.numpy()) < 1e-11
    for l in range(2):
        assert rel(per[l][0]["ln1_g"], tps[l]["ln1_g"].grad.numpy()) < 1e-11


# ------------------------------------------------------------------------------------
# Planted mistakes
# ------------------------------------------------------------------------------------
def _unbiased_ln(x, gamma, beta, eps=olayer.LN_EPS):
    mean = x.mean(axis=1)
    var = x.var(axis=1, ddof=1)
    rstd = 1 / np.sqrt(var + eps)
    return ((x - mean[:, None]) * rstd[:, None]) * gamma + beta, mean, rstd


def _eps_outside_ln(x, gamma, beta, eps=olayer.LN_EPS):
    mean = x.mean(axis=1)
    rstd = 1 / (np.sqrt(x.var(axis=1)) + eps)
    return ((x - mean[:, None]) * rstd[:, None]) * gamma + beta, mean, rstd


def _ln_bwd_no_mean_term(dout, x, gamma, eps=olayer.LN_EPS):
    mean, rstd = x.mean(axis=1, keepdims=True), 1 / np.sqrt(x.var(axis=1, keepdims=True) + eps)
    xhat, g = (x - mean) * rstd, dout * gamma
    dx = rstd * (g - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, (dout * xhat).sum(axis=0), dout.sum(axis=0)


def _ln_bwd_no_xhat_term(dout, x, gamma, eps=olayer.LN_EPS):
    mean, rstd = x.mean(axis=1, keepdims=True), 1 / np.sqrt(x.var(axis=1, keepdims=True) + eps)
    xhat, g = (x - mean) * rstd, dout * gamma
    dx = rstd * (g - g.mean(axis=1, keepdims=True))
    return dx, (dout * xhat).sum(axis=0), dout.sum(axis=0)


def _group_bwd_lost_residual(d_ln, d_res, r_out, keep, p, gamma, eps=olayer.LN_EPS):
    d = np.zeros_like(r_out)
    dg = db = None
    if d_ln is not None:
        dx, dg, db = olayer.layer_norm_backward(d_ln, r_out, gamma, eps)
        d = d + dx
    d_y = olayer.dropout(d, keep, p)
    return d, d_y, dg, db, d_y.sum(axis=0)


LAYER_MUTATIONS = {
    "unbiased_variance": ("layer_norm", _unbiased_ln),
    "eps_outside_root": ("layer_norm", _eps_outside_ln),
    "dropout_unscaled": ("dropout", lambda y, keep, p: y if keep is None else np.where(keep, y, 0.0)),
    "ln_bwd_no_mean_term": ("layer_norm_backward", _ln_bwd_no_mean_term),
    "ln_bwd_no_xhat_term": ("layer_norm_backward", _ln_bwd_no_xhat_term),
    "lost_residual_gradient": ("resid_group_backward", _group_bwd_lost_residual),
}


def _layer_pins():
    return [test_layer_norm_matches_torch, test_layer_norm_closed_forms, test_layer_norm_backward_matches_torch_autograd,
            test_dropout_special_cases, test_group_forward_backward_match_torch_autograd,
            test_group_backward_finite_differences, lambda: test_layer_matches_torch_autograd("gelu_tanh"),
            test_layer_with_biases_matches_torch_autograd,
            test_stack_matches_torch_autograd]


@pytest.mark.parametrize("name", sorted(LAYER_MUTATIONS))
def test_planted_layer_mistakes_are_caught(name, monkeypatch):
    attr, value = LAYER_MUTATIONS[name]
    monkeypatch.setattr(olayer, attr, value)
    monkeypatch.setattr(oracle, attr, value)
    failed = 0
    for pin in _layer_pins():
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught the planted mistake {name}"
