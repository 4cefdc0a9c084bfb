"""The small-kernel group between sublayers and the whole Domino transformer layer, in numpy
float64 (oracle; tests only).

The layer is the pre-LayerNorm transformer block of the deep-dive ("前向：多个计算片段轮转重叠
AllReduce" and the DominoTransformerLayer excerpt under "μ-batch 流水"): LayerNorm, the
attention (tensor-parallel, its partials all-reduced), dropout and the residual add,
LayerNorm, the MLP (tensor-parallel, all-reduced), dropout and the residual add. The pages
name the small kernels (Dropout, Residual, LayerNorm) without formulas; they are written
here from their usual definitions:

  LayerNorm over the hidden dimension of one row: mean μ, biased variance σ², eps inside
  the root, x̂ = (x − μ)/√(σ² + eps), out = x̂·γ + β;
  dropout with a given keep mask and drop probability p: keep·y/(1 − p) (inverted dropout);
  the residual group: r_out = r + dropout(y + bias), then LayerNorm(r_out).

The keep masks are inputs (drawn by the seeded generators), bit-packed: element j of a row
is bit j % 32 of 32-bit word j // 32 of that row.
"""
from __future__ import annotations

import numpy as np

import math

from .attention import _mha, _mha_backward
from .mlp import act_backward, act_forward

LN_EPS = 1e-5


def unpack_keep(keep_words, hidden: int) -> np.ndarray:
    """Bit-packed keep mask [rows, ceil(hidden/32)] (uint32 or int32 words) -> bool [rows, hidden]."""
    w = np.asarray(keep_words)
    w = w.view(np.uint32) if w.dtype == np.int32 else w.astype(np.uint32)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint32)[None, None, :]) & np.uint32(1)
    return bits.reshape(w.shape[0], -1)[:, :hidden].astype(bool)


def dropout(y: np.ndarray, keep: np.ndarray | None, p: float) -> np.ndarray:
    """Inverted dropout with a given keep mask; keep None means no dropout."""
    if keep is None:
        return y
    return np.where(keep, y / (1.0 - p), 0.0)


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = LN_EPS):
    """Row-wise LayerNorm; returns (out, mean, rstd) with rstd = 1/√(σ² + eps)."""
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean[:, None]) * rstd[:, None]
    return xhat * gamma[None, :] + beta[None, :], mean, rstd


def layer_norm_backward(dout: np.ndarray, x: np.ndarray, gamma: np.ndarray, eps: float = LN_EPS):
    """Gradients of LayerNorm: (dx, dgamma, dbeta). With g = dout·γ and n the row length,
    dx = rstd·(g − mean(g) − x̂·mean(g·x̂)) (the chain rule through μ and σ²)."""
    n = x.shape[1]
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    g = dout * gamma[None, :]
    dx = rstd * (g - g.sum(axis=1, keepdims=True) / n - xhat * (g * xhat).sum(axis=1, keepdims=True) / n)
    return dx, (dout * xhat).sum(axis=0), dout.sum(axis=0)


def resid_group_forward(resid, y, bias, keep, p, gamma, beta, eps: float = LN_EPS):
    """r_out = resid + dropout(y + bias); ln = LayerNorm(r_out) (None when gamma is None).
    y None: r_out = resid. Returns (r_out, ln, mean, rstd)."""
    r_out = resid.copy()
    if y is not None:
        z = y + (bias[None, :] if bias is not None else 0.0)
        r_out = resid + dropout(z, keep, p)
    if gamma is None:
        return r_out, None, None, None
    ln, mean, rstd = layer_norm(r_out, gamma, beta, eps)
    return r_out, ln, mean, rstd


def resid_group_backward(d_ln, d_res, r_out, keep, p, gamma, eps: float = LN_EPS):
    """Backward of resid_group_forward. d_ln: gradient of the LayerNorm output (None: no
    LayerNorm term); d_res: gradient reaching r_out from later residual adds (None: zero).
    Returns (d_resid, d_y, dgamma, dbeta, dbias): d_resid is the gradient of r_out (and of
    the residual input), d_y = dropout'(d_resid) the gradient of y (and of the bias)."""
    d = np.zeros_like(r_out) if d_res is None else d_res.copy()
    dgamma = dbeta = None
    if d_ln is not None:
        dx, dgamma, dbeta = layer_norm_backward(d_ln, r_out, gamma, eps)
        d = d + dx
    d_y = dropout(d, keep, p)
    return d, d_y, dgamma, dbeta, d_y.sum(axis=0)


# ----------------------------------------------------------------------------------------
# The whole pre-LayerNorm layer with full weights (what the Domino schedule over the
# tensor-parallel shards must equal), and a stack of such layers.
# Parameters per layer: ln1_g, ln1_b, Aqkv, bqkv, Bo, bo, ln2_g, ln2_b, A, b1, B, b2 (the
# biases may be absent or None: no bias); keep masks keep1 (after the attention) and keep2
# (after the MLP). The column-parallel biases (bqkv, b1) are added to the product before
# the attention / activation; the row-parallel ones (bo, b2) after the sum over ranks.
# ----------------------------------------------------------------------------------------
def _bias(b):
    return 0.0 if b is None else b[None, :]


def attention_sublayer(a, Aqkv, bqkv, Bo, batch, seq, heads, head_dim):
    """Attn(a) = MHA(a·Aqkv + bqkv)·Bo with all heads; returns (y, QKV)."""
    QKV = a @ Aqkv + _bias(bqkv)
    return _mha(QKV, batch, seq, heads, head_dim, 1.0 / math.sqrt(head_dim)) @ Bo, QKV


def attention_sublayer_backward(a, Aqkv, bqkv, Bo, dy, batch, seq, heads, head_dim):
    """(da, dbqkv) of attention_sublayer given dy."""
    _, QKV = attention_sublayer(a, Aqkv, bqkv, Bo, batch, seq, heads, head_dim)
    dQKV = _mha_backward(QKV, dy @ Bo.T, batch, seq, heads, head_dim, 1.0 / math.sqrt(head_dim))
    return dQKV @ Aqkv.T, dQKV.sum(axis=0)


def mlp_sublayer(m, A, b1, B, act):
    """MLP(m) = act(m·A + b1)·B."""
    return act_forward(m @ A + _bias(b1), act) @ B


def mlp_sublayer_backward(m, A, b1, B, dy, act):
    """(dm, db1) of mlp_sublayer given dy."""
    Hpre = m @ A + _bias(b1)
    dHpre = act_backward(Hpre, dy @ B.T, act)
    return dHpre @ A.T, dHpre.sum(axis=0)


def layer_forward(x, prm, keep1, keep2, p, batch, seq, heads_full, head_dim, act, eps: float = LN_EPS):
    """Returns (out, saved): out = h + dropout(MLP(LN2(h)) + b2) with
    h = x + dropout(Attn(LN1(x)) + bo); saved holds a = LN1(x), h, m = LN2(h), the
    sublayer outputs ya, ym and the LayerNorm statistics."""
    a, mu1, rs1 = layer_norm(x, prm["ln1_g"], prm["ln1_b"], eps)
    ya = attention_sublayer(a, prm["Aqkv"], prm.get("bqkv"), prm["Bo"], batch, seq, heads_full, head_dim)[0]
    h, m, mu2, rs2 = resid_group_forward(x, ya, prm.get("bo"), keep1, p, prm["ln2_g"], prm["ln2_b"], eps)
    ym = mlp_sublayer(m, prm["A"], prm.get("b1"), prm["B"], act)
    out = resid_group_forward(h, ym, prm.get("b2"), keep2, p, None, None)[0]
    return out, dict(a=a, ya=ya, h=h, m=m, ym=ym, mean1=mu1, rstd1=rs1, mean2=mu2, rstd2=rs2)


def layer_backward(x, prm, keep1, keep2, p, d_out, batch, seq, heads_full, head_dim, act, eps: float = LN_EPS):
    """Backward of layer_forward, in reverse order of its steps: the closing residual group,
    the MLP, the middle group (LayerNorm 2, dropout, residual), the attention, LayerNorm 1
    and the residual. Returns (dx, grads, saved) with grads holding the LayerNorm and bias
    gradients and the sublayer output gradients d_ym and d_ya (the dY of the MLP and of
    the attention, from which each rank's weight gradients follow)."""
    _, s = layer_forward(x, prm, keep1, keep2, p, batch, seq, heads_full, head_dim, act, eps)
    d_h, d_ym, _, _, db2 = resid_group_backward(None, d_out, s["h"], keep2, p, None, eps)
    dm, db1 = mlp_sublayer_backward(s["m"], prm["A"], prm.get("b1"), prm["B"], d_ym, act)
    d_h, d_ya, dg2, dbt2, dbo = resid_group_backward(dm, d_h, s["h"], keep1, p, prm["ln2_g"], eps)
    da, dbqkv = attention_sublayer_backward(s["a"], prm["Aqkv"], prm.get("bqkv"), prm["Bo"], d_ya, batch, seq,
                                            heads_full, head_dim)
    dx, _, dg1, dbt1, _ = resid_group_backward(da, d_h, x, None, p, prm["ln1_g"], eps)
    grads = dict(ln1_g=dg1, ln1_b=dbt1, ln2_g=dg2, ln2_b=dbt2, bo=dbo, b2=db2, bqkv=dbqkv, b1=db1, d_ym=d_ym,
                 d_ya=d_ya, dm=dm, da=da)
    return dx, grads, s


def stack_forward(x, layers, keeps, p, batch, seq, heads_full, head_dim, act, eps: float = LN_EPS):
    """A stack of layers; keeps[l] = (keep1, keep2) of layer l. Returns (out, inputs) with
    inputs[l] the residual stream entering layer l."""
    inputs = []
    for prm, (k1, k2) in zip(layers, keeps):
        inputs.append(x)
        x = layer_forward(x, prm, k1, k2, p, batch, seq, heads_full, head_dim, act, eps)[0]
    return x, inputs


def stack_backward(x, layers, keeps, p, d_out, batch, seq, heads_full, head_dim, act, eps: float = LN_EPS):
    """Backward of stack_forward: dx and each layer's (grads, saved), last layer first."""
    _, inputs = stack_forward(x, layers, keeps, p, batch, seq, heads_full, head_dim, act, eps)
    per = [None] * len(layers)
    d = d_out
    for l in range(len(layers) - 1, -1, -1):
        d, g, s = layer_backward(inputs[l], layers[l], keeps[l][0], keeps[l][1], p, d, batch, seq, heads_full,
                                 head_dim, act, eps)
        per[l] = (g, s)
    return d, per
