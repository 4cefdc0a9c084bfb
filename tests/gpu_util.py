"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

import oracle
import tensor_transformer_block_domino_amd as D

BF16_TOL = 1e-2   # normwise relative error bar for bf16 storage with fp32 accumulation
F32_TOL = 1e-5    # the same bar for the fp32 layer
# Per-row bar of the gradients that pass through the attention's softmax backward (dQ, dK,
# and what is computed from them: dQKV, dA_qkv_s, the attention's dX). There each score
# gradient is P·(dP − Δ), and Δ, a row's Σ P·dP, is formed from the bf16 O and dO; in rows
# with few visible keys dP − Δ is small next to its terms, so its rounding error, relative
# to that row's result, exceeds the tensor's normwise error (up to 1.5e-2 measured against
# ~4e-3 normwise). 3e-2 still fails a row with one wrong element among its 256 or more.
ATTN_BWD_ROW_TOL = 3e-2


def dev():
    D.load()
    return torch.device("cuda:0")


def f64(t) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def relerr(got, ref) -> float:
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values in GPU output"
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def row_relerr(got, ref) -> tuple:
    """Worst row of the normwise relative error: ‖g_r − r_r‖ / max(‖r_r‖, 0.1·rms row norm)
    over the rows of the tensor (its first axis; each element of a 1-D tensor is a row).
    A localized error (one wrong column band, a bad ragged tail, one wrong element in a
    row of ~100 or more) moves its own row by far more than the tolerance even when the
    whole tensor's Frobenius norm hides it. The floor keeps rows whose exact value is
    near zero from turning rounding noise into a large ratio."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0, -1
    g2 = got.reshape(got.shape[0], -1)
    r2 = ref.reshape(ref.shape[0], -1)
    rn = np.linalg.norm(r2, axis=1)
    floor = 0.1 * float(np.sqrt(np.mean(rn ** 2)))
    den = np.maximum(rn, max(floor, 1e-300))
    e = np.linalg.norm(g2 - r2, axis=1) / den
    worst = int(np.argmax(e))
    return float(e[worst]), worst


def check(name, got, ref, tol, row_tol=None):
    """Normwise relative error of the whole tensor within tol and, for a matrix, that of
    every row within row_tol (default tol; row_relerr). A vector (bias, LayerNorm and
    per-row statistics) gets the normwise bound alone: its elements are sums whose own
    relative error is not bounded by it, while one wrong element among a few thousand
    already moves the normwise error past the bar."""
    got, ref = np.asarray(got), np.asarray(ref)
    e = relerr(got, ref)
    rows = got.ndim >= 2
    row_tol = tol if row_tol is None else row_tol
    msg = f"  {name}: normwise rel err {e:.3e}"
    if rows:
        er, worst = row_relerr(got, ref)
        msg += f", worst row {er:.3e} (row {worst}, tol {row_tol:g})"
    print(msg + f" (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: {e:.3e} > {tol:g}"
    if rows:
        assert er <= row_tol, f"{name}: row {worst} has normwise rel err {er:.3e} > {row_tol:g}"
    return e


def poison(*tensors):
    """Fill outputs with NaN so a read-before-write or an unwritten element shows."""
    for t in tensors:
        t.fill_(float("nan"))


def sync():
    torch.cuda.synchronize()


__all__ = ["oracle", "D", "np", "torch", "dev", "f64", "relerr", "row_relerr", "check", "poison", "sync", "BF16_TOL", "F32_TOL", "ATTN_BWD_ROW_TOL"]
