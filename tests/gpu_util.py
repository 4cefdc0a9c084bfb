"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

import oracle
import tensor_transformer_block_domino_amd as D

BF16_TOL = 1e-2   # normwise relative error bar for bf16 storage with fp32 accumulation
F32_TOL = 1e-5    # the same bar for the fp32 layer


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


def check(name, got, ref, tol, rows=True):
    """Normwise relative error of the whole tensor within tol, and (rows=True) of every row
    within tol as well (row_relerr)."""
    e = relerr(got, ref)
    msg = f"  {name}: normwise rel err {e:.3e}"
    if rows:
        er, worst = row_relerr(got, ref)
        msg += f", worst row {er:.3e} (row {worst})"
    print(msg + f" (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: {e:.3e} > {tol:g}"
    if rows:
        assert er <= tol, f"{name}: row {worst} has normwise rel err {er:.3e} > {tol:g}"
    return e


def poison(*tensors):
    """Fill outputs with NaN so a read-before-write or an unwritten element shows."""
    for t in tensors:
        t.fill_(float("nan"))


def sync():
    torch.cuda.synchronize()


__all__ = ["oracle", "D", "np", "torch", "dev", "f64", "relerr", "row_relerr", "check", "poison", "sync", "BF16_TOL", "F32_TOL"]
