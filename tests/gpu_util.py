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


def check(name, got, ref, tol):
    e = relerr(got, ref)
    print(f"  {name}: normwise rel err {e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: {e:.3e} > {tol:g}"
    return e


def poison(*tensors):
    """Fill outputs with NaN so a read-before-write or an unwritten element shows."""
    for t in tensors:
        t.fill_(float("nan"))


def sync():
    torch.cuda.synchronize()


__all__ = ["oracle", "D", "np", "torch", "dev", "f64", "relerr", "check", "poison", "sync", "BF16_TOL", "F32_TOL"]
