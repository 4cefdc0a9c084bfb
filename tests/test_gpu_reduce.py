"""shard_reduce on the GPU against the oracle's shard sum (fp64)."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, sync, oracle, BF16_TOL, F32_TOL

pytestmark = pytest.mark.gpu


def _run(P, rows, cols, ld_in, ld_out, dtype, seed):
    d = dev()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    parts = [synth.randn((rows, ld_in), seed=seed + p, dtype=dtype).to(d) for p in range(P)]
    out = torch.full((rows, ld_out), float("nan"), dtype=td, device=d)
    D.shard_reduce(out, ld_out, parts, ld_in, rows, cols, D.DOMINO_BF16 if dtype == "bf16" else D.DOMINO_F32)
    sync()
    ref = oracle.shard_sum([f64(p)[:, :cols] for p in parts])
    got = f64(out)
    absum = sum(np.abs(f64(p)[:, :cols]) for p in parts)
    return got, ref, absum, out


@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shard_reduce_matches_oracle(P, dtype):
    rows, cols, ld_in, ld_out = 37, 264, 272, 280
    print(f"shard_reduce P={P} dtype={dtype} rows={rows} cols={cols}", flush=True)
    got, ref, absum, _ = _run(P, rows, cols, ld_in, ld_out, dtype, seed=100)
    check("out", got[:, :cols], ref, BF16_TOL if dtype == "bf16" else F32_TOL)
    # Elementwise bound: fp32 accumulation in order, then one rounding to the dtype.
    unit = 2.0 ** -8 if dtype == "bf16" else 0.0   # bf16 has 8 significant bits: RNE error <= 2^-8 relative
    bound = unit * np.abs(ref) + P * 2.0 ** -23 * absum + 1e-38
    assert np.all(np.abs(got[:, :cols] - ref) <= bound)
    # Padding columns beyond cols stay untouched.
    assert np.isnan(got[:, cols:]).all()


def test_shard_reduce_exact_for_representable_sums():
    # Small integers: every partial sum is exact in fp32 and the result exact in bf16.
    d = dev()
    P, rows, cols = 8, 64, 512
    g = torch.Generator().manual_seed(5)
    parts = [torch.randint(-8, 9, (rows, cols), generator=g).to(torch.bfloat16).to(d) for _ in range(P)]
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=d)
    D.shard_reduce(out, cols, parts, cols, rows, cols, D.DOMINO_BF16)
    sync()
    ref = sum(f64(p) for p in parts)
    assert np.array_equal(f64(out), ref)


def test_shard_reduce_in_place_and_large():
    # out aliases partial 0 (the rank's own buffer); a size with a ragged grid tail.
    d = dev()
    P, rows, cols = 8, 4099, 2560
    parts = [synth.randn((rows, cols), seed=300 + p).to(d) for p in range(P)]
    ref = oracle.shard_sum([f64(p) for p in parts])
    D.shard_reduce(parts[0], cols, parts, cols, rows, cols, D.DOMINO_BF16)
    sync()
    check("in-place", f64(parts[0]), ref, BF16_TOL)


def test_shard_reduce_empty_is_noop():
    d = dev()
    x = torch.full((4, 8), 3.0, dtype=torch.bfloat16, device=d)
    D.shard_reduce(x, 8, [x, x], 8, 0, 8, D.DOMINO_BF16)
    D.shard_reduce(x, 8, [x, x], 8, 4, 0, D.DOMINO_BF16)
    sync()
    assert (f64(x) == 3.0).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shard_reduce_large_matches_small_launches(dtype):
    # At least 2^25 elements: the launch takes the buffer-load kernel (one 32-bit offset per
    # group shared by the partials); a slab of the same rows reduced on its own (below that
    # size) takes the 64-bit kernel. Both sum in the same order: bit-identical. Sampled rows
    # are also checked against the oracle. Ragged rows, padded leading dimensions.
    d = dev()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    P, rows, cols, ld_in, ld_out = 8, 8195, 4096, 4104, 4112
    print(f"shard_reduce large P={P} dtype={dtype} rows={rows} cols={cols}", flush=True)
    parts = [synth.randn((rows, ld_in), seed=700 + p, dtype=dtype).to(d) for p in range(P)]
    out = torch.full((rows, ld_out), float("nan"), dtype=td, device=d)
    code = D.DOMINO_BF16 if dtype == "bf16" else D.DOMINO_F32
    D.shard_reduce(out, ld_out, parts, ld_in, rows, cols, code)
    r0, n = 4001, 1000
    slab = torch.full((n, ld_out), float("nan"), dtype=td, device=d)
    D.shard_reduce(slab, ld_out, [p[r0:] for p in parts], ld_in, n, cols, code)
    sync()
    assert torch.equal(out[r0:r0 + n, :cols].view(torch.int16 if dtype == "bf16" else torch.int32),
                       slab[:, :cols].view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.isnan(out[:, cols:]).all()
    sample = [0, 1, 4095, 8194]
    ref = oracle.shard_sum([f64(p[sample])[:, :cols] for p in parts])
    check("large (sampled rows)", f64(out[sample])[:, :cols], ref, BF16_TOL if dtype == "bf16" else F32_TOL)
