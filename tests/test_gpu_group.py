"""The dropout + residual + LayerNorm group and its backward against the fp64 oracle, through
the C ABI: widths with ragged chunk counts (h/8 not a multiple of 64 or 256), the largest
width (8192), one row, every optional input left out in turn, in-place use, repeatability
and accumulation of the parameter gradients."""
import pytest

import synth
from gpu_util import D, np, torch, dev, f64, check, poison, sync, oracle, BF16_TOL

pytestmark = pytest.mark.gpu

SHAPES = [(37, 64), (130, 264), (64, 2560), (33, 4096), (17, 5120), (5, 8192), (1, 8), (300, 1032)]
VARIANTS = ["full", "no_bias", "no_dropout", "ln_only", "no_ln"]


def run_group(rows, h, variant, p=0.1, seed=7, inplace=False):
    gi = synth.group_inputs(rows, h, seed=seed, p=p)
    d = dev()
    t = {k: v.to(d) for k, v in gi.items()}
    use_y = variant != "ln_only"
    use_bias = variant in ("full", "no_ln")
    use_keep = variant in ("full", "no_bias", "ln_only", "no_ln") and use_y
    use_ln = variant != "no_ln"
    desc = D.GroupDesc(rows=rows, hidden=h, eps=1e-5, p_drop=p)
    r_out = t["resid"].clone() if inplace else torch.empty_like(t["resid"])
    resid_in = r_out if inplace else t["resid"]
    ln = torch.empty_like(r_out)
    mean = torch.empty(rows, device=d, dtype=torch.float32)
    rstd = torch.empty_like(mean)
    if not inplace:
        poison(r_out)
    poison(ln, mean, rstd)
    D.domino_resid_ln_fwd(desc, resid_in, t["y"] if use_y else None, t["bias"] if use_bias else None,
                          t["keep"] if use_keep else None, r_out, t["gamma"] if use_ln else None,
                          t["beta"] if use_ln else None, ln if use_ln else None, mean if use_ln else None,
                          rstd if use_ln else None)
    # backward
    ws_bytes = D.domino_resid_ln_bwd_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=d)
    d_resid = torch.empty_like(r_out)
    d_y = torch.empty_like(r_out)
    dg = torch.empty(h, device=d, dtype=torch.float32)
    db = torch.empty_like(dg)
    dbias = torch.empty_like(dg)
    poison(d_resid, d_y, dg, db, dbias)
    D.domino_resid_ln_bwd(desc, t["d_ln"] if use_ln else None, t["d_res"], r_out, mean if use_ln else None,
                          rstd if use_ln else None, t["gamma"] if use_ln else None, t["keep"] if use_keep else None,
                          d_resid, d_y, dg if use_ln else None, db if use_ln else None, dbias, 0, ws, ws_bytes)
    sync()

    x = {k: oracle.to_f64(v) for k, v in gi.items() if k != "keep"}
    keep = oracle.unpack_keep(gi["keep"].numpy(), h) if use_keep else None
    r_ref, ln_ref, mu_ref, rs_ref = oracle.resid_group_forward(
        x["resid"], x["y"] if use_y else None, x["bias"] if use_bias else None, keep, p,
        x["gamma"] if use_ln else None, x["beta"] if use_ln else None)
    check("resid_out", f64(r_out), r_ref, BF16_TOL)
    if use_ln:
        check("ln_out", f64(ln), ln_ref, BF16_TOL)
        check("mean", f64(mean), mu_ref, BF16_TOL)
        check("rstd", f64(rstd), rs_ref, BF16_TOL)
    dr_ref, dy_ref, dg_ref, db_ref, dbias_ref = oracle.resid_group_backward(
        x["d_ln"] if use_ln else None, x["d_res"], r_ref, keep, p, x["gamma"] if use_ln else None)
    check("d_resid", f64(d_resid), dr_ref, BF16_TOL)
    check("d_y", f64(d_y), dy_ref, BF16_TOL)
    check("d_bias", f64(dbias), dbias_ref, BF16_TOL)
    if use_ln:
        check("d_gamma", f64(dg), dg_ref, BF16_TOL)
        check("d_beta", f64(db), db_ref, BF16_TOL)
    return dict(r_out=r_out, ln=ln, d_resid=d_resid, d_y=d_y, dg=dg, db=db, dbias=dbias, desc=desc, t=t, ws=ws,
                mean=mean, rstd=rstd, ws_bytes=ws_bytes, use_keep=use_keep)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{h}" for r, h in SHAPES])
def test_group_matches_oracle(shape):
    rows, h = shape
    print(f"group rows={rows} hidden={h} full", flush=True)
    run_group(rows, h, "full")


@pytest.mark.parametrize("variant", VARIANTS[1:])
def test_group_variants(variant):
    print(f"group variant {variant}", flush=True)
    run_group(130, 264, variant, seed=11)


def test_group_inplace_and_no_dropout_probability():
    print("group in place, p = 0", flush=True)
    run_group(64, 2560, "full", p=0.0, inplace=True, seed=3)


def test_group_backward_repeatable_and_accumulates():
    print("group backward: repeatable, accumulate", flush=True)
    r = run_group(96, 1032, "full", seed=5)
    t, desc = r["t"], r["desc"]
    first = [r[k].clone() for k in ("d_resid", "d_y", "dg", "db", "dbias")]
    D.domino_resid_ln_bwd(desc, t["d_ln"], t["d_res"], r["r_out"], r["mean"], r["rstd"], t["gamma"], t["keep"],
                          r["d_resid"], r["d_y"], r["dg"], r["db"], r["dbias"], 0, r["ws"], r["ws_bytes"])
    sync()
    for a, k in zip(first, ("d_resid", "d_y", "dg", "db", "dbias")):
        assert torch.equal(a, r[k]), k
    D.domino_resid_ln_bwd(desc, t["d_ln"], t["d_res"], r["r_out"], r["mean"], r["rstd"], t["gamma"], t["keep"],
                          r["d_resid"], r["d_y"], r["dg"], r["db"], r["dbias"], 1, r["ws"], r["ws_bytes"])
    sync()
    for a, k in zip(first[2:], ("dg", "db", "dbias")):
        torch.testing.assert_close(r[k], 2 * a, rtol=1e-6, atol=1e-6)


def test_group_empty_rows():
    desc = D.GroupDesc(rows=0, hidden=64, eps=1e-5, p_drop=0.1)
    D.domino_resid_ln_fwd(desc, None, None, None, None, None, None, None, None, None, None)
    dg = torch.full((64,), 3.0, device=dev())
    D.domino_resid_ln_bwd(desc, None, None, None, None, None, None, None, None, None, None, None, dg, 1, None, 0)
    sync()
    assert torch.all(dg == 3.0)
