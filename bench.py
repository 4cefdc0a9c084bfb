"""Throughput of one tensor-parallel rank's Domino MLP block (forward + backward) on one MI355X.

A step is one pass of the whole hot path over one batch of the workload: the forward
(GEMM1 with the activation epilogue, GEMM2 per chunk, each chunk's reduction of the 8
shard partials on a second stream) and the backward (activation-gradient GEMM and
input-gradient GEMM per chunk, each chunk's reduction of dX, then the two weight-gradient
GEMMs). Peer ranks' partials are produced once before timing (they are other GPUs' work
in a real tensor-parallel group). Inputs are resident in HBM when timing starts.

Prints one JSON line: value = rank's fwd+bwd GEMM-chain TFLOP/s (algorithmic FLOPs:
3 × 2·T·h·(n1 + f_s)), plus a roofline object for the dominant kernel (its average launch
time measured with HIP events recorded on its own stream by the library) and the CPU
oracle's throughput on this host.

`--workload gpt3_6p7b_attn_tp8_row` measures the attention block of one rank instead (QKV
product, causal attention over the rank's heads, out-projection per chunk and its
reduction; then the backward: dO, the attention backward, dX per chunk and its reduction,
both weight gradients), with algorithmic FLOPs 3 × (the three products) + 3.5 × the causal
attention's 4·d·S(S+1)/2 per (sequence, head).

`--workload gpt3_6p7b_layer_tp8_row` measures a stack of whole layers (LayerNorm, attention,
dropout + residual, LayerNorm, MLP, dropout + residual) in the μ-batch schedule, forward +
backward, with the FLOPs of the attention block and of the MLP per layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402  (seeded input generators; no arithmetic of the method)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
METRIC = "TP-shard block fwd+bwd TFLOP/s (bf16) + % MFMA peak; shard_reduce GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt3_2p7b_mlp_tp8_row")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=7)
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size first (for HBM counter calibration)")
    return ap.parse_args()


TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "traffic_*_gpt3_2p7b_mlp.txt")
GEMM_SOURCE = os.path.join(ROOT, "tensor_transformer_block_domino_amd", "csrc", "gemm_bf16.hip")


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, calibrated against a plain copy), or None if the summary covers another
    kernel or the kernel source changed since the counters were taken."""
    import glob
    import hashlib

    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        try:
            kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
            if kv.get("kernel_source_sha256", "").strip() == src and kv.get("kernel", "").strip() == kernel:
                return float(kv["calibrated_bytes_per_launch"])
        except (OSError, KeyError, ValueError):
            continue
    return None


def mlp_flops(w):
    fwd = 2.0 * w.tokens * w.hidden * w.n1 + 2.0 * w.tokens * w.ffn_shard * w.hidden
    return fwd, 3.0 * fwd


def kernel_flops(w, kind):
    """Algorithmic FLOPs of one launch of each GEMM kind in the workload's schedule."""
    T, h, f, n1 = w.tokens, w.hidden, w.ffn_shard, w.n1
    Tc = T // w.row_chunks
    hc_f = h // w.col_chunks
    bwd_rows = w.row_chunks
    bwd_cols = 1 if w.row_chunks > 1 else w.col_chunks
    return {
        "fwd_gemm1": 2.0 * Tc * h * n1,
        "fwd_gemm2": 2.0 * Tc * f * hc_f,
        "dgrad_b": 2.0 * (T // bwd_rows) * h * f,
        "dgrad_a": 2.0 * (T // bwd_rows) * n1 * (h // bwd_cols),
        "wgrad_b": 2.0 * T * f * h,
        "wgrad_a": 2.0 * T * h * n1,
    }[kind]


def cpu_baseline(w, inp, reps):
    """The oracle (numpy fp64) on this host: one rank's forward + backward of the workload."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    X, A, B, dY = (oracle.to_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    A0, B0 = oracle.mlp_shard_weights(A, B, w.act, w.n_partials, 0)
    A0, B0 = np.ascontiguousarray(A0), np.ascontiguousarray(B0)
    _, total = mlp_flops(w)
    best, done, start = None, 0, time.perf_counter()
    while done < max(1, reps):
        t0 = time.perf_counter()
        oracle.mlp_shard_forward(X, A0, B0, w.act)
        oracle.mlp_shard_backward(X, A0, B0, dY, w.act)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
        done += 1
        if time.perf_counter() - start > 25:  # bound the whole baseline to ~25 s of CPU work
            break
    return {"value": total / best / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one rank's full forward+backward of {w.name} (T={w.tokens}, fp64 numpy), best of "
                      f"{done} reps, {best:.2f} s each"}


def attn_flops(w):
    """Algorithmic FLOPs per step of each timed role of the attention block (one rank)."""
    T, h, hd = w.tokens, w.hidden, w.heads_shard * w.head_dim
    att = 4.0 * w.head_dim * w.seq * (w.seq + 1) / 2 * w.heads_shard * w.batch
    return {
        "qkv": 2.0 * T * h * 3 * hd, "attn": att, "outproj": 2.0 * T * hd * h,
        "outproj_dgrad": 2.0 * T * h * hd,
        # dK/dV kernel: S, dP, dV, dK over the causal pairs; dQ kernel: dQ (it also
        # computes S and dP again, which is not counted).
        "attn_bwd_prep": 0.0, "attn_bwd_dkdv": 2.0 * att, "attn_bwd_dq": 0.5 * att,
        "qkv_dgrad": 2.0 * T * 3 * hd * h, "outproj_wgrad": 2.0 * T * hd * h, "qkv_wgrad": 2.0 * T * h * 3 * hd,
    }


def cpu_baseline_attn(w, inp, reps, n_seq=2):
    """The oracle (numpy fp64) on this host: one rank's attention forward + backward over the
    first n_seq sequences of the workload."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    rows = n_seq * w.seq
    X, Aqkv, Bo, dY = (oracle.to_f64(inp[k]) for k in ("X", "Aqkv", "Bo", "dY"))
    A0, B0 = oracle.attn_shard_weights(Aqkv, Bo, w.heads_full, w.head_dim, w.n_partials, 0)
    A0, B0 = np.ascontiguousarray(A0), np.ascontiguousarray(B0)
    X, dY = np.ascontiguousarray(X[:rows]), np.ascontiguousarray(dY[:rows])
    sub = synth.AttnWorkload(w.name, batch=n_seq, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard,
                             head_dim=w.head_dim, dtype=w.dtype, row_chunks=1, n_partials=w.n_partials, seed=w.seed)
    total = sum(attn_flops(sub).values())
    best, done, start = None, 0, time.perf_counter()
    while done < max(1, reps):
        t0 = time.perf_counter()
        oracle.attn_shard_forward(X, A0, B0, n_seq, w.seq, w.heads_shard, w.head_dim)
        oracle.attn_shard_backward(X, A0, B0, dY, n_seq, w.seq, w.heads_shard, w.head_dim)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
        done += 1
        if time.perf_counter() - start > 25:  # bound the whole baseline to ~25 s of CPU work
            break
    return {"value": total / best / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one rank's attention forward+backward over {n_seq} of the {w.batch} sequences of {w.name} "
                      f"(fp64 numpy), best of {done} reps, {best:.2f} s each"}


def main_attn(args, w):
    import torch

    import tensor_transformer_block_domino_amd as D
    from tensor_transformer_block_domino_amd.tp_sim import AttnGroup

    dev = torch.device("cuda:0")
    inp = synth.attn_inputs(w)
    g = AttnGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                  row_chunks=w.row_chunks, n_partials=w.n_partials, X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"],
                  dY=inp["dY"], device=dev)
    g.peer_forward()
    g.forward()
    g.peer_backward()
    torch.cuda.synchronize()
    compute = torch.cuda.Stream()
    comm = torch.cuda.Stream()

    def step_domino():
        g.forward(compute, comm, no_join=1)
        g.backward(compute, comm)

    def step_unsplit():
        g.forward(compute, None, rank_alone=True, row_chunks=1)
        g.backward(compute, None, rank_alone=True, row_chunks=1)

    ms = timed_steps(step_domino, args.steps, args.warmup)
    print(f"[bench] attention domino step {ms:.3f} ms", file=sys.stderr, flush=True)
    ms_unsplit = timed_steps(step_unsplit, args.steps, 2)

    D.domino_timing_enable(True)
    for _ in range(args.steps):
        step_domino()
    torch.cuda.synchronize()
    fl = attn_flops(w)
    roles = list(fl) + ["reduce", "aux"]
    per = {r: D.domino_timing_read(r) for r in roles}
    kernel_of = {r: D.domino_timing_kernel(r) for r in roles}
    D.domino_timing_enable(False)
    total_flops = sum(fl.values())
    value = total_flops / (ms * 1e-3) / 1e12
    by_kernel = {}
    for r in fl:
        if fl[r] > 0:
            by_kernel.setdefault(kernel_of[r], []).append(r)
    dom = max(by_kernel, key=lambda k: sum(per[r][1] for r in by_kernel[k]))
    n_dom = sum(per[r][0] for r in by_kernel[dom])
    tot_dom = sum(per[r][1] for r in by_kernel[dom])
    flops_dom = sum(fl[r] for r in by_kernel[dom]) * args.steps
    achieved = flops_dom / (tot_dom * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads_shard": w.heads_shard, "head_dim": w.head_dim, "tp_partials": w.n_partials,
                   "split": f"rows x{w.row_chunks}", "pass": "fwd+bwd", "attention": "causal"},
        "mfma_peak_frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "t_domino_ms": round(ms, 4),
        "t_unsplit_no_reduce_ms": round(ms_unsplit, 4),
        "t_reduce_ms": round(per["reduce"][1] / args.steps, 4),
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()},
        "kernel_tflops": {r: round(fl[r] * args.steps / (per[r][1] * 1e-3) / 1e12, 1)
                          for r in fl if fl[r] > 0 and per[r][1] > 0},
        "kernel_of_role": kernel_of,
        "roofline": {"bound": "mfma", "kernel": dom, "roles": by_kernel[dom], "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_us": round(tot_dom / max(1, n_dom) * 1e3, 2), "launches": n_dom,
                     "flops_per_launch": flops_dom / max(1, n_dom)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_attn(w, inp, args.cpu_reps)
    print(json.dumps(out), flush=True)


def layer_flops(w):
    """Algorithmic FLOPs per step of each timed role of the layer stack (one rank, all layers)."""
    T, h, f = w.tokens, w.hidden, w.ffn_shard
    n1 = 2 * f if w.act == "swiglu" else f
    fl = {k: v * w.layers for k, v in attn_flops(w).items()}
    for k, v in {"fwd_gemm1": 2.0 * T * h * n1, "fwd_gemm2": 2.0 * T * f * h, "dgrad_b": 2.0 * T * h * f,
                 "dgrad_a": 2.0 * T * n1 * h, "wgrad_b": 2.0 * T * f * h, "wgrad_a": 2.0 * T * h * n1}.items():
        fl[k] = v * w.layers
    return fl


def cpu_baseline_layer(w, inp, n_seq=1):
    """The oracle on this host: the whole (unsharded) stack's forward + backward over the
    first n_seq sequences, counted at one rank's share of the FLOPs (÷ P)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    rows = slice(0, n_seq * w.seq)
    X = oracle.to_f64(inp["X"][rows])
    dY = oracle.to_f64(inp["dY"][rows])
    layers, keeps = [], []
    for lay in inp["layers"]:
        layers.append({k: oracle.to_f64(lay[k]) for k in ("ln1_g", "ln1_b", "Aqkv", "Bo", "ln2_g", "ln2_b", "A", "B")})
        keeps.append((oracle.unpack_keep(lay["keep1"][rows].numpy(), w.hidden),
                      oracle.unpack_keep(lay["keep2"][rows].numpy(), w.hidden)))
    sub = synth.LayerWorkload(w.name, batch=n_seq, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard,
                              head_dim=w.head_dim, ffn_shard=w.ffn_shard, act=w.act, row_chunks=1,
                              n_partials=w.n_partials, layers=w.layers, p_drop=w.p_drop, seed=w.seed)
    total = sum(layer_flops(sub).values())
    t0 = time.perf_counter()
    oracle.stack_backward(X, layers, keeps, w.p_drop, dY, n_seq, w.seq, w.heads_full, w.head_dim, w.act)
    dt = time.perf_counter() - t0
    # The oracle computes all P ranks' work (the unsharded layer): count its FLOPs as P shares.
    return {"value": total * w.n_partials / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the unsharded {w.layers}-layer stack's forward+backward (oracle.stack_backward, which runs the "
                      f"forward too) over {n_seq} of the {w.batch} sequences of {w.name} (fp64 numpy), one run, "
                      f"{dt:.1f} s"}


def main_layer(args, w):
    import torch

    import tensor_transformer_block_domino_amd as D
    from tensor_transformer_block_domino_amd.tp_sim import LayerGroup

    print("[bench] generating the layer inputs", file=sys.stderr, flush=True)
    inp = synth.layer_inputs(w)
    g = LayerGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                   ffn_shard=w.ffn_shard, act=w.act, row_chunks=w.row_chunks, n_partials=w.n_partials,
                   p_drop=w.p_drop, X=inp["X"], layers=inp["layers"], device=torch.device("cuda:0"))
    g.alloc_backward(inp["dY"])
    print("[bench] peer partials (the other ranks' work, once)", file=sys.stderr, flush=True)
    g.peer_forward()
    g.peer_backward()
    torch.cuda.synchronize()
    compute, comm = torch.cuda.Stream(), torch.cuda.Stream()

    def step_domino():
        g.forward(compute, comm)
        g.backward(compute, comm)

    def step_serial():
        g.forward(compute, None)
        g.backward(compute, None)

    def step_unsplit():
        g.forward(compute, comm, row_chunks=1)
        g.backward(compute, comm, row_chunks=1)

    ms = timed_steps(step_domino, args.steps, args.warmup)
    print(f"[bench] layer stack domino step {ms:.3f} ms", file=sys.stderr, flush=True)
    ms_serial = timed_steps(step_serial, args.steps, 2)
    ms_unsplit = timed_steps(step_unsplit, args.steps, 2)
    ms_graph = graph_steps(step_domino, compute, args.steps)
    D.domino_timing_enable(True)
    for _ in range(args.steps):
        step_domino()
    torch.cuda.synchronize()
    fl = layer_flops(w)
    roles = list(fl) + ["reduce", "aux", "group_fwd", "group_bwd"]
    per = {r: D.domino_timing_read(r) for r in roles}
    kernel_of = {r: D.domino_timing_kernel(r) for r in roles}
    D.domino_timing_enable(False)
    total_flops = sum(fl.values())
    value = total_flops / (ms * 1e-3) / 1e12
    by_kernel = {}
    for r in fl:
        if fl[r] > 0 and per[r][0] > 0:
            by_kernel.setdefault(kernel_of[r], []).append(r)
    dom = max(by_kernel, key=lambda k: sum(per[r][1] for r in by_kernel[k]))
    n_dom = sum(per[r][0] for r in by_kernel[dom])
    tot_dom = sum(per[r][1] for r in by_kernel[dom])
    flops_dom = sum(fl[r] for r in by_kernel[dom]) * args.steps
    achieved = flops_dom / (tot_dom * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads_shard": w.heads_shard, "head_dim": w.head_dim, "ffn_shard": w.ffn_shard, "act": w.act,
                   "layers": w.layers, "p_drop": w.p_drop, "tp_partials": w.n_partials,
                   "split": f"rows x{w.row_chunks} (mu-batches)", "pass": "fwd+bwd"},
        "mfma_peak_frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "t_domino_ms": round(ms, 4),
        "t_serial_ms": round(ms_serial, 4),
        "t_unsplit_ms": round(ms_unsplit, 4),
        "t_graph_ms": round(ms_graph, 4),
        "t_reduce_ms": round(per["reduce"][1] / args.steps, 4),
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()},
        "kernel_tflops": {r: round(fl[r] * args.steps / (per[r][1] * 1e-3) / 1e12, 1)
                          for r in fl if fl[r] > 0 and per[r][1] > 0},
        "kernel_of_role": kernel_of,
        "roofline": {"bound": "mfma", "kernel": dom, "roles": by_kernel[dom], "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_us": round(tot_dom / max(1, n_dom) * 1e3, 2), "launches": n_dom,
                     "flops_per_launch": flops_dom / max(1, n_dom)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_layer(w, inp)
    print(json.dumps(out), flush=True)


def graph_steps(fn, stream, steps):
    """The step captured once into a HIP graph on `stream` and replayed: ms per replay."""
    import torch

    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    return timed_steps(graph.replay, steps, 2)


def timed_steps(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported: the library sums the "
              f"tensor-parallel partials on one GPU, with no collective between GPUs", file=sys.stderr)
        sys.exit(2)
    import torch

    import tensor_transformer_block_domino_amd as D
    from tensor_transformer_block_domino_amd.tp_sim import MlpGroup

    D.load()
    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS[args.workload]
    if isinstance(w, synth.AttnWorkload):
        return main_attn(args, w)
    if isinstance(w, synth.LayerWorkload):
        return main_layer(args, w)
    assert isinstance(w, synth.MlpWorkload) and w.dtype == "bf16"
    dev = torch.device("cuda:0")
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn_shard=w.ffn_shard, act=w.act, dtype=w.dtype,
                 row_chunks=w.row_chunks, col_chunks=w.col_chunks, n_partials=w.n_partials, X=inp["X"], A=inp["A"],
                 B=inp["B"], dY=inp["dY"], device=dev)
    g.peer_forward()
    g.forward()
    g.peer_backward()
    torch.cuda.synchronize()
    compute = torch.cuda.Stream()
    comm = torch.cuda.Stream()

    def step_domino():
        g.forward(compute, comm, no_join=1)
        g.backward(compute, comm)

    def step_serial():
        g.forward(compute, None, row_chunks=1, col_chunks=1)
        g.backward(compute, None, row_chunks=1, col_chunks=1)

    def step_unsplit():
        d_f = g.desc(rank_alone=True, row_chunks=1, col_chunks=1)
        D.domino_block_fwd(d_f, g.X, g.A_s[0], g.B_s[0], g.Hpre[0], g.H[0], g.Y_own[0], None, None, g.ws, g.ws_bytes,
                           compute, None)
        D.domino_block_bwd(d_f, g.X, g.A_s[0], g.B_s[0], g.Hpre[0], g.H[0], g.dY, g.dHpre[0], g.dX_own[0], None,
                           None, g.dA, g.dB, 0, g.ws, g.ws_bytes, compute, None)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    # The timed region: Domino chunks, reductions on the second stream.
    ms = timed(step_domino, args.steps, args.warmup)
    print(f"[bench] domino step {ms:.3f} ms", file=sys.stderr, flush=True)
    ms_serial = timed(step_serial, args.steps, 2)
    ms_unsplit = timed(step_unsplit, args.steps, 2)
    ms_graph = graph_steps(step_domino, compute, args.steps)
    print(f"[bench] serial {ms_serial:.3f} ms, unsplit without reduce {ms_unsplit:.3f} ms", file=sys.stderr,
          flush=True)

    # Per-kernel durations: the same Domino steps with the library's event timing on.
    D.domino_timing_enable(True)
    for _ in range(args.steps):
        step_domino()
    torch.cuda.synchronize()
    per, kernel_of = {}, {}
    for kind in ("reduce", "fwd_gemm1", "fwd_gemm2", "dgrad_b", "dgrad_a", "wgrad_b", "wgrad_a", "aux"):
        n, tot = D.domino_timing_read(kind)
        per[kind] = (n, tot)
        kernel_of[kind] = D.domino_timing_kernel(kind)
    # shard_reduce alone: the whole [T, h] output, the 8 partials, on an idle GPU. The rate is
    # taken over back-to-back launches between one pair of events on their stream (the gaps
    # between launches included); the library's per-launch events, which also span each
    # launch's dispatch and completion signal, are reported beside it.
    D.domino_timing_enable(True)
    parts = [g.Y_own[r] for r in g.ranks]
    for _ in range(args.steps):
        D.shard_reduce(g.Y, w.hidden, parts, w.hidden, w.tokens, w.hidden, D.DOMINO_BF16, compute)
    torch.cuda.synchronize()
    n_sa, tot_sa = D.domino_timing_read("reduce")
    D.domino_timing_enable(False)
    red_ev_us = tot_sa / max(1, n_sa) * 1e3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(args.steps, 20)
    e0.record(compute)
    for _ in range(reps):
        D.shard_reduce(g.Y, w.hidden, parts, w.hidden, w.tokens, w.hidden, D.DOMINO_BF16, compute)
    e1.record(compute)
    torch.cuda.synchronize()
    red_sa_us = e0.elapsed_time(e1) / reps * 1e3
    red_sa_gbps = (w.n_partials + 1) * w.tokens * w.hidden * 2 / (red_sa_us * 1e-6) / 1e9

    fwd_flops, total_flops = mlp_flops(w)
    value = total_flops / (ms * 1e-3) / 1e12
    gemm_kinds = ["fwd_gemm1", "fwd_gemm2", "dgrad_b", "dgrad_a", "wgrad_b", "wgrad_a"]
    # Dominant kernel: the GEMM kernel (one template instantiation, as the profiler names
    # it) with the most time per step, over every schedule role that launched it.
    by_kernel = {}
    for r in gemm_kinds:
        by_kernel.setdefault(kernel_of[r], []).append(r)
    dom = max(by_kernel, key=lambda k: sum(per[r][1] for r in by_kernel[k]))
    n_dom = sum(per[r][0] for r in by_kernel[dom])
    tot_dom = sum(per[r][1] for r in by_kernel[dom])
    flops_dom = sum(per[r][0] * kernel_flops(w, r) for r in by_kernel[dom])
    avg_ms = tot_dom / max(1, n_dom)
    achieved = flops_dom / (tot_dom * 1e-3) / 1e12
    n_red, tot_red = per["reduce"]
    # Reduced bytes per step: Y and dX, each (P+1)·T·h·2 bytes.
    red_bytes_step = 2 * (w.n_partials + 1) * w.tokens * w.hidden * 2
    red_ms_step = tot_red / args.steps
    red_gbps = red_bytes_step / (red_ms_step * 1e-3) / 1e9
    gemm_ms_step = sum(per[k][1] for k in gemm_kinds) / args.steps
    hidden_frac = 1.0 - (ms - ms_unsplit) / red_ms_step if red_ms_step > 0 else None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "ffn_shard": w.ffn_shard, "act": w.act, "tp_partials": w.n_partials,
                   "split": f"rows x{w.row_chunks}, cols x{w.col_chunks}", "pass": "fwd+bwd"},
        "mfma_peak_frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "gemm_chain_tflops": round(total_flops / (gemm_ms_step * 1e-3) / 1e12, 2),
        "shard_reduce_GBps": round(red_sa_gbps, 1),
        "shard_reduce_hbm_frac": round(red_sa_gbps / HBM_PEAK_GBPS, 4),
        "shard_reduce_avg_us": round(red_sa_us, 2),
        "shard_reduce_event_us": round(red_ev_us, 2),
        "shard_reduce_in_step_GBps": round(red_gbps, 1),
        "t_domino_ms": round(ms, 4),
        "t_serial_ms": round(ms_serial, 4),
        "t_unsplit_no_reduce_ms": round(ms_unsplit, 4),
        "t_graph_ms": round(ms_graph, 4),
        "t_reduce_ms": round(red_ms_step, 4),
        "hidden_fraction": None if hidden_frac is None else round(hidden_frac, 3),
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()},
        "kernel_of_role": kernel_of,
        "roofline": {"bound": "mfma", "kernel": dom, "roles": by_kernel[dom], "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(dom) if args.workload == "gpt3_2p7b_mlp_tp8_row" else None,
                     "avg_launch_us": round(avg_ms * 1e3, 2), "launches": n_dom,
                     "flops_per_launch": flops_dom / max(1, n_dom)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
