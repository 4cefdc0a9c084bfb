"""Throughput of one tensor-parallel rank's Domino block on one MI355X.

Default line: the Llama-2-13B-shaped SwiGLU MLP shard at TP 8 with the 2D split (rows ×2,
columns ×2), forward + backward — the largest workload that fits one GPU. A step is one
pass of the whole hot path over one batch: GEMM1 with the SwiGLU epilogue once over all
rows; GEMM2 per 2D chunk (r0c0, r0c1, r1c0, r1c1), each chunk's reduction of the 8 shard
partials on a second stream; the activation-gradient GEMM; the input-gradient GEMM per
row chunk, each chunk's reduction of dX on the second stream; the two weight-gradient
GEMMs behind the last reduction. Peer ranks' partials are produced once before timing
(other GPUs' work in a real tensor-parallel group). Inputs are resident in HBM when
timing starts.

Timing policy: before every timed step a 1 GiB scratch buffer is read and written on the
compute stream (outside the step's event pair), so no step starts with the previous
step's operands in the 256 MB last-level cache or the L2s; each step is bracketed by HIP
events on the compute stream (its reductions join that stream at the end), and
ms_per_step is their mean. The same steps back to back without the flush are reported
beside it (`t_domino_backtoback_ms`).

Prints one JSON line: value = the rank's fwd+bwd GEMM-chain TFLOP/s (algorithmic FLOPs:
3 × 2·T·h·(n1 + f_s)); a roofline object for the dominant kernel (its launches timed by
events the launches' own dispatches record); T_unsplit (one chunk, no reduction: tensor-
parallel communication disabled), T_serial (one chunk, reductions on the same stream),
T_domino and the standalone reduction time, with hidden_fraction = 1 − (T_domino −
T_unsplit) / T_reduce; the CPU oracle's throughput on this host; and, as extra keys, the
same step figures for the Llama-2-7B column-split and GPT-3-2.7B row-split MLP workloads,
the GPT-3-6.7B attention block's forward alone (with its last reduction exposed) and the
two-layer GPT-3-6.7B stack (forward + backward, μ-batch schedule).

`--workload gpt3_6p7b_attn_tp8_row` measures the attention block of one rank instead (QKV
product, causal attention over the rank's heads, out-projection per chunk and its
reduction; then the backward: dO, the attention backward, dX per chunk and its reduction,
both weight gradients), with algorithmic FLOPs 3 × (the three products) + 3.5 × the causal
attention's 4·d·S(S+1)/2 per (sequence, head).

`--workload gpt3_6p7b_layer_tp8_row` measures a stack of whole layers (LayerNorm, attention,
dropout + residual, LayerNorm, MLP, dropout + residual) in the μ-batch schedule, forward +
backward, with the FLOPs of the attention block and of the MLP per layer.

`--traffic-summary FETCH.csv WRITE.csv KERNEL COPY_MIB WORKLOAD OUT.txt` writes the HBM
traffic summary of one kernel from two rocprofv3 counter runs of this bench (one
FETCH_SIZE, one WRITE_SIZE), calibrated against the plain device copy that
`--calibration-copy-mib` runs first; bench reports that traffic while the kernel source
is unchanged.
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
DEFAULT_WORKLOAD = "llama2_13b_swiglu_tp8_2d"
DEFAULT_ALSO = "llama2_7b_swiglu_tp8_col,gpt3_2p7b_mlp_tp8_row,gpt3_6p7b_attn_tp8_row,gpt3_6p7b_layer_tp8_row"
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads whose step figures are added as extra keys "
                         f"(default with the default workload: {DEFAULT_ALSO}; 'none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=2)
    ap.add_argument("--no-flush", action="store_true", help="time steps back to back without the cache flush")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size first (for HBM counter calibration)")
    ap.add_argument("--traffic-summary", nargs=6, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL", "COPY_MIB",
                                                           "WORKLOAD", "OUT"))
    ap.add_argument("--traffic-workgroups", default="",
                    help="with --traffic-summary: only the kernel's dispatches of these workgroup counts "
                         "(comma-separated)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_CSV", "OUT"),
                    help="per-kernel, per-launch-shape statistics of a rocprofv3 kernel trace")
    ap.add_argument("--timeline-summary", nargs=3, metavar=("TRACE_CSV", "OUT", "TITLE"),
                    help="write one Domino step of a rocprofv3 kernel trace of this bench as a timeline")
    ap.add_argument("--counter-summary", nargs="+", metavar="OUT TITLE CSV",
                    help="write per-kernel averages of rocprofv3 counter runs: OUT TITLE CSV [CSV ...]")
    ap.add_argument("--trace-command", default="", help="the command that made the trace (recorded in the summary)")
    return ap.parse_args()


KERNEL_SOURCES = [os.path.join(ROOT, "tensor_transformer_block_domino_amd", "csrc", f)
                  for f in ("gemm_bf16.hip", "gemm8.hip", "gemm_common.hpp", "common.hpp")]


def kernel_source_sha():
    import hashlib

    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` in `workload` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or None if no summary
    covers that kernel and workload or the GEMM source changed since the counters were
    taken."""
    import glob

    src = kernel_source_sha()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"traffic_*_{workload}.txt"))):
        try:
            kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
            if kv.get("kernel_source_sha256", "").strip() == src and kv.get("kernel", "").strip() == kernel:
                return float(kv["calibrated_bytes_per_launch"])
        except (OSError, KeyError, ValueError):
            continue
    return None


def traffic_summary(fetch_csv, write_csv, kernel, copy_mib, workload, out_path, workgroups=""):
    """Writes the traffic summary bench reads (measured_traffic) from two counter runs,
    over the kernel's dispatches of the given workgroup counts (comma-separated; all of
    them when empty)."""
    import csv

    shapes = {int(x) for x in str(workgroups).split(",") if x.strip()}

    def values(path, counter):
        out = {}
        for row in csv.DictReader(open(path)):
            wgs = int(row["Grid_Size"]) // max(1, int(row["Workgroup_Size"]))
            if row["Counter_Name"] == counter and (not shapes or wgs in shapes
                                                   or "copyBuffer" in row["Kernel_Name"]):
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return out

    def norm(name):
        # rocprofv3 prints the demangled symbol with "void", the namespaces and the
        # parameter list; the library names the template instantiation alone.
        n = name.replace(" ", "").replace("domino::(anonymousnamespace)::", "")
        return n[4:] if n.startswith("void") else n

    def match(vals):
        want = norm(kernel)
        return [v for name, vs in vals.items() if norm(name).startswith(want + "(") for v in vs]

    copy_kib = float(copy_mib) * 1024
    fetch, write = values(fetch_csv, "FETCH_SIZE"), values(write_csv, "WRITE_SIZE")
    f_copy = sum(fetch["__amd_rocclr_copyBuffer"]) / len(fetch["__amd_rocclr_copyBuffer"])
    w_copy = sum(write["__amd_rocclr_copyBuffer"]) / len(write["__amd_rocclr_copyBuffer"])
    fs, ws = copy_kib / f_copy, copy_kib / w_copy
    fk, wk = match(fetch), match(write)
    if not fk or not wk:
        raise SystemExit(f"kernel {kernel} not found in the counter files")
    f_avg, w_avg = sum(fk) / len(fk), sum(wk) / len(wk)
    lines = [
        f"kernel: {kernel}",
        f"workload: {workload}",
        f"workgroups: {workgroups or 'all launch shapes'}",
        f"kernel_source_sha256: {kernel_source_sha()}",
        f"fetch_kib_per_launch: {f_avg:.1f}",
        f"write_kib_per_launch: {w_avg:.1f}",
        f"fetch_scale: {fs:.4f}",
        f"write_scale: {ws:.4f}",
        f"calibrated_bytes_per_launch: {int(round((f_avg * fs + w_avg * ws) * 1024))}",
        f"# {len(fk)} dispatches averaged; the {copy_mib} MiB copy read FETCH_SIZE {f_copy:.0f} KiB and "
        f"WRITE_SIZE {w_copy:.0f} KiB for {copy_kib:.0f} KiB moved each way.",
    ]
    cmd = f"python3 bench.py --workload {workload} --also none --no-cpu-baseline --steps 3 --warmup 1 " \
          f"--calibration-copy-mib {copy_mib}"
    header = [
        f"# HBM traffic of {kernel} in the {workload} bench step.",
        "# Two rocprofv3 counter runs of the bench command, one counter each, then this summary:",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o fetch -- {cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o write -- {cmd}",
        f"#   python3 bench.py --traffic-summary <dir>/fetch_counter_collection.csv "
        f"<dir>/write_counter_collection.csv '{kernel}' {copy_mib} {workload} <this file>"
        + (f" --traffic-workgroups {workgroups}" if workgroups else ""),
    ]
    tail = [l.rstrip("\n") for l in open(out_path) if l.startswith("algorithmic") or l.startswith("# ")
            and not l.startswith("# HBM") and not l.startswith("#   ") and not l.startswith("# Two")
            and "dispatches averaged" not in l] if os.path.exists(out_path) else []
    with open(out_path, "w") as f:
        f.write("\n".join(header + lines + tail) + "\n")
    print("\n".join(lines))


def trace_summary(trace_csv, out_path, command=""):
    """Writes per-kernel statistics of a rocprofv3 kernel trace, one line per kernel and
    launch shape (grid size): a kernel launched on chunks and on whole tensors gets one
    line for each, so the average of the launches a bench figure covers can be read off."""
    import csv

    rows = {}
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"].replace("domino::(anonymous namespace)::", "").replace("void ", "")
        name = name[:name.rfind(">(") + 1] if ">(" in name else name.split("(")[0]
        key = (name, int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])), int(r["Workgroup_Size_X"]))
        d = rows.setdefault(key, {"n": 0, "tot": 0.0, "min": 1e30, "max": 0.0, "vgpr": r["VGPR_Count"],
                                  "agpr": r["Accum_VGPR_Count"], "lds": r["LDS_Block_Size"]})
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        d["n"] += 1
        d["tot"] += us
        d["min"] = min(d["min"], us)
        d["max"] = max(d["max"], us)
    total = sum(d["tot"] for d in rows.values())
    lines = [f"# Kernel statistics per launch shape: `{os.path.basename(trace_csv)}`", ""]
    if command:
        lines += ["Made by:", "", "```", command,
                  f"python3 bench.py --trace-summary {trace_csv} {out_path} --trace-command '<the line above>'",
                  "```", ""]
    lines += ["| kernel | workgroups | threads | calls | avg µs | min µs | max µs | total ms | % | VGPR | AGPR | LDS B |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (name, wgs, thr), d in sorted(rows.items(), key=lambda kv: -kv[1]["tot"]):
        lines.append(f"| `{name}` | {wgs} | {thr} | {d['n']} | {d['tot'] / d['n']:.1f} | {d['min']:.1f} | "
                     f"{d['max']:.1f} | {d['tot'] * 1e-3:.3f} | {100 * d['tot'] / total:.1f} | {d['vgpr']} | "
                     f"{d['agpr']} | {d['lds']} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def timeline_summary(trace_csv, out_path, title, command=""):
    """Writes one Domino step of a rocprofv3 kernel trace of this bench as a timeline: the
    timed Domino steps come first in the trace, each after the cache flush (an elementwise
    torch kernel); the step shown is the one of median length among those whose kernels ran
    on two queues (the compute stream and the reductions' stream)."""
    import csv

    rows = []
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"].replace("domino::(anonymous namespace)::", "").replace("void ", "")
        name = name[:name.rfind(">(") + 1] if ">(" in name else name.split("(")[0]
        rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r.get("Queue_Id", "?"), name,
                     int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))))
    rows.sort()
    flush = [i for i, r in enumerate(rows) if "elementwise" in r[3]]
    steps = []
    for a, b in zip(flush, flush[1:]):
        win = rows[a + 1:b]
        if win and len({r[2] for r in win}) > 1 and any("shard_reduce" in r[3] for r in win):
            steps.append(win)
        elif steps:
            break       # the Domino phase is over
    if not steps:
        raise SystemExit("no Domino step found in the trace")
    dur = lambda win: max(r[1] for r in win) - win[0][0]
    order = sorted(range(len(steps)), key=lambda i: dur(steps[i]))
    pick = order[len(order) // 2]
    win = steps[pick]
    t0 = win[0][0]
    queues = sorted({r[2] for r in win}, key=lambda q: -sum(r[1] - r[0] for r in win if r[2] == q))
    main_q = queues[0]

    def busy(q):
        iv = sorted((r[0], r[1]) for r in win if r[2] == q)
        out, cur = [], None
        for a, b in iv:
            if cur and a <= cur[1]:
                cur[1] = max(cur[1], b)
            else:
                cur = [a, b]
                out.append(cur)
        return out

    def overlap(x, y):
        tot = 0
        for a, b in x:
            for c, d in y:
                tot += max(0, min(b, d) - max(a, c))
        return tot

    bq = {q: busy(q) for q in queues}
    span = dur(win)
    lines = [f"# One Domino step on the timeline ({title})", ""]
    if command:
        lines += ["Made by:", "", "```", command,
                  f"python3 bench.py --timeline-summary {os.path.basename(trace_csv)} <this file> '<title>' "
                  "--trace-command '<the line above>'", "```", ""]
    lines += [
        f"Step {pick + 1} of the {len(steps)} flushed Domino steps in the trace (the median length; "
        f"lengths {dur(steps[order[0]]) / 1e3:.1f}-{dur(steps[order[-1]]) / 1e3:.1f} µs). Queue {main_q} is the "
        "compute stream; the reductions run on the other queue.", "",
        f"- step, first kernel start to last kernel end: {span / 1e3:.1f} µs",
    ]
    for q in queues:
        b = sum(e - s for s, e in bq[q])
        lines.append(f"- queue {q} busy: {b / 1e3:.1f} µs ({100 * b / span:.0f}% of the step)")
    if len(queues) > 1:
        ov = overlap(bq[queues[0]], bq[queues[1]])
        comm = sum(e - s for s, e in bq[queues[1]])
        lines.append(f"- reductions' queue busy while the compute queue is busy: {ov / 1e3:.1f} µs "
                     f"({100 * ov / max(1, comm):.0f}% of its busy time)")
    lines += ["", "| start µs | end µs | dur µs | queue | workgroups | kernel |", "|---:|---:|---:|---:|---:|---|"]
    for s0, e0, q, name, wgs in win:
        lines.append(f"| {(s0 - t0) / 1e3:.1f} | {(e0 - t0) / 1e3:.1f} | {(e0 - s0) / 1e3:.1f} | {q} | {wgs} | `{name}` |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:14]))


def counter_summary(out_path, title, command, *csv_paths):
    """Writes per-kernel averages of rocprofv3 counter runs of this bench (one line per kernel
    and launch shape), with the clock each kernel ran at: GRBM_GUI_ACTIVE counts GPU cycles
    summed over the 8 XCDs, so cycles / 8 / the dispatch's duration is its clock."""
    import csv
    import collections

    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].replace("domino::(anonymous namespace)::", "").replace("domino::", "")
            name = name.replace("void ", "")
            name = name[:name.rfind(">(") + 1] if ">(" in name else name.split("(")[0]
            key = (name, int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            agg[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[key][(path, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    names = sorted({c for v in agg.values() for c in v})
    cols = [c for c in ("MfmaUtil", "LdsUtil", "LdsBankConflict", "LdsLatency") if c in names]
    extra = [c for c in names if c not in cols and c not in ("GRBM_GUI_ACTIVE", "TA_BUSY_avr", "TD_TD_BUSY_sum")]
    unit = "TA_BUSY_avr" in names and "TD_TD_BUSY_sum" in names and "GRBM_GUI_ACTIVE" in names
    lines = [f"# Hardware counters per kernel ({title})", "", "Made by:", "", "```"] + list(command.split("\n")) + [
        f"python3 bench.py --counter-summary <this file> '<title>' <dir>/*_counter_collection.csv "
        "--trace-command '<the lines above>'", "```", "",
        "Averages over every dispatch of a kernel and launch shape in the command (warmup, timed, serial and "
        "unsplit steps alike). `MfmaUtil` = MFMA-busy cycles / (active cycles × SIMDs); `LdsUtil` = LDS-busy "
        "fraction; `LdsBankConflict` = bank-conflict cycles per LDS access cycle. The clock is GRBM_GUI_ACTIVE "
        "/ 8 / the dispatch's duration (meaningful for dispatches of more than ~50 µs)."]
    if unit:
        lines += ["TA busy = TA_BUSY_avr / (GRBM_GUI_ACTIVE / 8); TD busy = TD_TD_BUSY_sum / 256 CUs / "
                  "(GRBM_GUI_ACTIVE / 8). TA addresses vector-memory requests (copies to LDS included), TD "
                  "returns their data."]
    hdr = ["kernel", "workgroups", "dispatches", "avg µs"] + (["clock GHz"] if "GRBM_GUI_ACTIVE" in names else []) \
        + cols + (["TA busy %", "TD busy %"] if unit else []) + extra
    lines += ["", "| " + " | ".join(hdr) + " |", "|" + "---|" * len(hdr)]
    order = sorted(agg, key=lambda k: -sum(dur[k].values()))
    for key in order:
        v = {c: sum(x) / len(x) for c, x in agg[key].items()}
        d = list(dur[key].values())
        us = sum(d) / len(d) / 1e3
        n = len(d) // len(csv_paths)
        row = [f"`{key[0]}`", str(key[1]), str(n), f"{us:.1f}"]
        if "GRBM_GUI_ACTIVE" in names:
            row.append(f"{v['GRBM_GUI_ACTIVE'] / 8 / (us * 1e3):.2f}" if "GRBM_GUI_ACTIVE" in v and us > 0 else "")
        for c in cols:
            row.append(f"{v[c]:.3f}" if c == "LdsBankConflict" else f"{v[c]:.1f}" if c in v else "")
        if unit:
            cyc = v.get("GRBM_GUI_ACTIVE", 0) / 8
            row.append(f"{100 * v['TA_BUSY_avr'] / cyc:.0f}" if cyc else "")
            row.append(f"{100 * v['TD_TD_BUSY_sum'] / 256 / cyc:.0f}" if cyc else "")
        for c in extra:
            row.append(f"{v[c]:.3g}" if c in v else "")
        lines.append("| " + " | ".join(row) + " |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mlp_role_flops(w):
    """Algorithmic FLOPs per step of each GEMM role of the MLP block's schedule (the shapes
    the library launches: GEMM1 and the activation-gradient product once over all rows,
    GEMM2 per chunk, the input-gradient product per dX chunk, both weight gradients)."""
    T, h, f, n1 = w.tokens, w.hidden, w.ffn_shard, w.n1
    return {
        "fwd_gemm1": 2.0 * T * h * n1,
        "fwd_gemm2": 2.0 * T * f * h,
        "dgrad_b": 2.0 * T * h * f,
        "dgrad_a": 2.0 * T * n1 * h,
        "wgrad_b": 2.0 * T * f * h,
        "wgrad_a": 2.0 * T * h * n1,
    }


def mlp_flops(w):
    fwd = 2.0 * w.tokens * w.hidden * w.n1 + 2.0 * w.tokens * w.ffn_shard * w.hidden
    return fwd, 3.0 * fwd


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, inp, reps, max_tokens=8192):
    """The oracle (numpy fp64) on this host: one rank's forward + backward over the first
    `max_tokens` tokens of the workload (the whole workload when smaller)."""
    import numpy as np

    import oracle

    rows = min(w.tokens, max_tokens)
    X, A, B, dY = (oracle.to_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    A0, B0 = oracle.mlp_shard_weights(A, B, w.act, w.n_partials, 0)
    A0, B0 = np.ascontiguousarray(A0), np.ascontiguousarray(B0)
    X, dY = np.ascontiguousarray(X[:rows]), np.ascontiguousarray(dY[:rows])
    total = 3.0 * (2.0 * rows * w.hidden * w.n1 + 2.0 * rows * w.ffn_shard * w.hidden)
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
    return {"value": total / best / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"one rank's full forward+backward of {w.name} over its first {rows} of {w.tokens} tokens "
                      f"(fp64 numpy), best of {done} reps, {best:.2f} s each"}


class StepTimer:
    """Times steps on `stream`: each step between two events, and (unless disabled) a
    read+write of a 1 GiB scratch buffer on the stream before it, outside the events.
    `comm` is the one reduction stream every workload of the run uses: streams are spread
    over the device's few hardware queues in creation order, and a reduction stream made
    per workload once landed on the compute stream's queue, which serialised the two (the
    GPT-3 6.7B stack measured after four other workloads: 8.76 instead of 8.17 ms)."""

    def __init__(self, stream, flush=True):
        import torch

        self.stream = stream
        self.comm = torch.cuda.Stream()
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0") if flush else None

    def flush(self):
        import torch

        if self.buf is not None:
            with torch.cuda.stream(self.stream):
                self.buf.add_(1.0)

    def run(self, fn, steps, warmup):
        """Mean ms per step over `steps` event-timed steps after `warmup` untimed ones."""
        import torch

        for _ in range(warmup):
            self.flush()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            self.flush()
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)
        self.last = {"median": t[len(t) // 2], "min": t[0], "max": t[-1]}
        return sum(t) / steps


def backtoback(fn, steps, warmup):
    """ms per step of `steps` steps issued back to back (wall clock between synchronisations)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def reduce_standalone_us(D, out, parts, rows, cols, ld, dtype, stream, reps):
    """shard_reduce of a [rows, cols] region alone on an idle GPU: µs per launch over
    back-to-back launches between one pair of events on their stream."""
    import torch

    for _ in range(3):
        D.shard_reduce(out, ld, parts, ld, rows, cols, dtype, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        D.shard_reduce(out, ld, parts, ld, rows, cols, dtype, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def dominant(per, kernel_of, role_flops, steps):
    """The GEMM kernel (one template instantiation, as the profiler names it) with the most
    time per step over every schedule role that launched it, and its rate."""
    by_kernel = {}
    for r, fl in role_flops.items():
        if fl > 0 and per[r][0] > 0:
            by_kernel.setdefault(kernel_of[r], []).append(r)
    dom = max(by_kernel, key=lambda k: sum(per[r][1] for r in by_kernel[k]))
    n_dom = sum(per[r][0] for r in by_kernel[dom])
    tot_ms = sum(per[r][1] for r in by_kernel[dom])
    flops = sum(role_flops[r] for r in by_kernel[dom]) * steps
    achieved = flops / (tot_ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": dom, "roles": by_kernel[dom], "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None, "avg_launch_us": round(tot_ms / max(1, n_dom) * 1e3, 2), "launches": n_dom,
            "flops_per_launch": flops / max(1, n_dom)}


def measure_mlp(w, args, timer, detail):
    """The MLP block's step figures for workload `w` (bf16)."""
    import torch

    import tensor_transformer_block_domino_amd as D
    from tensor_transformer_block_domino_amd.tp_sim import MlpGroup

    print(f"[bench] {w.name}: inputs and peer partials", file=sys.stderr, flush=True)
    inp = synth.mlp_inputs(w)
    g = MlpGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn_shard=w.ffn_shard, act=w.act, dtype=w.dtype,
                 row_chunks=w.row_chunks, col_chunks=w.col_chunks, n_partials=w.n_partials, X=inp["X"], A=inp["A"],
                 B=inp["B"], dY=inp["dY"], device=torch.device("cuda:0"))
    g.peer_forward()
    g.forward()
    g.peer_backward()
    torch.cuda.synchronize()
    compute = timer.stream
    comm = timer.comm

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

    ms = timer.run(step_domino, args.steps, args.warmup)
    spread = {k: round(v, 4) for k, v in timer.last.items()}
    print(f"[bench] {w.name}: domino step {ms:.3f} ms", file=sys.stderr, flush=True)
    ms_serial = timer.run(step_serial, args.steps, 2)
    ms_unsplit = timer.run(step_unsplit, args.steps, 2)
    print(f"[bench] {w.name}: serial {ms_serial:.3f} ms, unsplit without reduce {ms_unsplit:.3f} ms",
          file=sys.stderr, flush=True)
    parts = [g.Y_own[r] for r in g.ranks]
    red_us = reduce_standalone_us(D, g.Y, parts, w.tokens, w.hidden, w.hidden, D.DOMINO_BF16, compute,
                                  max(args.steps, 10))
    red_gbps = (w.n_partials + 1) * w.tokens * w.hidden * 2 / (red_us * 1e-6) / 1e9
    t_reduce_ms = 2 * red_us * 1e-3     # Y and dX, each [T, hidden], per step
    _, total_flops = mlp_flops(w)
    value = total_flops / (ms * 1e-3) / 1e12
    out = {
        "value": round(value, 2), "ms_per_step": round(ms, 4), "ms_per_step_spread": spread,
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "ffn_shard": w.ffn_shard, "act": w.act, "tp_partials": w.n_partials,
                   "split": f"rows x{w.row_chunks}, cols x{w.col_chunks}", "pass": "fwd+bwd"},
        "mfma_peak_frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "t_domino_ms": round(ms, 4), "t_serial_ms": round(ms_serial, 4),
        "t_unsplit_no_reduce_ms": round(ms_unsplit, 4),
        "t_reduce_standalone_ms": round(t_reduce_ms, 4),
        "hidden_fraction": round(1.0 - (ms - ms_unsplit) / t_reduce_ms, 3),
        "domino_over_serial": round(ms / ms_serial, 4),
        "domino_over_unsplit": round(ms / ms_unsplit, 4),
        "shard_reduce_GBps": round(red_gbps, 1),
        "shard_reduce_hbm_frac": round(red_gbps / HBM_PEAK_GBPS, 4),
        "shard_reduce_avg_us": round(red_us, 2),
    }
    if not detail:
        del g
        torch.cuda.empty_cache()
        return out, None
    out["t_domino_backtoback_ms"] = round(backtoback(step_domino, args.steps, 2), 4)
    out["t_graph_ms"] = round(graph_steps(step_domino, timer, args.steps), 4)
    # Per-kernel durations: the same Domino steps with the library's event timing on.
    D.domino_timing_enable(True)
    for _ in range(args.steps):
        timer.flush()
        step_domino()
    torch.cuda.synchronize()
    roles = ["reduce", "fwd_gemm1", "fwd_gemm2", "dgrad_b", "dgrad_a", "wgrad_b", "wgrad_a", "aux"]
    per = {r: D.domino_timing_read(r) for r in roles}
    kernel_of = {r: D.domino_timing_kernel(r) for r in roles}
    D.domino_timing_enable(False)
    rf = mlp_role_flops(w)
    gemm_ms_step = sum(per[k][1] for k in rf) / args.steps
    roof = dominant(per, kernel_of, rf, args.steps)
    roof["traffic"] = measured_traffic(roof["kernel"], w.name)
    out.update({
        "gemm_chain_tflops": round(total_flops / (gemm_ms_step * 1e-3) / 1e12, 2),
        "shard_reduce_in_step_GBps": round(2 * (w.n_partials + 1) * w.tokens * w.hidden * 2 /
                                           (per["reduce"][1] / args.steps * 1e-3) / 1e9, 1),
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()},
        "kernel_tflops": {r: round(rf[r] * args.steps / (per[r][1] * 1e-3) / 1e12, 1) for r in rf if per[r][1] > 0},
        "kernel_of_role": kernel_of,
        "roofline": roof,
    })
    return out, (g, inp)


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


def measure_attn(w, args, timer, detail):
    """The attention block's figures for workload `w`: its forward alone (Domino row chunks,
    each chunk's out-projection reduced on the second stream; the last reduction has no
    later work of the block to hide behind, so it is reported as exposed) and, with
    `detail`, the forward + backward step with per-kernel times and the roofline."""
    import torch

    import tensor_transformer_block_domino_amd as D
    from tensor_transformer_block_domino_amd.tp_sim import AttnGroup

    print(f"[bench] {w.name}: inputs and peer partials", file=sys.stderr, flush=True)
    inp = synth.attn_inputs(w)
    g = AttnGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                  row_chunks=w.row_chunks, n_partials=w.n_partials, X=inp["X"], Aqkv=inp["Aqkv"], Bo=inp["Bo"],
                  dY=inp["dY"] if detail else None, device=torch.device("cuda:0"))
    g.peer_forward()
    g.forward()
    if detail:
        g.peer_backward()
    torch.cuda.synchronize()
    compute = timer.stream
    comm = timer.comm

    # Forward alone.
    fl = attn_flops(w)
    fwd_flops = fl["qkv"] + fl["attn"] + fl["outproj"]
    ms_f = timer.run(lambda: g.forward(compute, comm), args.steps, args.warmup)
    ms_f_serial = timer.run(lambda: g.forward(compute, None, row_chunks=1), args.steps, 2)
    ms_f_unsplit = timer.run(lambda: g.forward(compute, None, rank_alone=True, row_chunks=1), args.steps, 2)
    ms_f_chunks = timer.run(lambda: g.forward(compute, None, rank_alone=True), args.steps, 2)
    print(f"[bench] {w.name}: forward domino {ms_f:.3f} ms, serial {ms_f_serial:.3f}, unsplit {ms_f_unsplit:.3f}",
          file=sys.stderr, flush=True)
    parts = [g.Y_own[r] for r in range(w.n_partials)]
    red_us = reduce_standalone_us(D, g.Y, parts, w.tokens, w.hidden, w.hidden, D.DOMINO_BF16, compute,
                                  max(args.steps, 10))
    out = {
        "forward": {
            "value": round(fwd_flops / (ms_f * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "t_domino_ms": round(ms_f, 4), "t_serial_ms": round(ms_f_serial, 4),
            "t_unsplit_no_reduce_ms": round(ms_f_unsplit, 4), "t_chunks_no_reduce_ms": round(ms_f_chunks, 4),
            "t_reduce_standalone_ms": round(red_us * 1e-3, 4),
            # The last chunk's reduction: what the Domino forward adds over its chunks alone.
            "exposed_last_reduce_ms": round(ms_f - ms_f_chunks, 4),
            "hidden_fraction": round(1.0 - (ms_f - ms_f_unsplit) / (red_us * 1e-3), 3),
            "domino_over_serial": round(ms_f / ms_f_serial, 4),
            "domino_over_unsplit": round(ms_f / ms_f_unsplit, 4),
            "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "heads_shard": w.heads_shard,
                       "head_dim": w.head_dim, "tp_partials": w.n_partials, "split": f"rows x{w.row_chunks}",
                       "pass": "fwd", "attention": "causal"},
        }
    }
    if not detail:
        del g
        torch.cuda.empty_cache()
        return out, None

    def step_domino():
        g.forward(compute, comm, no_join=1)
        g.backward(compute, comm)

    def step_unsplit():
        g.forward(compute, None, rank_alone=True, row_chunks=1)
        g.backward(compute, None, rank_alone=True, row_chunks=1)

    ms = timer.run(step_domino, args.steps, args.warmup)
    print(f"[bench] {w.name}: domino fwd+bwd step {ms:.3f} ms", file=sys.stderr, flush=True)
    ms_unsplit = timer.run(step_unsplit, args.steps, 2)
    D.domino_timing_enable(True)
    for _ in range(args.steps):
        timer.flush()
        step_domino()
    torch.cuda.synchronize()
    roles = list(fl) + ["reduce", "aux"]
    per = {r: D.domino_timing_read(r) for r in roles}
    kernel_of = {r: D.domino_timing_kernel(r) for r in roles}
    D.domino_timing_enable(False)
    total_flops = sum(fl.values())
    value = total_flops / (ms * 1e-3) / 1e12
    t_reduce_ms = 2 * red_us * 1e-3
    out.update({
        "value": round(value, 2), "ms_per_step": round(ms, 4),
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads_shard": w.heads_shard, "head_dim": w.head_dim, "tp_partials": w.n_partials,
                   "split": f"rows x{w.row_chunks}", "pass": "fwd+bwd", "attention": "causal"},
        "mfma_peak_frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "t_domino_ms": round(ms, 4),
        "t_unsplit_no_reduce_ms": round(ms_unsplit, 4),
        "t_reduce_standalone_ms": round(t_reduce_ms, 4),
        "hidden_fraction": round(1.0 - (ms - ms_unsplit) / t_reduce_ms, 3),
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()},
        "kernel_tflops": {r: round(fl[r] * args.steps / (per[r][1] * 1e-3) / 1e12, 1)
                          for r in fl if fl[r] > 0 and per[r][1] > 0},
        "kernel_of_role": kernel_of,
        "roofline": dominant(per, kernel_of, fl, args.steps),
    })
    return out, (g, inp)


def main_attn(args, w, timer):
    res, (g, inp) = measure_attn(w, args, timer, detail=True)
    out = headline(args, res)
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


def measure_layer(w, args, timer, detail):
    """The layer stack's step figures for workload `w`: Domino, serial and one-μ-batch
    steps, and with `detail` the graph replay, per-kernel times and the roofline."""
    import torch

    import tensor_transformer_block_domino_amd as D
    from tensor_transformer_block_domino_amd.tp_sim import LayerGroup

    print(f"[bench] {w.name}: generating the layer inputs", file=sys.stderr, flush=True)
    inp = synth.layer_inputs(w)
    g = LayerGroup(batch=w.batch, seq=w.seq, hidden=w.hidden, heads_shard=w.heads_shard, head_dim=w.head_dim,
                   ffn_shard=w.ffn_shard, act=w.act, row_chunks=w.row_chunks, n_partials=w.n_partials,
                   p_drop=w.p_drop, X=inp["X"], layers=inp["layers"], device=torch.device("cuda:0"))
    g.alloc_backward(inp["dY"])
    print("[bench] peer partials (the other ranks' work, once)", file=sys.stderr, flush=True)
    g.peer_forward()
    g.peer_backward()
    torch.cuda.synchronize()
    compute, comm = timer.stream, timer.comm

    def step_domino():
        g.forward(compute, comm)
        g.backward(compute, comm)

    def step_serial():
        g.forward(compute, None)
        g.backward(compute, None)

    def step_unsplit():
        g.forward(compute, comm, row_chunks=1)
        g.backward(compute, comm, row_chunks=1)

    ms = timer.run(step_domino, args.steps, args.warmup)
    print(f"[bench] {w.name}: domino step {ms:.3f} ms", file=sys.stderr, flush=True)
    ms_serial = timer.run(step_serial, args.steps, 2)
    ms_unsplit = timer.run(step_unsplit, args.steps, 2)
    fl = layer_flops(w)
    total_flops = sum(fl.values())
    value = total_flops / (ms * 1e-3) / 1e12
    res = {
        "value": round(value, 2), "ms_per_step": round(ms, 4),
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads_shard": w.heads_shard, "head_dim": w.head_dim, "ffn_shard": w.ffn_shard, "act": w.act,
                   "layers": w.layers, "p_drop": w.p_drop, "tp_partials": w.n_partials,
                   "split": f"rows x{w.row_chunks} (mu-batches)", "pass": "fwd+bwd"},
        "mfma_peak_frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "t_domino_ms": round(ms, 4),
        "t_serial_ms": round(ms_serial, 4),
        "t_unsplit_ms": round(ms_unsplit, 4),
        "domino_over_serial": round(ms / ms_serial, 4),
    }
    if detail:
        res["t_graph_ms"] = round(graph_steps(step_domino, timer, args.steps), 4)
        D.domino_timing_enable(True)
        for _ in range(args.steps):
            timer.flush()
            step_domino()
        torch.cuda.synchronize()
        roles = list(fl) + ["reduce", "aux", "group_fwd", "group_bwd"]
        per = {r: D.domino_timing_read(r) for r in roles}
        kernel_of = {r: D.domino_timing_kernel(r) for r in roles}
        D.domino_timing_enable(False)
        res.update({
            "t_reduce_in_step_ms": round(per["reduce"][1] / args.steps, 4),
            "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in per.items()},
            "kernel_tflops": {r: round(fl[r] * args.steps / (per[r][1] * 1e-3) / 1e12, 1)
                              for r in fl if fl[r] > 0 and per[r][1] > 0},
            "kernel_of_role": kernel_of,
            "roofline": dominant(per, kernel_of, fl, args.steps),
        })
    return res, (g, inp)


def main_layer(args, w, timer):
    res, (g, inp) = measure_layer(w, args, timer, detail=True)
    out = headline(args, res)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_layer(w, inp)
    print(json.dumps(out), flush=True)


def graph_steps(fn, timer, steps):
    """The step captured once into a HIP graph on the timer's stream and replayed: ms per
    replay (timed like the eager steps)."""
    import torch

    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=timer.stream):
        fn()
    torch.cuda.synchronize()

    def replay():
        with torch.cuda.stream(timer.stream):   # replay() launches on the current stream
            graph.replay()

    return timer.run(replay, steps, 2)


def headline(args, res):
    """The JSON line's fixed keys, then the workload's figures."""
    out = {
        "metric": METRIC, "value": res.pop("value"), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": res.pop("config"),
        "timing": ("mean of per-step HIP-event times on the compute stream; a 1 GiB scratch read+write before "
                   "each step, outside the events" if not args.no_flush else
                   "mean of per-step HIP-event times on the compute stream, steps back to back"),
    }
    out.update(res)
    return out


def main():
    args = parse()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary, workgroups=args.traffic_workgroups)
    if args.trace_summary:
        return trace_summary(*args.trace_summary, args.trace_command)
    if args.counter_summary:
        return counter_summary(args.counter_summary[0], args.counter_summary[1], args.trace_command,
                               *args.counter_summary[2:])
    if args.timeline_summary:
        return timeline_summary(*args.timeline_summary, args.trace_command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported: the library sums the "
              f"tensor-parallel partials on one GPU, with no collective between GPUs", file=sys.stderr)
        sys.exit(2)
    import torch

    import tensor_transformer_block_domino_amd as D

    D.load()
    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    timer = StepTimer(torch.cuda.Stream(), flush=not args.no_flush)
    w = synth.WORKLOADS[args.workload]
    if isinstance(w, synth.AttnWorkload):
        return main_attn(args, w, timer)
    if isinstance(w, synth.LayerWorkload):
        return main_layer(args, w, timer)
    assert isinstance(w, synth.MlpWorkload) and w.dtype == "bf16"
    res, (g, inp) = measure_mlp(w, args, timer, detail=True)
    out = headline(args, res)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_reps)
    del g
    torch.cuda.empty_cache()
    also = args.also if args.also is not None else (DEFAULT_ALSO if args.workload == DEFAULT_WORKLOAD else "none")
    others = {}
    for name in [n for n in also.split(",") if n and n != "none"]:
        ow = synth.WORKLOADS[name]
        if isinstance(ow, synth.MlpWorkload):
            others[name] = measure_mlp(ow, args, timer, detail=False)[0]
        elif isinstance(ow, synth.AttnWorkload):
            others[name] = measure_attn(ow, args, timer, detail=False)[0]["forward"]
        elif isinstance(ow, synth.LayerWorkload):
            others[name] = measure_layer(ow, args, timer, detail=False)[0]
        torch.cuda.empty_cache()
    if others:
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
