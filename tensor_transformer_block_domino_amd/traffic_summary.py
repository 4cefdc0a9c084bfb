"""Writes the HBM-traffic summary of a kernel from two rocprofv3 counter runs of the bench
command (one FETCH_SIZE, one WRITE_SIZE), each calibrated against the plain device copy the
bench runs first (--calibration-copy-mib): the counter value per KiB actually moved.

  python -m tensor_transformer_block_domino_amd.traffic_summary FETCH.csv WRITE.csv KERNEL COPY_MIB OUT.txt

The summary records the sha256 of the GEMM source it was taken with; bench.py reports the
traffic only while that source is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys

GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm_bf16.hip")


def _values(path, counter):
    out = {}
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] == counter:
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def _match(values, kernel):
    hits = [v for name, vs in values.items() if name.split("(domino")[0].replace("domino::(anonymous namespace)::", "")
            .replace("void ", "").strip().startswith(kernel.replace("(domino::Epi)", "(Epi)")) for v in vs]
    if not hits:
        hits = [v for name, vs in values.items() if kernel.split("<")[0] in name and
                kernel.split("<")[1].split(",")[:5] == name.split("<")[1].split(",")[:5] for v in vs]
    return hits


def main(fetch_csv, write_csv, kernel, copy_mib, out_path):
    copy_kib = float(copy_mib) * 1024
    fetch, write = _values(fetch_csv, "FETCH_SIZE"), _values(write_csv, "WRITE_SIZE")
    f_copy = sum(fetch["__amd_rocclr_copyBuffer"]) / len(fetch["__amd_rocclr_copyBuffer"])
    w_copy = sum(write["__amd_rocclr_copyBuffer"]) / len(write["__amd_rocclr_copyBuffer"])
    fs, ws = copy_kib / f_copy, copy_kib / w_copy
    fk, wk = _match(fetch, kernel), _match(write, kernel)
    if not fk or not wk:
        raise SystemExit(f"kernel {kernel} not found in the counter files")
    f_avg, w_avg = sum(fk) / len(fk), sum(wk) / len(wk)
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    lines = [
        f"kernel: {kernel}",
        f"kernel_source_sha256: {sha}",
        f"fetch_kib_per_launch: {f_avg:.1f}",
        f"write_kib_per_launch: {w_avg:.1f}",
        f"fetch_scale: {fs:.4f}",
        f"write_scale: {ws:.4f}",
        f"calibrated_bytes_per_launch: {int(round((f_avg * fs + w_avg * ws) * 1024))}",
        f"# {len(fk)} dispatches averaged; the {copy_mib} MiB copy read FETCH_SIZE {f_copy:.0f} KiB and "
        f"WRITE_SIZE {w_copy:.0f} KiB for {copy_kib:.0f} KiB moved each way.",
    ]
    header = [
        f"# HBM traffic of {kernel} in the bench command's step",
        "# (default workload: GPT-3 2.7B-shaped MLP shard, tokens 8192, hidden 2560, ffn_shard 1280, TP 8, rows x2).",
        "# Two rocprofv3 counter runs of the bench command, one counter each, then this summary:",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o fetch -- python3 bench.py --no-cpu-baseline "
        f"--steps 5 --warmup 1 --calibration-copy-mib {copy_mib}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o write -- python3 bench.py --no-cpu-baseline "
        f"--steps 5 --warmup 1 --calibration-copy-mib {copy_mib}",
        "#   python -m tensor_transformer_block_domino_amd.traffic_summary <dir>/fetch_counter_collection.csv "
        f"<dir>/write_counter_collection.csv '{kernel}' {copy_mib} <this file>",
    ]
    tail = [l.rstrip("\n") for l in open(out_path) if l.startswith("algorithmic") or l.startswith("# algorithmic")
            or l.startswith("# for the other") or l.startswith("# above")] if os.path.exists(out_path) else []
    with open(out_path, "w") as f:
        f.write("\n".join(header + lines + tail) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main(*sys.argv[1:6])
