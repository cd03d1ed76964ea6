"""Launches for hardware-counter runs of the two hot kernels.

Run under a counter profiler, for example

    rocprofv3 --pmc FETCH_SIZE -- python3 traffic.py

It launches, on synthetic inputs already resident on the GPU:
  * a plain device-to-device copy of 256 MiB (``copy``), the calibration of
    the byte counters against a transfer of known size;
  * the lm-head verify GEMM, hidden [192, 4096] x W [4096, 151936] bf16 ->
    fp32 (``lmhead``), with W packed in the MFMA operand order (the form the
    benchmark times) and then from W as stored;
  * the accept/reject pass at B=64, K=7, V=128256 bf16 (``accept``).
Each is launched ``--reps`` times after one warm-up.  ``summarize`` turns the
profiler's counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run into
per-launch bytes.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

COPY_BYTES = 256 << 20
ROOT = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.join(ROOT, "speculative_decoding_verification_accept_amd")


def source_digest() -> str:
    """SHA-256 over the HIP sources and header the counters describe."""
    h = hashlib.sha256()
    for rel in ("csrc/spec_verify_linear.hip", "csrc/spec_verify_linear_packed.hip", "csrc/spec_accept.hip",
                "csrc/device_common.hpp", "csrc/philox.hpp", "../include/spec_verify.h"):
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def run(which, reps):
    import torch

    import speculative_decoding_verification_accept_amd as sv
    from speculative_decoding_verification_accept_amd import workloads
    sv.load_library()
    dev = torch.device("cuda:0")
    if "copy" in which:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(reps + 1):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if "lmhead" in which:
        M, H, V = 192, workloads.HIDDEN, workloads.LMHEAD_N
        X, W = workloads.linear_inputs(M, H, V, seed=5, device=dev)
        Y = torch.empty(M, V, dtype=torch.float32, device=dev)
        # the benchmark's form: W packed once in the MFMA operand order
        Wp = sv.pack_weight(W)
        need = sv.linear_packed_workspace_bytes(M, V, H)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        for _ in range(reps + 1):
            sv.verify_linear_packed(X, Wp, V, out=Y, workspace=ws)
        torch.cuda.synchronize()
        # and from W as stored
        need = sv.linear_workspace_bytes(M, V, H)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        for _ in range(reps + 1):
            sv.verify_linear(X, W, out=Y, workspace=ws)
        torch.cuda.synchronize()
        del X, W, Wp, Y, ws
    if "accept" in which:
        z, q, x, L = workloads.large_accept_device(3000, dev)
        ws = sv.accept_workspace(64, 7, 128256, dev)
        for r in range(reps + 1):
            sv.accept(z, q, x, L, temperature=0.8, seed=77, offset=r, workspace=ws)
        torch.cuda.synchronize()


def _per_launch(path):
    """Mean counter value per (kernel name, grid size): one entry per kind of launch."""
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size"]))
            vals.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in vals.items()}


def _short(name):
    """Kernel name without namespaces and argument list."""
    name = re.sub(r"specv::\(anonymous namespace\)::", "", name)
    name = re.sub(r"^void ", "", name)
    depth, out = 0, []
    for ch in name:  # drop the parameter list: the first '(' at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).strip()


def _sum_kib(table, needles):
    return sum(mean for (name, _), (mean, _n) in table.items() if any(n in name for n in needles))


def summarize(fetch_csv, write_csv):
    """HBM bytes per call of each hot path, the counters scaled by what they
    read for the copy of known size (FETCH_SIZE and WRITE_SIZE in KiB)."""
    fetch, write = _per_launch(fetch_csv), _per_launch(write_csv)
    cf = _sum_kib({k: v for k, v in fetch.items() if "copyBuffer" in k[0] and v[0] * 1024 > COPY_BYTES / 4},
                  ["copyBuffer"])
    cw = _sum_kib({k: v for k, v in write.items() if "copyBuffer" in k[0] and v[0] * 1024 > COPY_BYTES / 4},
                  ["copyBuffer"])
    kf, kw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    res = {"copy_bytes": COPY_BYTES, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": kf, "write_scale": kw, "launches": {}, "calls": {}}
    for (name, grid), (mean, n) in sorted(fetch.items()):
        if "specv" in name:
            w = write.get((name, grid), (0.0, 0))[0]
            res["launches"][f"{_short(name)} grid={grid}"] = {
                "dispatches": n, "fetch_kib": mean, "write_kib": w,
                "bytes": mean * 1024 * kf + w * 1024 * kw}
    for call, needles in (("lmhead", ("k_packed",)), ("lmhead_stored_w", ("k_dma", "k_reduce", "k_tile", "k_strip")),
                          ("accept", ("k_accept",))):
        f, w = _sum_kib(fetch, needles), _sum_kib(write, needles)
        res["calls"][call] = {"fetch_bytes": f * 1024 * kf, "write_bytes": w * 1024 * kw,
                              "bytes": f * 1024 * kf + w * 1024 * kw}
    return res


def markdown(res, command):
    """The committed summary: figures, the commands, and a machine-readable line."""
    lines = ["# HBM traffic per call: lm-head verify GEMM and accept pass at scale", "",
             "Counters: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over all L2 channels),",
             "one profiler pass each, scaled by what they read for a device-to-device copy of",
             f"{res['copy_bytes'] >> 20} MiB in the same process "
             f"(FETCH_SIZE read {res['copy_fetch_kib']:.0f} KiB -> x{res['fetch_scale']:.4f}; "
             f"WRITE_SIZE read {res['copy_write_kib']:.0f} KiB -> x{res['write_scale']:.4f}).", "",
             "Commands (repository root as $REPO, on one MI355X):", "", "```", command, "```", "",
             "| launch | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes |", "|---|---|---|---|---|"]
    for k, v in res["launches"].items():
        lines.append(f"| `{k}` | {v['dispatches']} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | {v['bytes']:.4g} |")
    lines += ["", "| call | fetched bytes | written bytes | total |", "|---|---|---|---|"]
    for k, v in res["calls"].items():
        lines.append(f"| {k} | {v['fetch_bytes']:.4g} | {v['write_bytes']:.4g} | {v['bytes']:.4g} |")
    lines += ["", "Machine-readable (bench.py reports `traffic` from it while the sources still",
              "hash to this digest):", "",
              "traffic: " + json.dumps({"source_sha256": source_digest(),
                                         "lmhead_bytes": round(res["calls"]["lmhead"]["bytes"]),
                                         "accept_bytes": round(res["calls"]["accept"]["bytes"])})]
    return "\n".join(lines) + "\n"


def kernel_stats(trace_csv, top=24):
    """Markdown table of kernel durations from a rocprofv3 --kernel-trace CSV,
    one row per (kernel, grid size): the library's kernels split by launch
    shape (the lm-head product runs as whole tiles, then a K-split tail)."""
    groups = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            key = (_short(r["Kernel_Name"]), grid if "specv" in r["Kernel_Name"] else None)
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            groups.setdefault(key, []).append(d)
    total = sum(sum(v) for v in groups.values())
    lines = ["| kernel | grid (threads) | calls | avg us | median us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]:
        ds = sorted(ds)
        lines.append(f"| `{name[:90]}` | {grid if grid is not None else '-'} | {len(ds)} | "
                     f"{sum(ds) / len(ds):.2f} | {ds[len(ds) // 2]:.2f} | {ds[0]:.2f} | {ds[-1]:.2f} | "
                     f"{100 * sum(ds) / total:.2f} |")
    return "\n".join(lines) + "\n"


def read_committed(path):
    """The traffic figures of a committed summary if they describe the current
    sources, else None."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("traffic: "):
                    d = json.loads(line[len("traffic: "):])
                    return d if d.get("source_sha256") == source_digest() else None
    except OSError:
        return None
    return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--which", default="copy,lmhead,accept")
    ap.add_argument("--digest", action="store_true", help="print the source digest and exit")
    ap.add_argument("--summarize", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the markdown summary of two counter runs to stdout")
    ap.add_argument("--command", default="", help="the profiling commands, quoted in the summary")
    ap.add_argument("--kernel-stats", metavar="TRACE_CSV",
                    help="print a table of kernel durations from a --kernel-trace CSV")
    args = ap.parse_args(argv)
    if args.digest:
        print(source_digest())
        return
    if args.kernel_stats:
        print(kernel_stats(args.kernel_stats), end="")
        return
    if args.summarize:
        print(markdown(summarize(*args.summarize), args.command), end="")
        return
    run(args.which.split(","), args.reps)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main()
