"""Turn rocprofv3 output for the GCA benchmark step into the summaries kept under profiles/.

Two kinds of run, each its own process under rocprofv3 (commands in the summaries):

  kernel stats     rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run --
                       python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-inference
  HBM traffic      rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o run --
                       python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-inference --copy-calibration
                   (then the same with WRITE_SIZE into DIR_W)

    python -m long_context_lm_amd.profiling stats DIR OUT.md
    python -m long_context_lm_amd.profiling traffic DIR_F DIR_W OUT.json

The traffic summary scales each kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the
bytes-per-KiB the same counter reads for a plain device copy of known size (torch copy_ of
1 GiB, run by bench.py --copy-calibration), and records a hash of the kernel sources so that
bench.py reports the traffic only while the kernels are unchanged.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/attend.hip", "csrc/retrieve.hip", "csrc/gca_device.hpp", "csrc/gca_internal.hpp"]
SHORT = ["score_topk", "topk_merge", "attend_fwd", "inverse_index", "bwd_query", "bwd_key", "score_grad"]
COPY_BYTES = 1 << 30


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(kernel: str):
    for s in SHORT:
        if s in kernel:
            return s
    if "copy" in kernel.lower() or "elementwise" in kernel.lower():
        return "copy"
    return None


def _rows(directory: str, suffix: str):
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def stats(directory: str, out_md: str, command: str, warmup: int = 2) -> None:
    """Per-kernel durations from the kernel trace, leaving out each kernel's first `warmup`
    dispatches (the benchmark's warm-up steps), plus rocprofv3's own all-dispatch statistics."""
    per = {}
    for r in sorted(_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        s = short_name(r["Kernel_Name"])
        if s is None or s == "copy":
            continue
        per.setdefault(s, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = _rows(directory, "kernel_stats.csv")
    allstat = {short_name(r["Name"]): r for r in rows if short_name(r["Name"]) not in (None, "copy")}
    lines = [
        "# Kernel durations: GCA retrieve + forward + backward, 16K training workload",
        "",
        "Workload: B=8, L=16384 (256 chunks of 64), H=12, d=64, K=8, G=2, Gumbel top-k, bf16.",
        "",
        f"Command (repository root, on an MI355X): `{command}`",
        "",
        f"Kernel sources hash: `{source_hash()}`.  Timed columns leave out each kernel's first "
        f"{warmup} dispatches (warm-up steps); the last columns are rocprofv3 --stats over all calls.",
        "",
        "| kernel | timed calls | average (us) | min (us) | max (us) | all calls | all-call average (us) |",
        "|---|---|---|---|---|---|---|",
    ]
    order = sorted(per, key=lambda k: -sum(per[k][warmup:] or per[k]))
    for k in order:
        d = per[k][warmup:] or per[k]
        a = allstat.get(k)
        lines.append(f"| {k} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} | "
                     f"{a['Calls'] if a else ''} | {float(a['AverageNs']) / 1e3 if a else 0:.1f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _per_kernel(directory: str, counter: str):
    per = {}
    for r in _rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        s = short_name(r["Kernel_Name"])
        if s is None:
            continue
        per.setdefault(s, []).append(float(r["Counter_Value"]))
    return per


def traffic(dir_fetch: str, dir_write: str, out_json: str, commands) -> None:
    fetch = _per_kernel(dir_fetch, "FETCH_SIZE")
    write = _per_kernel(dir_write, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise RuntimeError("the copy calibration kernel is missing from the counter runs")
    # the calibration copy reads and writes COPY_BYTES; use its largest dispatch
    f_scale = COPY_BYTES / max(fetch["copy"])
    w_scale = COPY_BYTES / max(write["copy"])
    out = {"source_hash": source_hash(), "fetch_bytes_per_kib": f_scale, "write_bytes_per_kib": w_scale,
           "copy_bytes": COPY_BYTES, "commands": commands, "kernels": {}}
    for k in SHORT:
        if k in fetch and k in write:
            fk = sum(fetch[k]) / len(fetch[k])
            wk = sum(write[k]) / len(write[k])
            out["kernels"][k] = {"fetch_kib": fk, "write_kib": wk, "hbm_bytes": fk * f_scale + wk * w_scale}
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]) or "see long_context_lm_amd/profiling.py")
    elif what == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    else:
        raise SystemExit(__doc__)
