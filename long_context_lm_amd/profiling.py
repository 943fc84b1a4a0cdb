"""Turn rocprofv3 output for the GCA benchmark step into the summaries kept under profiles/.

Two kinds of run, each its own process under rocprofv3 (commands in the summaries):

  kernel stats     rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- python3 bench.py
                   (the default benchmark command; its JSON line goes to BENCH_LOG)
  HBM traffic      rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o run --
                       python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-inference --copy-calibration
                   (then the same with WRITE_SIZE into DIR_W)

    python -m long_context_lm_amd.profiling stats DIR OUT.md BENCH_LOG COMMAND...
    python -m long_context_lm_amd.profiling traffic DIR_F DIR_W OUT.json COMMAND_F COMMAND_W

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
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/attend.hip", "csrc/retrieve.hip", "csrc/landmark.hip", "csrc/fetch.hip", "csrc/gca_api.hip",
                  "csrc/gca_device.hpp", "csrc/gca_internal.hpp"]
SHORT = ["score_topk", "topk_merge", "attend_fwd", "inverse_index", "bwd_query", "bwd_key", "score_grad",
         "lmk_query_grad", "lmk_key_grad", "fetch_chunks", "decode_tokens", "sw_fwd", "sw_bwd_query",
         "sw_bwd_key", "fused_fwd", "fused_bwd_query"]
COPY_BYTES = 1 << 30


def code_text(src: str) -> str:
    """The code of a C++/HIP source: comments removed and whitespace runs collapsed, so that an
    edit of comments or layout alone leaves it unchanged (the sources hold no string literal with
    a comment marker in it)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout excluded): profiles taken with
    another hash describe other kernels."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(kernel: str):
    # whole kernel names (with an optional variant suffix, e.g. attend_fwd_wave_kernel or the
    # two-wave fused_fwd2_kernel) only: "bwd_query" must not match sw_bwd_query_kernel
    for s in SHORT:
        if re.search(r"(?<![A-Za-z0-9_])" + s + r"[0-9]?(_[a-z]+)?_kernel\b", kernel):
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


def stats(directory: str, out_md: str, command: str, bench_log: str | None = None, warmup: int = 5,
          steps: int = 20) -> None:
    """Per-kernel durations of the timed training steps from the kernel trace: dispatches
    [warmup, warmup + steps) of each kernel in time order (the inference runs that follow are left
    out), next to the bench's own event-timed averages read from the JSON line of the same run."""
    per = {}
    for r in sorted(_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        s = short_name(r["Kernel_Name"])
        if s is None or s == "copy":
            continue
        per.setdefault(s, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    bench = {}
    if bench_log:
        with open(bench_log) as fh:
            line = [l for l in fh if l.startswith("{")][-1]
        res = json.loads(line)
        bench = {k: v["avg_ms"] * 1e3 for k, v in res["kernels"].items()}
        bench["_step_ms"] = res["ms_per_step"]
        bench["_dominant"] = res["roofline"]["kernel"]
    lines = [
        "# Kernel durations: GCA retrieve + forward + backward, 16K training workload",
        "",
        "Workload: B=8, L=16384 (256 chunks of 64), H=12, d=64, K=8, G=2, Gumbel top-k, bf16.",
        "",
        f"Command (repository root, on an MI355X): `{command}`",
        "",
        f"Kernel sources hash: `{source_hash()}`.  Trace columns: dispatches {warmup}..{warmup + steps - 1} of "
        "each kernel (the timed training steps; warm-up and the inference runs left out).  Last column: the "
        "average that bench.py itself measured with HIP events around each launch in the same run"
        + (f" (step {bench['_step_ms']:.3f} ms; roofline kernel `{bench['_dominant']}`)." if bench else "."),
        "",
        "| kernel | timed calls | trace average (us) | min (us) | max (us) | bench events average (us) |",
        "|---|---|---|---|---|---|",
    ]
    order = sorted(per, key=lambda k: -sum(per[k][warmup:warmup + steps]))
    if bench:  # only the kernels of the training step (not those that run only in inference)
        order = [k for k in order if k in bench]
    for k in order:
        d = per[k][warmup:warmup + steps] or per[k]
        ev = f"{bench[k]:.1f}" if k in bench else ""
        lines.append(f"| {k} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} | {ev} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def infer_stats(directory: str, out_md: str, command: str, bench_log: str) -> None:
    """Decode-step kernels of the same run (the 1M- and 16M-token history latency runs), one row
    per kernel and launch shape, next to the per-step latencies bench.py reported."""
    groups = {}
    for r in _rows(directory, "kernel_trace.csv"):
        s = short_name(r["Kernel_Name"])
        if s not in ("score_topk", "topk_merge", "attend_fwd", "fetch_chunks", "decode_tokens"):
            continue
        wg = int(r["Workgroup_Size_X"])
        blocks = int(r["Grid_Size_X"]) // wg
        groups.setdefault((s, blocks, wg), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    with open(bench_log) as fh:
        res = json.loads([l for l in fh if l.startswith("{")][-1])
    inf = res.get("inference_latency") or {}
    # launch shapes of the decode steps (G = 2 rows of one batch row, H = 12, K = 8)
    shapes = {("score_topk", 128, 256): "1M scan (2 rows x 64 blocks)", ("topk_merge", 2, 1024): "1M / 16M merge",
              ("score_topk", 512, 256): "16M scan (2 rows x 256 blocks)", ("attend_fwd", 48, 512): "1M / 16M attend (24 tiles x 2 halves)",
              ("fetch_chunks", 192, 256): "host-memory K/V fetch (2 groups x 8 slots x 12 heads, 3 MiB)",
              ("decode_tokens", 24, 512): "one-token decode, 16M history (2 groups x 12 heads)"}
    lines = [
        "# Kernel durations: one decode step over a 1M- / 16M-token history (retrieve + attend)",
        "",
        "Workload: B=1, G=2, H=12, d=64, K=8, one new 64-token chunk; history 16,384 / 262,144 chunks of bf16 K, V "
        "and landmarks resident in HBM.",
        "",
        f"Command (repository root, on an MI355X): `{command}`",
        "",
        f"Kernel sources hash: `{source_hash()}`.  All dispatches of each launch shape in the run (warm and "
        "cold repetitions, eager and graph replay).",
        "",
        "| kernel | launch (workgroups x threads) | workload | dispatches | average (us) | min (us) |",
        "|---|---|---|---|---|---|",
    ]
    for key in sorted(groups, key=lambda k: (k[0], k[1])):
        if key not in shapes:
            continue
        d = groups[key]
        lines.append(f"| {key[0]} | {key[1]} x {key[2]} | {shapes[key]} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} |")
    lines += ["", "Per-step latency measured by bench.py in the same run, under the profiler, whose per-dispatch "
              "overhead inflates these figures (HIP events around retrieve + forward; the unprofiled bench "
              "line carries the reported latencies):", "",
              "| history | warm median (us) | cold median (us) | graph replay warm (us) | graph replay cold (us) |",
              "|---|---|---|---|---|"]
    def cell(v, mode):
        return f"{v[mode]['median_us']:.1f}" if mode in v else "-"

    for label, v in inf.items():
        lines.append(f"| {label} | {cell(v, 'warm')} | {cell(v, 'cold')} | {cell(v, 'graph_warm')} | "
                     f"{cell(v, 'graph_cold')} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _copy_calibration(directory: str, counter: str):
    """Bytes per counter unit of the plain 1 GiB device copy bench.py --copy-calibration runs (the
    runtime's copyBuffer blit kernel; other copy-like kernels of the run, such as random-number
    fills of a long history, may move more data and must not be taken for it)."""
    blit, other = [], []
    for r in _rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        if "copyBuffer" in r["Kernel_Name"]:
            blit.append(float(r["Counter_Value"]))
        elif short_name(r["Kernel_Name"]) == "copy":
            other.append(float(r["Counter_Value"]))
    vals = blit or other
    if not vals:
        raise RuntimeError("the copy calibration kernel is missing from the counter runs")
    return COPY_BYTES / max(vals)


# Launch shapes of the decode-step kernels (G = 2 rows of one batch row, H = 12, K = 8).
DECODE_SHAPES = {("score_topk", 128, 256): "1M scan (2 rows x 64 blocks)",
                 ("score_topk", 512, 256): "16M scan (2 rows x 256 blocks)",
                 ("topk_merge", 2, 1024): "1M / 16M merge",
                 ("attend_fwd", 48, 512): "1M / 16M attend (24 tiles x 2 halves)",
                 ("fetch_chunks", 192, 256): "host-memory K/V fetch (2 groups x 8 slots x 12 heads)",
                 ("decode_tokens", 24, 512): "one-token decode, 16M history (2 groups x 12 heads)"}
# Algorithmic bytes per dispatch: landmarks scanned (G rows x history x 64 x 2 B) plus the query
# landmarks; the attend and fetch kernels read the retrieved K/V tiles (G x K x H x 2 x 8 KiB).
DECODE_BYTES = {"1M scan (2 rows x 64 blocks)": 2 * 16384 * 128 + 2 * 128,
                "16M scan (2 rows x 256 blocks)": 2 * 262144 * 128 + 2 * 128,
                "1M / 16M attend (24 tiles x 2 halves)": 2 * 8 * 12 * 2 * 8192 + 2 * 2 * 12 * 64 * 128,
                "host-memory K/V fetch (2 groups x 8 slots x 12 heads)": 2 * 8 * 12 * 2 * 8192,
                "one-token decode, 16M history (2 groups x 12 heads)": 2 * 8 * 12 * 2 * 8192}


def infer_traffic(dir_fetch: str, dir_write: str, out_md: str, commands) -> None:
    """FETCH_SIZE / WRITE_SIZE of the decode-step kernels per launch shape, scaled by the plain
    copy's readings, next to the algorithmic bytes of each launch."""
    def shape_values(directory, counter):
        per = {}
        for r in _rows(directory, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            k = short_name(r["Kernel_Name"])
            wg = int(r["Workgroup_Size"])
            key = (k, int(r["Grid_Size"]) // wg, wg)
            if key in DECODE_SHAPES:
                per.setdefault(DECODE_SHAPES[key], []).append(float(r["Counter_Value"]))
        return per, _copy_calibration(directory, counter)

    fetch, f_scale = shape_values(dir_fetch, "FETCH_SIZE")
    write, w_scale = shape_values(dir_write, "WRITE_SIZE")
    lines = [
        "# HBM traffic: decode-step kernels over 1M- and 16M-token histories",
        "",
        "Workload: B=1, G=2, H=12, d=64, K=8, one new 64-token chunk; bf16 K, V and landmarks in HBM "
        "(the fetch reads pinned host memory).",
        "",
        "Commands (repository root, on an MI355X): " + "; ".join(f"`{c}`" for c in commands),
        "",
        f"Kernel sources hash: `{source_hash()}`.  Per launch shape, the average over its dispatches of "
        f"FETCH_SIZE and WRITE_SIZE (KiB), scaled by what the counters read for a 1 GiB device copy "
        f"({f_scale:.0f} and {w_scale:.0f} bytes per KiB).  Repeated dispatches find their data in "
        "the caches, so the scans of a history that fits the MALL (1M) read less than once.",
        "",
        "| kernel launch | dispatches | fetched (MB) | written (MB) | algorithmic bytes read (MB) |",
        "|---|---|---|---|---|",
    ]
    for name in DECODE_SHAPES.values():
        if name not in fetch:
            continue
        f = sum(fetch[name]) / len(fetch[name]) * f_scale
        w = sum(write.get(name, [0.0])) / max(len(write.get(name, [])), 1) * w_scale
        alg = DECODE_BYTES.get(name)
        lines.append(f"| {name} | {len(fetch[name])} | {f / 1e6:.2f} | {w / 1e6:.3f} | "
                     + (f"{alg / 1e6:.2f}" if alg else "-") + " |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _per_kernel(directory: str, counter: str, warmup: int, steps: int):
    """Counter values per kernel, in dispatch order, of the timed training steps: dispatches
    [warmup, warmup + steps) of each kernel at the grid of its first dispatch (bench.py runs the
    training step first, one launch of each kernel per step).  Later runs at the same grid (the
    skewed-retrieval steps, whose hub lists change the key-major work) and at other launch shapes
    (the forward-only workload, the context-length sweep) are left out."""
    rows = []
    for r in _rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        s = short_name(r["Kernel_Name"])
        if s is None:
            continue
        rows.append((int(r["Dispatch_Id"]), s, int(r["Grid_Size"]), float(r["Counter_Value"])))
    per, grid = {}, {}
    for _did, s, g, v in sorted(rows):
        grid.setdefault(s, g)
        if s == "copy" or g == grid[s]:
            per.setdefault(s, []).append(v)
    return {s: (v if s == "copy" else v[warmup:warmup + steps]) for s, v in per.items()}


def traffic(dir_fetch: str, dir_write: str, out_json: str, commands, warmup: int = 1, steps: int = 2) -> None:
    fetch = _per_kernel(dir_fetch, "FETCH_SIZE", warmup, steps)
    write = _per_kernel(dir_write, "WRITE_SIZE", warmup, steps)
    # the calibration copy reads and writes COPY_BYTES
    f_scale = _copy_calibration(dir_fetch, "FETCH_SIZE")
    w_scale = _copy_calibration(dir_write, "WRITE_SIZE")
    out = {"source_hash": source_hash(), "fetch_bytes_per_kib": f_scale, "write_bytes_per_kib": w_scale,
           "copy_bytes": COPY_BYTES, "commands": commands,
           "dispatches": f"{warmup}..{warmup + steps - 1} of each kernel (the timed training steps)", "kernels": {}}
    for k in SHORT:
        if k in fetch and k in write:
            fk = sum(fetch[k]) / len(fetch[k])
            wk = sum(write[k]) / len(write[k])
            out["kernels"][k] = {"fetch_kib": fk, "write_kib": wk, "hbm_bytes": fk * f_scale + wk * w_scale}
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)


def counters(directory: str, out_md: str, command: str, warmup: int = 1, steps: int = 2, n_xcc: int = 8,
             n_simd: int = 1024) -> None:
    """Issue counters of the training step's attention kernels (one rocprofv3 --pmc pass): how busy
    the matrix cores were, how often a VALU instruction issued while they were busy, and the VALU
    and LDS activity, per dispatch of the timed steps (dispatches [warmup, warmup + steps))."""
    dur = {}  # dispatch id -> duration (us), from the kernel trace of the same run
    try:
        for r in _rows(directory, "kernel_trace.csv"):
            dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    except FileNotFoundError:
        pass
    per = {}
    for r in _rows(directory, "counter_collection.csv"):
        k = short_name(r["Kernel_Name"])
        if k not in ("attend_fwd", "bwd_query", "bwd_key"):
            continue
        did = int(r["Dispatch_Id"])
        us = dur.get(did, 0.0)
        if not us and "End_Timestamp" in r:
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        e = per.setdefault(k, {}).setdefault(did, {"us": us, "grid": int(r["Grid_Size"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = [
        "# Issue counters: attention kernels of the GCA training step (16K workload)",
        "",
        "Workload: B=8, L=16384 (256 chunks of 64), H=12, d=64, K=8, G=2, Gumbel top-k, bf16.",
        "",
        f"Command (repository root, on an MI355X): `{command}`",
        "",
        f"Kernel sources hash: `{source_hash()}`.  Dispatches {warmup}..{warmup + steps - 1} of each kernel "
        "(the timed steps).  Cycles = GRBM_GUI_ACTIVE / 8 XCDs.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
        "(cycles x 1024 SIMDs).  Co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (share of "
        "matrix-busy cycles in which a VALU instruction also issued).  VALU and MFMA instructions are per "
        "SIMD per 1,000 cycles.  LDS active = SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs).",
        "",
        "| kernel | duration (us) | cycles | clock (GHz) | MFMA busy | co-issue | VALU instr. / kcycle / SIMD | "
        "MFMA instr. / kcycle / SIMD | LDS active |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for k in ("attend_fwd", "bwd_query", "bwd_key"):
        if k not in per:
            continue
        disp = [per[k][key] for key in sorted(per[k])][warmup:warmup + steps]
        if not disp:
            continue
        avg = {c: sum(x.get(c, 0.0) for x in disp) / len(disp) for c in disp[0] if c != "grid"}
        cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / n_xcc
        if cyc <= 0:
            continue
        busy = avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        co = avg.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0)
        lines.append(
            f"| {k} | {avg['us']:.1f} | {cyc:.0f} | {cyc / (avg['us'] * 1e3):.2f} | {busy / (cyc * n_simd):.1%} | "
            f"{(co / busy if busy else 0):.1%} | {1e3 * avg.get('SQ_INSTS_VALU', 0) / (cyc * n_simd):.0f} | "
            f"{1e3 * avg.get('SQ_INSTS_MFMA', 0) / (cyc * n_simd):.1f} | "
            f"{avg.get('SQ_LDS_IDX_ACTIVE', 0) / (cyc * (n_simd // 4)):.1%} |")
    lines += ["", "Every dispatch of these kernels at the training shape in the run (warm-up, timed and "
              "single-step runs): the cycle count stays nearly fixed while the duration follows the shader "
              "clock.", "",
              "| kernel | dispatch | duration (us) | cycles | clock (GHz) |", "|---|---|---|---|---|"]
    for k in ("attend_fwd", "bwd_query", "bwd_key"):
        ids = sorted(per.get(k, {}))
        if not ids:
            continue
        grid = per[k][ids[0]]["grid"]
        for did in ids:
            e = per[k][did]
            if e["grid"] != grid:
                continue
            cyc = e.get("GRBM_GUI_ACTIVE", 0.0) / n_xcc
            if e["us"] > 0 and cyc > 0:
                lines.append(f"| {k} | {did} | {e['us']:.1f} | {cyc:.0f} | {cyc / (e['us'] * 1e3):.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "stats":  # stats DIR OUT.md BENCH_LOG COMMAND...
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[5:]) or "see long_context_lm_amd/profiling.py",
              bench_log=sys.argv[4])
    elif what == "infer":  # infer DIR OUT.md BENCH_LOG COMMAND...
        infer_stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[5:]), sys.argv[4])
    elif what == "infer-traffic":  # infer-traffic DIR_F DIR_W OUT.md COMMAND_F COMMAND_W
        infer_traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    elif what == "counters":  # counters DIR OUT.md COMMAND...
        counters(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif what == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    else:
        raise SystemExit(__doc__)
