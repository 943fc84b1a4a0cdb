"""Instruction-issue floors of the three attention kernels, counted from their gfx950 assembly.

    python -m long_context_lm_amd.issue_model

Compiles csrc/attend.hip to assembly with the library's own flags, finds each kernel's main loop
(the loop whose body holds the most matrix-core instructions, innermost on ties), counts its
instructions by class and prices them with per-instruction issue costs measured on an MI355X
with microbenchmarks (cycles of one SIMD per wave instruction, two or more waves per SIMD):

    float32 add / multiply / FMA                        2.9   (twice the rate of other VALU)
    other VALU (max3, convert, move, select, DPP, ...)  4.5
    transcendental (exp, log, reciprocal)               8.3
    v_mfma_f32_32x32x16_bf16                            33
    ds_read_b128 (CU's LDS, per wave instruction)       4.7
    ds_read_b64_tr_b16                                  3.45

Matrix-core and VALU time add up on a SIMD (measured), so a kernel's issue floor per wave and
slot is the sum of its priced instructions; the LDS figure is per CU.  Multiplied by the
(tile, slot) pairs per SIMD of a workload, these give the floors the measured cycle counts are
compared with.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from long_context_lm_amd import build as B

COST = {"fp32": 2.9, "valu": 4.5, "trans": 8.3, "mfma": 33.0}
LDS_COST = {"ds_read_b128": 4.7, "ds_read_b64_tr_b16": 3.45}
FP32 = {"v_fma_f32", "v_fmac_f32", "v_mul_f32", "v_add_f32", "v_sub_f32", "v_subrev_f32", "v_mac_f32"}
TRANS = {"v_exp_f32", "v_log_f32", "v_rcp_f32", "v_sqrt_f32", "v_rsq_f32"}
# kernel -> (fragment of its mangled name, matrix-core instructions per wave and slot, waves per pair)
KERNELS = {
    "attend_fwd": ("22attend_fwd_wave_kernelILb1E", 32, 1),   # one wave, 64 queries
    "bwd_query": ("16bwd_query_kernelINS_6bf16_tEE", 24, 2),  # two waves, 32 queries each
    "bwd_key": ("14bwd_key_kernelINS_6bf16_tEE", 32, 2),      # two waves, 32 keys each
}


def assemble() -> str:
    src = os.path.join(B.HERE, "csrc", "attend.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "attend.s")
        cmd = [B.hipcc(), *B.COMMON_FLAGS, *B.FILE_FLAGS.get("csrc/attend.hip", []), "--cuda-device-only",
               "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(r.stderr)
        with open(out) as fh:
            return fh.read()


def kernel_lines(asm: str, fragment: str) -> list[str]:
    lines = asm.splitlines()
    start = next(i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + re.escape(fragment) + r"\S*:", l))
    end = next(i for i in range(start, len(lines)) if lines[i].strip().startswith("s_endpgm"))
    return [l.split(";")[0].rstrip() for l in lines[start:end + 1]]


def main_loop(body: list[str]) -> list[str]:
    labels = {l[:-1]: i for i, l in enumerate(body) if re.match(r"^\.LBB\d+_\d+:$", l)}
    best = None
    for name, head in labels.items():
        back = [i for i in range(head + 1, len(body))
                if re.match(r"^\s*s_(cbranch_\w+|branch)\s+" + re.escape(name) + r"$", body[i])]
        if not back:
            continue
        span = body[head:back[-1] + 1]
        n = sum(1 for l in span if "v_mfma" in l)
        key = (n, -len(span))
        if best is None or key > best[0]:
            best = (key, span)
    if best is None:
        raise RuntimeError("no loop found")
    return best[1]


def classify(op: str) -> str | None:
    base = re.sub(r"_e(32|64)$", "", op)
    if base.startswith("v_mfma"):
        return "mfma"
    if base in TRANS:
        return "trans"
    if base in FP32:
        return "fp32"
    if base.startswith("v_"):
        return "valu"
    if base in LDS_COST:
        return base
    return None


def floors(asm: str | None = None) -> dict:
    asm = asm or assemble()
    res = {}
    for k, (frag, mfma_per_slot, waves) in KERNELS.items():
        loop = main_loop(kernel_lines(asm, frag))
        counts: dict[str, int] = {}
        for l in loop:
            parts = l.split()
            if not parts or parts[0].startswith("."):
                continue
            c = classify(parts[0])
            if c:
                counts[c] = counts.get(c, 0) + 1
        slots = counts.get("mfma", 0) / mfma_per_slot  # slots per loop iteration (unrolling)
        per = {c: n / slots for c, n in counts.items()}
        simd = sum(per.get(c, 0) * COST[c] for c in COST)
        lds = sum(per.get(c, 0) * LDS_COST[c] for c in LDS_COST)
        res[k] = {"slots_per_iteration": slots, "per_wave_slot": per, "simd_cycles_per_wave_slot": simd,
                  "simd_cycles_per_pair": simd * waves, "lds_cycles_per_pair": lds * waves, "waves": waves}
    return res


def main() -> None:
    pairs = 376  # (tile, slot) pairs per SIMD at the 16K, G=2 training step (384,768 over 1,024 SIMDs)
    r = floors()
    print("kernel       VALU fp32  VALU other  transc.  MFMA   SIMD cycles/pair  LDS cycles/pair (CU)  floor (Mcycles/SIMD)")
    for k, v in r.items():
        p = v["per_wave_slot"]
        print(f"{k:12s} {p.get('fp32', 0):9.0f} {p.get('valu', 0):11.0f} {p.get('trans', 0):8.0f} "
              f"{p.get('mfma', 0):5.0f} {v['simd_cycles_per_pair']:17.0f} {v['lds_cycles_per_pair']:21.0f} "
              f"{pairs * v['simd_cycles_per_pair'] / 1e6:21.3f}")
    print("(instruction counts per wave and slot; floors at 376 (tile, slot) pairs per SIMD)")


if __name__ == "__main__":
    sys.exit(main())
