"""Build the GCA HIP library (libgca.so) in-tree for gfx950.

    python -m long_context_lm_amd.build        # compiles every source, always

Objects go to ``_build/`` at the repository root; the shared library lands next to this file
so that it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/retrieve.hip", "csrc/attend.hip", "csrc/landmark.hip", "csrc/fetch.hip", "csrc/gca_api.hip"]
# Per-file device flags.  The attention kernels never produce or test NaN (inputs are finite,
# masked values are -inf), so fmax needs no NaN quieting there; infinities stay honoured.  The
# retrieval kernels keep strict IEEE semantics for their bit-exact scores.
FILE_FLAGS = {"csrc/attend.hip": ["-Xarch_device", "-fno-honor-nans"]}
LIB = os.path.join(HERE, "libgca.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep matrix-core accumulators in ordinary VGPRs: the softmax reads them right away, and
    # the AGPR form costs a v_accvgpr_read per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the GCA library)")


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return src, r.returncode, err


# Files whose kernels copy tiles into LDS with copy16_async_untracked (gca_device.hpp) and wait
# for those copies with counted vmcnt waits.  The counts assume that the only vector memory
# operations in flight are the ones the kernel issued itself.  Compiler-issued ones would make a
# counted wait release before the copy it guards: scratch spills and reloads, flat instructions
# (LDS or global memory reached through generic pointers count in vmcnt too), or memory
# instructions inside a called function.  guard_untracked_copies() fails the build if the device
# code of these files contains any of them.
UNTRACKED_COPY_SOURCES = ["csrc/attend.hip", "csrc/retrieve.hip"]
_MEMORY_OPS = ("global_", "flat_", "scratch_", "buffer_", "ds_", "s_load", "s_buffer", "s_store")


def _device_asm(src: str) -> str:
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(HERE, src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device assembly of {src} failed:\n{r.stderr}")
    return r.stdout


def untracked_copy_violations(asm: str) -> list[str]:
    """Reasons the counted waits of this device assembly could be wrong (empty list: none)."""
    bad = []
    kernel = None
    for line in asm.splitlines():
        t = line.strip()
        if t.startswith(".amdhsa_kernel "):
            kernel = t.split()[1]
        elif t.startswith(".end_amdhsa_kernel"):
            kernel = None
        elif kernel and t.startswith(".amdhsa_private_segment_fixed_size") and t.split()[1] != "0":
            bad.append(f"{kernel}: uses scratch ({t.split()[1]} bytes per lane)")
        elif kernel and t.startswith(".amdhsa_uses_dynamic_stack") and t.split()[1] != "0":
            bad.append(f"{kernel}: dynamic stack")
    # instructions, by function; functions other than kernels are callees
    kernels = set()
    for line in asm.splitlines():
        t = line.strip()
        if t.startswith(".amdhsa_kernel "):
            kernels.add(t.split()[1])
    fn = None
    for line in asm.splitlines():
        label = re.match(r"([A-Za-z_][\w$]*):", line)
        if label:
            fn = label.group(1)
            continue
        if fn is None or not line.startswith("\t") or line.lstrip().startswith((";", ".")):
            continue
        op = line.split()[0] if line.split() else ""
        if op.startswith("flat_"):
            bad.append(f"{fn}: flat instruction {op}")
        elif fn not in kernels and op.startswith(_MEMORY_OPS):
            bad.append(f"{fn} (called from a kernel): memory instruction {op}")
    return sorted(set(bad))


def loop_vmcnt_waits(asm: str) -> list[str]:
    """Compiler-placed vmcnt waits in the matrix-core blocks of loops (empty list: none).

    A vmcnt wait counts the untracked prefetch copies too, so one that the compiler places
    inside a pipelined loop (typically for a value loaded before the loop, at its first use)
    runs in every iteration and waits for the next tile's copies: the prefetch is lost.  Waits
    written in the kernels' inline assembly are the counted ones and are not reported, nor is
    the wait of a workgroup barrier (followed by s_barrier).  Only functions that issue copies
    from inline assembly are checked (a kernel whose copies the compiler tracks needs its waits)."""
    bad = []
    fn = block = None
    in_loop = in_asm = False
    pending = []  # (block, wait) of the current block, reported if the block issues a product
    mfma = False
    found = []  # (function, block, wait) candidates
    untracked = set()  # functions with copies issued from inline assembly

    def flush():
        if mfma and in_loop:
            found.extend((fn, b, w) for b, w in pending)

    lines = asm.splitlines()
    for n, line in enumerate(lines):
        t = line.strip()
        func = re.match(r"([A-Za-z_][\w$]*):", line)
        blk = re.match(r"(\.LBB\d+_\d+):(.*)", line)
        if func or blk:
            flush()
            pending, mfma = [], False
            if func:
                fn, block, in_loop = func.group(1), "entry", False
            else:
                block, in_loop = blk.group(1), "Loop" in blk.group(2)
            continue
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm and t.startswith("global_load_lds"):
            untracked.add(fn)
        elif t.startswith("v_mfma"):
            mfma = True
        elif t.startswith("s_waitcnt") and "vmcnt" in t and not in_asm:
            nxt = next((x.strip() for x in lines[n + 1:] if x.strip() and not x.strip().startswith(";")), "")
            if not nxt.startswith("s_barrier"):
                pending.append((block, t.split(";")[0].strip()))
    flush()
    bad = [f"{f} {b}: {w}" for f, b, w in found if f in untracked]
    return sorted(set(bad))


def guard_untracked_copies() -> None:
    """Fail if a file using untracked LDS copies compiles to code that breaks their waits, or
    that waits for them by accident inside a pipelined loop."""
    bad = []
    for src in UNTRACKED_COPY_SOURCES:
        asm = _device_asm(src)
        bad += [f"{src}: {b}" for b in untracked_copy_violations(asm)]
        bad += [f"{src}: compiler vmcnt wait in a loop: {b}" for b in loop_vmcnt_waits(asm)]
    if bad:
        raise RuntimeError("untracked LDS copies with compiler-issued memory operations:\n  " + "\n  ".join(bad))


def build(verbose: bool = True) -> str:
    """Compile every source and link libgca.so; returns the library path."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.basename(s).replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 4)) as ex:
        guard = ex.submit(guard_untracked_copies)
        results = list(ex.map(_compile, SOURCES, objs))
        guard.result()
    failed = False
    for src, rc, err in results:
        if err.strip() and (verbose or rc != 0):
            print(f"[build] {src}:\n{err}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("GCA library compilation failed")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
