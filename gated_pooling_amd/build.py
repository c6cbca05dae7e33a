"""Build libcsa.so (the HIP library) in-tree for gfx950.

    python -m gated_pooling_amd.build
    python -m gated_pooling_amd.build --resources OUT.md   # per-kernel resource report

Flags: -ffp-contract=off so only explicit fmas are fused (the fp32
evaluation order is fixed); packed fp32 instructions are disabled.

--resources compiles the kernels once more for the device only with the
compiler's kernel-resource-usage remarks and writes, for every kernel
instance, its VGPRs, AGPRs, SGPRs, scratch, spills, static LDS and the
occupancy the compiler derives from them (waves per SIMD).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa.so")
SOURCES = [os.path.join(CSRC, "csa_kernels.hip"), os.path.join(CSRC, "csa_api.cpp")]
HEADERS = [os.path.join(CSRC, "csa_launch.h"), os.path.join(CSRC, "csa_walk.h"), os.path.join(ROOT, "include", "csa.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


DEBUG_LIB = os.path.join(HERE, "libcsa_debug.so")


def build(verbose: bool = False, extra_flags=None, debug: bool = True) -> str:
    """Build libcsa.so and, with debug=True, next to it (in a second hipcc
    process running at the same time) libcsa_debug.so: the same library with
    -DCSA_DEBUG_OWNERSHIP, whose backward also counts the stores to every
    dkv/dscore element (used by tests/test_ownership_gpu.py only)."""
    jobs = [(LIB, [])] + ([(DEBUG_LIB, ["-DCSA_DEBUG_OWNERSHIP"])] if debug else [])
    procs = []
    for out, defs in jobs:
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, *FLAGS, *defs, *(extra_flags or []), "-o", tmp, *SOURCES]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    noise = "is not a recognized feature for this target"
    failed = []
    for out, tmp, pr in procs:
        _, stderr = pr.communicate()
        err = "\n".join(l for l in stderr.splitlines() if noise not in l)
        if pr.returncode != 0:
            failed.append(f"{os.path.basename(out)}: hipcc failed ({pr.returncode}):\n{err}")
            continue
        if verbose and err.strip():
            print(err, file=sys.stderr)
        os.replace(tmp, out)
    if failed:
        raise RuntimeError("\n".join(failed))
    return LIB


def resource_usage(extra_flags=None):
    """{demangled kernel name: {field: value}} from the compiler's
    kernel-resource-usage remarks on the device code of csa_kernels.hip."""
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], *(extra_flags or []), "--cuda-device-only",
               "-c", "-Rpass-analysis=kernel-resource-usage", "-o", os.path.join(tmp, "k.o"), SOURCES[0]]
        res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+(?:\[[^\]]*\])?): (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    names = list(kernels)
    import shutil
    filt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    dem = subprocess.run([filt], input="\n".join(names), capture_output=True, text=True).stdout.splitlines() \
        if filt else names
    return {(dem[i] if i < len(dem) else n): kernels[n] for i, n in enumerate(names)}


# Instances the standard workloads launch: ratio 2 / 4 at coff 2 and the
# ragged coff-1 pack (2 columns per lane, 256 threads, device-table (0) or
# argument-table (2) lookups, wave-uniform rows, forward prefetch 2, backward
# 3), every ratio-128 instance, the dAPE reduce and the segment scans.
LAUNCHED = [r"^fwd_kernel<(2, 2|4, [12]), 2, 256, [02], true, 2, false>$",
            r"^bwd_kernel<(2, 2|4, [12]), 2, 256, [02], true, 3, false>$",
            r"^(fwd|bwd)128_kernel<", r"^dape_reduce_kernel$", r"^seg_scan_kernel<"]


def write_resource_report(path, extra_flags=None):
    """Markdown table of the compiler's resource report for the launched
    instances (LAUNCHED), with the sources' digest."""
    import hashlib
    rows = resource_usage(extra_flags)
    cols = ["VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]", "VGPRs Spill", "SGPRs Spill",
            "LDS Size [bytes/block]", "Occupancy [waves/SIMD]"]
    h = hashlib.sha256()  # the same digest bench.py records with its counters
    for f in SOURCES + [os.path.join(CSRC, "csa_launch.h"), os.path.join(CSRC, "csa_walk.h")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    table = {}
    for name in rows:
        short = name.replace("csa::(anonymous namespace)::", "")
        short = short[short.find(" ") + 1:] if short.startswith("void ") else short
        short = re.sub(r"\(.*\)$", "", short)
        table[short] = rows[name]
    keep = sorted(k for k in table if any(re.search(p, k) for p in LAUNCHED))
    spills = [k for k in keep if table[k].get("VGPRs Spill", "0") != "0" or table[k].get("SGPRs Spill", "0") != "0"]
    with open(path, "w") as f:
        f.write("# Kernel resources (compiler report)\n\n"
                f"Sources sha256 {h.hexdigest()[:16]}. "
                "Command (no GPU needed):\n\n    python -m gated_pooling_amd.build --resources OUT.md\n\n"
                "The compiler's kernel-resource-usage remarks for the instances the workloads launch: the headline "
                "and ratio-2 packs (ratio, coff 2, 2 columns per lane, 256 threads, table kind 0 = device table or "
                "2 = kernel arguments, wave-uniform rows, forward prefetch 2 / backward 3), the ragged coff-1 pack, "
                "ratio 128 (<coff, table kind>), the dAPE reduce and the segment scans. LDS here is static LDS "
                "only (the ratio-128 backward's two window buffers are static); the launches add dynamic LDS (see "
                "the kernel traces). Occupancy is the compiler's bound from VGPRs and LDS; the launched grids use "
                "fewer waves per SIMD, and the measured average residency is in the *_occupancy.md files. "
                + ("No launched instance spills." if not spills else "Spills: " + ", ".join(spills) + ".")
                + "\n\n")
        f.write("| kernel instance | " + " | ".join(cols) + " |\n|" + "---|" * (len(cols) + 1) + "\n")
        for k in keep:
            f.write(f"| `{k}` | " + " | ".join(table[k].get(c, "") for c in cols) + " |\n")
        f.write(f"\n{len(table)} kernel instances are compiled in all; the launched ones are listed.\n")
    return path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--resources", metavar="OUT.md", help="write the per-kernel resource report and exit")
    a = ap.parse_args()
    if a.resources:
        print(write_resource_report(a.resources))
    else:
        print(build(verbose=True))
