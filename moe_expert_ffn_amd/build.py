"""Build the gfx950 HIP library libmegamoe.so in-tree with hipcc.

Run as ``python -m moe_expert_ffn_amd.build``.  Objects are compiled in
parallel into moe_expert_ffn_amd/_build and linked into
moe_expert_ffn_amd/libmegamoe.so.

The build also guards the grouped GEMM's register budget.  Its K loop issues
the global -> LDS copies from inline assembly, which the compiler's wait-count
pass does not see; any compiler-visible vector load that lands in the loop (a
spill reload, for instance) gets a wait that in hardware also waits for every
copy in flight and drains the copy ring.  Every instantiation of the GEMM
kernel must therefore compile with no spills and with no more registers than
recorded in GEMM_REGISTERS below; the build fails otherwise.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmegamoe.so")
# measurement probes (not part of the MegaMoE path): libmegamoe_probe.so
PROBE_SRC = os.path.join(CSRC, "probes")
PROBE_LIB = os.path.join(HERE, "libmegamoe_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # IEEE semantics for the rounding points the oracle checks bit for bit
    "-ffp-contract=off",
    # no packed fp32 instructions in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
# per-kernel register, spill and LDS report of the device compiler
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"

# Registers of each GEMM tile configuration, keyed by its template arguments
# (BM, WAVES_M, WAVES_N, NS, TRIM, SKIP, PRIO, NTB): (VGPRs, AGPRs).  The
# 256-row tiles run 16 waves per CU, so 128 registers per wave is the ceiling.
GEMM_REGISTERS = {
    (64, 1, 4, 3, 1, 1, 16, 1): (102, 92),
    (256, 4, 4, 4, 0, 1, 0, 0): (124, 0),
    (256, 4, 4, 4, 0, 1, 0, 1): (124, 0),
}


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIPFLAGS, RESOURCE_REMARKS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def kernel_resources(remarks: str) -> dict[str, dict[str, int]]:
    """Per-kernel figures from the compiler's kernel-resource-usage remarks."""
    out: dict[str, dict[str, int]] = {}
    cur = None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


def gemm_template_args(name: str):
    """(BM, WAVES_M, WAVES_N, NS, TRIM, SKIP, PRIO, NTB) of a mangled
    gmm_i8_ring_kernel instantiation, else None."""
    if "gmm_i8_ring_kernel" not in name:
        return None
    args = name.split("gmm_i8_ring_kernel", 1)[1]
    return tuple(int(v) for v in re.findall(r"L[ib](\d+)E", args))


def check_gemm_resources(remarks: str) -> list[str]:
    """Every GEMM instantiation: no spills, registers within the record."""
    problems = []
    found = 0
    for name, r in kernel_resources(remarks).items():
        key = gemm_template_args(name)
        if key is None:
            continue
        found += 1
        spills = r.get("VGPRs Spill", 0) + r.get("SGPRs Spill", 0)
        if spills:
            problems.append(f"GEMM {key}: {spills} spilled registers")
        rec = GEMM_REGISTERS.get(key)
        got = (r.get("VGPRs", 0), r.get("AGPRs", 0))
        if rec is None:
            problems.append(f"GEMM {key}: no register record (VGPRs {got[0]}, AGPRs {got[1]})")
        elif got[0] > rec[0] or got[1] > rec[1]:
            problems.append(f"GEMM {key}: VGPRs {got[0]}, AGPRs {got[1]} above the record "
                            f"{rec[0]}, {rec[1]}")
    if not found:
        problems.append("no GEMM kernel found in the resource report")
    return problems


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    remarks = "\n".join(r for _, r in done)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(remarks)
    problems = check_gemm_resources(remarks)
    if problems:
        raise RuntimeError("GEMM register guard failed:\n  " + "\n  ".join(problems))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probes(verbose)
    return LIB


def build_probes(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PROBE_SRC, "*.hip")))
    tmp = PROBE_LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *HIPFLAGS, "-shared", *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
