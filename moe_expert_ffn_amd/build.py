"""Build the gfx950 HIP library libmegamoe.so in-tree with hipcc.

Run as ``python -m moe_expert_ffn_amd.build``.  Objects are compiled in
parallel into moe_expert_ffn_amd/_build and linked into
moe_expert_ffn_amd/libmegamoe.so.

The build also guards the grouped GEMM's register budget.  Its K loop issues
the global -> LDS copies from inline assembly, which the compiler's wait-count
pass does not see; any compiler-visible vector load that lands in the loop (a
spill reload, for instance) gets a wait that in hardware also waits for every
copy in flight and drains the copy ring.  The next tile's first copies are
issued before the current tile's epilogue, so copies are in flight almost
everywhere.  The build therefore compiles the GEMM to assembly as well and
fails if the kernel accesses scratch (spill) memory anywhere, or if an
instantiation uses more registers or spills more values than recorded in
GEMM_RESOURCES below.
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
# (BM, WAVES_M, WAVES_N, NS, TRIM, SKIP, PRIO, NTB): (VGPRs, AGPRs, spilled
# vector values, spilled scalar values).  The 256-row tiles run 16 waves per
# CU, so 128 registers per wave is the ceiling.  Spilled scalar values go to
# lanes of a vector register (v_writelane / v_readlane), not to memory; a
# spilled vector value would go to scratch memory, which the checks below
# forbid anywhere in the kernel.
GEMM_RESOURCES = {
    (64, 1, 4, 3, 1, 1, 16, 1): (110, 92, 0, 4),
    (256, 4, 4, 4, 0, 1, 0, 0): (128, 0, 0, 23),
    (256, 4, 4, 4, 0, 1, 0, 1): (128, 0, 0, 23),
}
GEMM_SRC = os.path.join(CSRC, "gmm.hip")


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
    """Every GEMM instantiation: registers and spills within the record."""
    problems = []
    found = 0
    for name, r in kernel_resources(remarks).items():
        key = gemm_template_args(name)
        if key is None:
            continue
        found += 1
        got = (r.get("VGPRs", 0), r.get("AGPRs", 0), r.get("VGPRs Spill", 0),
               r.get("SGPRs Spill", 0))
        rec = GEMM_RESOURCES.get(key)
        desc = "VGPRs {}, AGPRs {}, vector spills {}, scalar spills {}"
        if rec is None:
            problems.append(f"GEMM {key}: no record ({desc.format(*got)})")
        elif any(g > r_ for g, r_ in zip(got, rec)):
            problems.append(f"GEMM {key}: {desc.format(*got)} above the record "
                            f"{desc.format(*rec)}")
    if not found:
        problems.append("no GEMM kernel found in the resource report")
    return problems


def check_gemm_loops(asm: str) -> list[str]:
    """No scratch access in a GEMM kernel, and none inside a copy loop.

    The ring copies (global_load_lds_dwordx4) are in flight through almost
    the whole kernel: the next tile's first copies are issued before the
    current tile's epilogue.  A scratch load (a spill reload) anywhere after
    them gets a vmcnt wait that also waits for every copy and store issued
    before it, so no GEMM kernel may access scratch memory at all.  The
    device assembly also marks each basic block with its loop depth; the run
    of nested blocks (depth 2 or more: the K loops inside the tile loop) that
    contains a copy is reported separately, as that is where a reload would
    drain the ring at every K step."""
    problems = []
    found = 0
    for func in asm.split("; -- Begin function ")[1:]:
        name = func.split("\n", 1)[0].strip()
        if "gmm_i8_ring_kernel" not in name:
            continue
        found += 1
        body = func.split(".Lfunc_end", 1)[0]
        depth, region = 0, []

        def close():
            if (any("global_load_lds_dwordx4" in x for x in region)
                    and any("scratch_" in x for x in region)):
                problems.append(f"GEMM {gemm_template_args(name)}: a spill access inside a "
                                "loop that issues the ring copies")

        for line in body.splitlines():
            d = None
            m = re.search(r"Depth=(\d+)", line)
            if line.startswith(".LBB") or (m and "Loop Header" in line):
                d = int(m.group(1)) if m else 0
            if d is not None:
                if d < 2 and depth >= 2:
                    close()
                    region = []
                depth = d
            if depth >= 2:
                region.append(line)
        close()
        if re.search(r"^\s*scratch_", body, re.M):
            problems.append(f"GEMM {gemm_template_args(name)}: scratch (spill) accesses "
                            "in the kernel")
    if not found:
        problems.append("no GEMM kernel found in the assembly")
    return problems


def _gemm_asm() -> str:
    out = os.path.join(BUILD, "gmm.s")
    cmd = [HIPCC, *HIPFLAGS, "-S", "--cuda-device-only", GEMM_SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {GEMM_SRC}:\n{r.stderr}")
    with open(out) as f:
        return f.read()


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        asm = ex.submit(_gemm_asm)
        done = list(ex.map(_compile, srcs))
        gemm_asm = asm.result()
    objs = [o for o, _ in done]
    remarks = "\n".join(r for _, r in done)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(remarks)
    problems = check_gemm_resources(remarks) + check_gemm_loops(gemm_asm)
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
