"""Host-side checks that need no GPU.

* The quantiser's division (FrontReorder step 2c: q = CAST_ROUND(x / scale)):
  the FMA-corrected reciprocal form the GPU kernel uses gives the same int8
  code as rounding the IEEE quotient for every finite fp16 row maximum and
  every fp16 value up to it, and SwiGLU's rounding of the re-quantised product
  by adding 1.5 * 2^23 equals rintf for every float up to 128 in magnitude
  (tests/csrc/quant_exhaustive.c).
* The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
  clean on small shapes with dropped routes, zero rows, E = 1 and top_k = E
  (tests/csrc/oracle_asan_main.c).
* The grouped GEMM's register guard: the compiler's resource report of every
  GEMM instantiation shows no more registers or spilled values than recorded,
  and its assembly has no scratch (spill) access at all.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from moe_expert_ffn_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tests", "csrc")


def _gcc():
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    return cc


def test_quantiser_division_exhaustive(tmp_path):
    exe = str(tmp_path / "quant_exhaustive")
    subprocess.check_call([_gcc(), "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           os.path.join(CSRC, "quant_exhaustive.c"), "-o", exe, "-lm"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    words = r.stdout.split()
    assert words[0] == "pairs" and int(words[1]) > 10 ** 9 and words[3] == "0"
    # SwiGLU's CAST_RINT by adding 1.5 * 2^23: every float with |p| <= 128
    assert words[4:6] == ["rint", "values"] and int(words[6]) > 2 * 10 ** 9 and words[8] == "0"


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.check_call([_gcc(), "-O1", "-g", "-std=c11", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", os.path.join(CSRC, "oracle_asan_main.c"),
                           os.path.join(ROOT, "oracle", "megamoe_oracle.c"), "-o", exe, "-lm"])
    # verify_asan_link_order=0: the sanitizer runtime need not be the first
    # library loaded when the environment preloads another one
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count(" ok") == 6


def test_gemm_register_guard():
    src = os.path.join(ROOT, "moe_expert_ffn_amd", "csrc", "gmm.hip")
    r = subprocess.run([B.HIPCC, *B.HIPFLAGS, B.RESOURCE_REMARKS, "--offload-device-only",
                        "-S", src, "-o", "-"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    res = {B.gemm_template_args(k): v for k, v in B.kernel_resources(r.stderr).items()
           if B.gemm_template_args(k) is not None}
    assert set(res) == set(B.GEMM_RESOURCES), res
    assert B.check_gemm_resources(r.stderr) == []
    # the shipped kernel: no spill access inside a loop that issues ring copies
    assert B.check_gemm_loops(r.stdout) == []


_GEMM_NAME = "_ZN7megamoe18gmm_i8_ring_kernelILi256ELi4ELi4ELi4ELb0ELb1ELi0ELb0EEEvNS_9GmmParamsE"


def test_gemm_register_guard_rejects_spills_and_growth():
    fake = (f"x.hip:1:1: remark: Function Name: {_GEMM_NAME} "
            "[-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs: 130 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs Spill: 9 [-Rpass-analysis=kernel-resource-usage]\n")
    problems = B.check_gemm_resources(fake)
    assert any("above the record" in p for p in problems)


def _fake_asm(reload: str) -> str:
    """A GEMM function in the compiler's assembly layout: a tile loop (depth
    1) holding a K loop (depth 2) that issues a copy; one spill reload inside
    the K loop ("loop"), after it ("after"), or none ("none")."""
    rl = "\tscratch_load_dword v0, off, off offset:8 ; 4-byte Folded Reload\n"
    return (f"; -- Begin function {_GEMM_NAME}\n"
            ".LBB2_48:                ; =>This Loop Header: Depth=1\n"
            "\tv_mov_b32 v1, 0\n"
            ".LBB2_85:                ;   Parent Loop BB2_48 Depth=1\n"
            "                         ; =>  This Inner Loop Header: Depth=2\n"
            "\tglobal_load_lds_dwordx4 v2, s[4:5]\n"
            + (rl if reload == "loop" else "") +
            "\tv_mfma_i32_16x16x64_i8 v[0:3], v[4:7], v[8:11], v[0:3]\n"
            "\ts_cbranch_scc1 .LBB2_85\n"
            ".LBB2_97:                ;   in Loop: Header=BB2_48 Depth=1\n"
            + (rl if reload == "after" else "") +
            "\ts_cbranch_scc1 .LBB2_48\n"
            ".Lfunc_end2:\n")


def test_gemm_loop_guard_rejects_any_reload():
    # the next tile's copies are in flight through the epilogue, so a reload
    # after the K loop is rejected as well as one inside it
    assert B.check_gemm_loops(_fake_asm("none")) == []
    after = B.check_gemm_loops(_fake_asm("after"))
    assert len(after) == 1 and "scratch" in after[0]
    inside = B.check_gemm_loops(_fake_asm("loop"))
    assert any("inside a loop" in p for p in inside) and any("scratch" in p for p in inside)
