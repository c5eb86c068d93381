"""Host-side checks that need no GPU.

* The quantiser's division (FrontReorder step 2c: q = CAST_ROUND(x / scale)):
  the FMA-corrected reciprocal form the GPU kernel uses gives the same int8
  code as rounding the IEEE quotient for every finite fp16 row maximum and
  every fp16 value up to it (tests/csrc/quant_exhaustive.c).
* The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
  clean on small shapes with dropped routes, zero rows, E = 1 and top_k = E
  (tests/csrc/oracle_asan_main.c).
* The grouped GEMM's register guard: the compiler's resource report of every
  GEMM instantiation shows no spills and no more registers than recorded.
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


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.check_call([_gcc(), "-O1", "-g", "-std=c11", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", os.path.join(CSRC, "oracle_asan_main.c"),
                           os.path.join(ROOT, "oracle", "megamoe_oracle.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count(" ok") == 6


def test_gemm_register_guard():
    src = os.path.join(ROOT, "moe_expert_ffn_amd", "csrc", "gmm.hip")
    r = subprocess.run([B.HIPCC, *B.HIPFLAGS, B.RESOURCE_REMARKS, "--offload-device-only",
                        "-S", src, "-o", os.devnull], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    res = {B.gemm_template_args(k): v for k, v in B.kernel_resources(r.stderr).items()
           if B.gemm_template_args(k) is not None}
    assert set(res) == set(B.GEMM_REGISTERS), res
    assert B.check_gemm_resources(r.stderr) == []


def test_gemm_register_guard_rejects_spills_and_growth():
    name = ("_ZN7megamoe18gmm_i8_ring_kernelILi256ELi4ELi4ELi4ELb0ELb1ELi0ELb0EEEvNS_9GmmParamsE")
    fake = (f"x.hip:1:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]\n")
    problems = B.check_gemm_resources(fake)
    assert any("spilled" in p for p in problems)
    assert any("above the record" in p for p in problems)
