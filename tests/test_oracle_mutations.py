"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle source (on the CPU only),
builds it into a temporary library and runs the pin suite against it: the suite
has to fail.  Mistakes cover rounding modes, operand halves, indexing, sort
stability, a dropped rounding step and the scale arithmetic.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "megamoe_oracle.c")

MUTATIONS = {
    "quant_rint_not_round": ("float r = roundf(v / scale);", "float r = rintf(v / scale);"),
    "quant_reciprocal": ("float r = roundf(v / scale);", "float r = roundf(v * (127.0f / amax));"),
    "silu_on_gate_half": (
        "float u = orc_h2f(c_row[i]) * pts1;\n        float g = orc_h2f(c_row[I + i]) * pts1;",
        "float g = orc_h2f(c_row[i]) * pts1;\n        float u = orc_h2f(c_row[I + i]) * pts1;"),
    "requant_round_not_rint": ("float r = rintf(y[i] * mul);", "float r = roundf(y[i] * mul);"),
    "dequant_scale_index": ("float prod = (float)acc[n] * scale[n];",
                            "float prod = (float)acc[n] * scale[0];"),
    "unstable_sort": ("for (int64_t r = 0; r < R; ++r) {\n            if (expert_idx[r] == e) {",
                      "for (int64_t r = R - 1; r >= 0; --r) {\n            if (expert_idx[r] == e) {"),
    "combine_no_cast": ("float d = orc_bf2f(orc_f2bf(deq));", "float d = deq;"),
    "half_truncates": ("double n = nearbyint(a / q);", "double n = floor(a / q);"),
    "prob_slot_index": ("float weighted = d * probs_t[s];", "float weighted = d * probs_t[0];"),
    "gmm_drops_last_k": ("for (int32_t k = 0; k < Kred; ++k) {", "for (int32_t k = 0; k + 1 < Kred; ++k) {"),
    "pts1_after_silu": ("float s = u / den;",
                        "float s = (u / pts1) / (1.0f + expf(-(u / pts1))) * pts1;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, name
    csrc = tmp_path / "mutant.c"
    csrc.write_text(src.replace(before, after))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *O.CFLAGS, str(csrc), "-o", str(lib), "-lm"])
    env = dict(os.environ, MEGAMOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"{name}: pins did not catch the mistake\n{r.stdout[-2000:]}"
