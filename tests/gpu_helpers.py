"""Runs the HIP path through the C ABI and compares it with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from moe_expert_ffn_amd import megamoe as MM


def to_dev(inp: dict, device="cuda") -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in inp.items()}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def prepack(d, dev: dict):
    n1, n2 = MM.megamoe_packed_weight_bytes(d)
    w1p = torch.empty(n1, dtype=torch.int8, device="cuda")
    w2p = torch.empty(n2, dtype=torch.int8, device="cuda")
    MM.megamoe_prepack_w1(d, dev["w1"], w1p)
    MM.megamoe_prepack_w2(d, dev["w2"], w2p)
    return w1p, w2p


def run_stages(w, dev: dict, w1p, w2p, debug_acc: bool = True, gather: bool = False,
               paired: bool = False) -> dict:
    """Each stage through its own entry point; every intermediate returned (device).

    gather: the first two stages as the forward runs them
    (megamoe_permute_tokens + megamoe_gmm1_gather); o["qx"] then holds the
    token-major quantised x and o["gmA"] stays zero.
    paired (with gather): all stages as the forward runs them, SwiGLU and GMM2
    passing q2 in the row-paired layout (o["q2p"], o["prow"]; o["q2"] stays
    zero); GMM1 also through megamoe_gmm1_gather_split, twice, into
    o["gmC_split"] and o["gmC_split2"]."""
    assert gather or not paired
    d = MM.dims(w.M, w.K, w.E, w.top_k, w.I)
    R = w.R
    cu = dict(device="cuda")
    o = dict(
        gmA=torch.zeros((R, w.K), dtype=torch.int8, **cu),
        pts1=torch.zeros(R, dtype=torch.float32, **cu),
        expanded_row_idx=torch.empty(R, dtype=torch.int32, **cu),
        sorted_route=torch.empty(R, dtype=torch.int32, **cu),
        tokens_per_expert=torch.empty(w.E, dtype=torch.int32, **cu),
        expert_cumsum=torch.empty(w.E, dtype=torch.int32, **cu),
        gmC=torch.zeros((R, w.N1), dtype=torch.float16, **cu),
        q2=torch.zeros((R, w.I), dtype=torch.int8, **cu),
        pts2=torch.zeros(R, dtype=torch.float32, **cu),
        gmm2_out=torch.zeros((R, w.K), dtype=torch.float16, **cu),
        out=torch.empty((w.M, w.K), dtype=torch.bfloat16, **cu),
    )
    if debug_acc:
        o["acc1"] = torch.zeros((R, w.N1), dtype=torch.int32, **cu)
        o["acc2"] = torch.zeros((R, w.K), dtype=torch.int32, **cu)
    ws = torch.empty(MM.megamoe_permute_workspace_bytes(d), dtype=torch.uint8, **cu)
    if paired:
        o["qx"] = torch.zeros((w.M, w.K), dtype=torch.int8, **cu)
        o["prow"] = torch.full((R,), -1, dtype=torch.int32, **cu)
        o["q2p"] = torch.zeros(MM.megamoe_paired_q2_bytes(d), dtype=torch.int8, **cu)
        MM.megamoe_permute_tokens_paired(d, dev["x"], dev["expert_idx"], o["qx"], o["pts1"],
                                         o["expanded_row_idx"], o["sorted_route"],
                                         o["tokens_per_expert"], o["expert_cumsum"], o["prow"],
                                         ws)
        MM.megamoe_gmm1_gather(d, o["qx"], o["sorted_route"], o["expert_cumsum"], w1p,
                               dev["scale1"], o["gmC"], o.get("acc1"))
        # GMM1 as the forward runs it (a sparse last round split over K), twice
        # on one zero-filled buffer: the second call finds the counters the
        # first one left
        sws = torch.zeros(MM.megamoe_gmm1_split_workspace_bytes(d), dtype=torch.uint8, **cu)
        for k in ("gmC_split", "gmC_split2"):
            o[k] = torch.zeros((R, w.N1), dtype=torch.float16, **cu)
            MM.megamoe_gmm1_gather_split(d, o["qx"], o["sorted_route"], o["expert_cumsum"], w1p,
                                         dev["scale1"], o[k], sws)
        MM.megamoe_swiglu_quant_paired(d, o["gmC"], o["pts1"], o["expert_cumsum"], o["prow"],
                                       o["q2p"], o["pts2"])
        MM.megamoe_gmm2_paired(d, o["q2p"], o["expert_cumsum"], w2p, dev["scale2"],
                               o["gmm2_out"], o.get("acc2"))
        MM.megamoe_unpermute(d, o["gmm2_out"], o["pts2"], o["expanded_row_idx"], dev["probs"],
                             o["out"])
        o["dropped"] = MM.megamoe_last_error(ws)
        return o
    if gather:
        o["qx"] = torch.zeros((w.M, w.K), dtype=torch.int8, **cu)
        MM.megamoe_permute_tokens(d, dev["x"], dev["expert_idx"], o["qx"], o["pts1"],
                                  o["expanded_row_idx"], o["sorted_route"],
                                  o["tokens_per_expert"], o["expert_cumsum"], ws)
        MM.megamoe_gmm1_gather(d, o["qx"], o["sorted_route"], o["expert_cumsum"], w1p,
                               dev["scale1"], o["gmC"], o.get("acc1"))
    else:
        MM.megamoe_permute(d, dev["x"], dev["expert_idx"], o["gmA"], o["pts1"],
                           o["expanded_row_idx"], o["sorted_route"], o["tokens_per_expert"],
                           o["expert_cumsum"], ws)
        MM.megamoe_gmm1(d, o["gmA"], o["expert_cumsum"], w1p, dev["scale1"], o["gmC"],
                        o.get("acc1"))
    MM.megamoe_swiglu_quant(d, o["gmC"], o["pts1"], o["expert_cumsum"], o["q2"], o["pts2"])
    MM.megamoe_gmm2(d, o["q2"], o["expert_cumsum"], w2p, dev["scale2"], o["gmm2_out"],
                    o.get("acc2"))
    MM.megamoe_unpermute(d, o["gmm2_out"], o["pts2"], o["expanded_row_idx"], dev["probs"],
                         o["out"])
    o["dropped"] = MM.megamoe_last_error(ws)
    return o


def run_forward(w, dev: dict, w1p, w2p) -> tuple[torch.Tensor, int]:
    d = MM.dims(w.M, w.K, w.E, w.top_k, w.I)
    ws = torch.empty(MM.megamoe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda")
    MM.megamoe_forward(d, dev["x"], dev["expert_idx"], dev["probs"], w1p, dev["scale1"], w2p,
                       dev["scale2"], out, ws)
    return out, MM.megamoe_last_error(ws)


def assert_int8_within_1lsb(gpu: np.ndarray, ref: np.ndarray, what: str, frac: float = 1e-3):
    diff = np.abs(gpu.astype(np.int32) - ref.astype(np.int32))
    assert diff.max(initial=0) <= 1, f"{what}: max diff {diff.max()}"
    bad = np.count_nonzero(diff)
    assert bad <= frac * max(diff.size, 1), f"{what}: {bad} of {diff.size} differ by 1"
    return bad


def assert_out_close(gpu_out_f32: np.ndarray, ref_f32: np.ndarray, what: str = "out"):
    """|out - out_ref| <= 2e-2 * max|out_ref| (the out tolerance of the pipeline)."""
    assert np.all(np.isfinite(gpu_out_f32)), f"{what}: non-finite values"
    scale = float(np.abs(ref_f32).max(initial=0.0))
    err = float(np.abs(gpu_out_f32 - ref_f32).max(initial=0.0))
    assert err <= 2e-2 * scale + 1e-30, f"{what}: max err {err} vs 2e-2*{scale}"
    return err / max(scale, 1e-30)


def run_stages_on_oracle_inputs(w, o_ref: dict, dev: dict, w1p, w2p) -> dict:
    """Each GPU stage fed with the oracle's own inputs to that stage (its gmA,
    gmC and pts1, q2, gmm2_out and pts2, expanded_row_idx, expert_cumsum), so a
    difference upstream cannot hide or excuse one downstream: GMM2 is checked
    on every row even where the GPU's own q2 differs from the oracle's by an
    LSB.  Returns the GPU results (device tensors)."""
    d = MM.dims(w.M, w.K, w.E, w.top_k, w.I)
    R = w.R
    cu = dict(device="cuda")

    def up(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to("cuda")

    cum = up(o_ref["expert_cumsum"])
    o = dict(
        acc1=torch.zeros((R, w.N1), dtype=torch.int32, **cu),
        gmC=torch.zeros((R, w.N1), dtype=torch.float16, **cu),
        q2=torch.zeros((R, w.I), dtype=torch.int8, **cu),
        pts2=torch.zeros(R, dtype=torch.float32, **cu),
        acc2=torch.zeros((R, w.K), dtype=torch.int32, **cu),
        gmm2_out=torch.zeros((R, w.K), dtype=torch.float16, **cu),
        out=torch.empty((w.M, w.K), dtype=torch.bfloat16, **cu),
    )
    MM.megamoe_gmm1(d, up(o_ref["gmA"]), cum, w1p, dev["scale1"], o["gmC"], o["acc1"])
    MM.megamoe_swiglu_quant(d, up(o_ref["gmC"]), up(o_ref["pts1"]), cum, o["q2"], o["pts2"])
    MM.megamoe_gmm2(d, up(o_ref["q2"]), cum, w2p, dev["scale2"], o["gmm2_out"], o["acc2"])
    MM.megamoe_unpermute(d, up(o_ref["gmm2_out"]), up(o_ref["pts2"]),
                         up(o_ref["expanded_row_idx"]), dev["probs"], o["out"])
    return o


def compare_stages_on_oracle_inputs(w, o_ref: dict, g: dict) -> None:
    """Gates for run_stages_on_oracle_inputs: the int32 accumulators and the
    fp16 GEMM outputs bit-exact on every valid row, q2 within 1 LSB on at most
    0.1% of elements and pts2 within 1e-6 relative, and the combine + unpermute
    bit-exact (the same slot-order multiply-then-add in fp32 and the same two
    round-to-nearest-even bf16 casts as the oracle)."""
    Rv = w.R - o_ref["dropped"]
    acc1 = g["acc1"].cpu().numpy()[:Rv]
    assert np.array_equal(acc1, o_ref["acc1"][:Rv]), "acc1 (oracle gmA)"
    assert np.array_equal(g["gmC"].cpu().numpy()[:Rv].view(np.uint16),
                          o_ref["gmC"][:Rv].view(np.uint16)), "gmC (oracle gmA)"
    assert_int8_within_1lsb(g["q2"].cpu().numpy()[:Rv], o_ref["q2"][:Rv], "q2 (oracle gmC)")
    np.testing.assert_allclose(g["pts2"].cpu().numpy()[:Rv], o_ref["pts2"][:Rv], rtol=1e-6,
                               atol=0)
    assert np.array_equal(g["acc2"].cpu().numpy()[:Rv], o_ref["acc2"][:Rv]), "acc2 (oracle q2)"
    assert np.array_equal(g["gmm2_out"].cpu().numpy()[:Rv].view(np.uint16),
                          o_ref["gmm2_out"][:Rv].view(np.uint16)), "gmm2_out (oracle q2)"
    assert np.array_equal(bf16_bits(g["out"]), o_ref["out"]), "out (oracle gmm2_out, pts2)"
