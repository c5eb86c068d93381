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


def run_stages(w, dev: dict, w1p, w2p, debug_acc: bool = True, gather: bool = False) -> dict:
    """Each stage through its own entry point; every intermediate returned (device).

    gather: the first two stages as the forward runs them
    (megamoe_permute_tokens + megamoe_gmm1_gather); o["qx"] then holds the
    token-major quantised x and o["gmA"] stays zero."""
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
