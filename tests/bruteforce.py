"""Independent per-token brute force of the MegaMoE forward, in numpy.

Used only to pin the C oracle.  It never sorts or groups: every token walks its
own top-k slots, looks up its expert's weights and evaluates the stage formulas
of the pto-isa MegaMoE overview page directly.  Float narrowings use numpy's
float16 conversion and torch's bfloat16 conversion (both IEEE round-to-nearest-
even), not the oracle's own rounding code.
"""
from __future__ import annotations

import numpy as np
import torch


def to_bf16_f32(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and widen back to float32."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quant(x_row_f16: np.ndarray):
    v = x_row_f16.astype(np.float32)
    amax = np.float32(np.abs(v).max())
    if amax == 0:
        return np.zeros(v.shape, np.int8), np.float32(0)
    sc = np.float32(amax / np.float32(127.0))
    r = (v / sc).astype(np.float32)
    # half away from zero; |r| + 0.5 is exact in float64
    q = np.sign(r) * np.floor(np.abs(r.astype(np.float64)) + 0.5)
    return np.clip(q, -127, 127).astype(np.int8), sc


def gmm(a_row_i8: np.ndarray, w_kn: np.ndarray, scale: np.ndarray):
    acc = (a_row_i8.astype(np.int64)[:, None] * w_kn.astype(np.int64)).sum(axis=0)
    assert np.all(np.abs(acc) < 2**31)
    acc = acc.astype(np.int32)
    c = (acc.astype(np.float32) * scale.astype(np.float32)).astype(np.float16)
    return acc, c


def swiglu_quant(c_row_f16: np.ndarray, pts1: np.float32):
    I = c_row_f16.shape[0] // 2
    c = c_row_f16.astype(np.float32) * np.float32(pts1)
    u, g = c[:I], c[I:]
    # exp evaluated in float64 and rounded once to float32
    ex = np.exp(-u.astype(np.float64)).astype(np.float32)
    s = (u / (ex + np.float32(1.0))).astype(np.float32)
    y = (s * g).astype(np.float32)
    amax = np.float32(np.abs(y).max())
    if amax == 0:
        return np.zeros(I, np.int8), np.float32(0), y
    pts2 = np.float32(amax / np.float32(127.0))
    mul = np.float32(np.float32(127.0) / amax)
    q = np.clip(np.rint((y * mul).astype(np.float32)), -127, 127).astype(np.int8)
    return q, pts2, y


def forward_token(inp: dict, t: int):
    """Returns dict with per-slot intermediates and out (bf16 bits), out_f32."""
    x = inp["x"][t]
    ei = inp["expert_idx"][t]
    probs = inp["probs"][t].astype(np.float32)
    E, K, N1 = inp["w1"].shape
    qa, pts1 = quant(x)
    acc = np.zeros(K, np.float32)
    slots = []
    for s, e in enumerate(ei):
        if not (0 <= e < E):
            slots.append(None)
            continue
        acc1, gmC = gmm(qa, inp["w1"][e], inp["scale1"][e])
        q2, pts2, _ = swiglu_quant(gmC, pts1)
        acc2, g2 = gmm(q2, inp["w2"][e], inp["scale2"][e])
        d = to_bf16_f32(g2.astype(np.float32) * pts2)
        acc = (acc + (d * probs[s]).astype(np.float32)).astype(np.float32)
        slots.append(dict(acc1=acc1, gmC=gmC, q2=q2, pts2=pts2, acc2=acc2, gmm2_out=g2))
    return dict(qa=qa, pts1=pts1, slots=slots, out=to_bf16_bits(acc), out_f32=acc)


def forward_unquantised_f64(inp: dict, t: int) -> np.ndarray:
    """The same MoE FFN with no quantisation at all, in float64 (sanity only)."""
    x = inp["x"][t].astype(np.float64)
    out = np.zeros_like(x)
    E, K, N1 = inp["w1"].shape
    I = N1 // 2
    for s, e in enumerate(inp["expert_idx"][t]):
        w1 = inp["w1"][e].astype(np.float64) * inp["scale1"][e].astype(np.float64)[None, :]
        h = x @ w1
        u, g = h[:I], h[I:]
        y = u / (1 + np.exp(-u)) * g
        w2 = inp["w2"][e].astype(np.float64) * inp["scale2"][e].astype(np.float64)[None, :]
        out += inp["probs"][t, s] * (y @ w2)
    return out
