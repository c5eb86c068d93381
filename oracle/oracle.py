"""ctypes wrapper around the plain C oracle (megamoe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this.

Every function takes and returns numpy arrays; fp16 and bf16 values travel as
their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "megamoe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O3", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (gcc)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MEGAMOE_ORACLE_LIB", _LIB)   # planted-mistake builds in tests
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32, u16 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint16
        L.orc_f2h.argtypes, L.orc_f2h.restype = [f32], u16
        L.orc_h2f.argtypes, L.orc_h2f.restype = [u16], f32
        L.orc_f2bf.argtypes, L.orc_f2bf.restype = [f32], u16
        L.orc_bf2f.argtypes, L.orc_bf2f.restype = [u16], f32
        L.orc_route_sort.argtypes = [i32, i32, i32, P, P, P, P, P, P]
        L.orc_route_sort.restype = i64
        L.orc_quant_token.argtypes = [i32, P, P, P]
        L.orc_quant_token.restype = None
        L.orc_gmm_row.argtypes = [i32, i32, P, P, P, P, P]
        L.orc_gmm_row.restype = None
        L.orc_swiglu_quant_row.argtypes = [i32, P, f32, P, P]
        L.orc_swiglu_quant_row.restype = None
        L.orc_unpermute_token.argtypes = [i32, i32, P, P, P, P, P, P]
        L.orc_unpermute_token.restype = None
        L.orc_forward.argtypes = [i32] * 5 + [P] * 22
        L.orc_forward.restype = i64
        L.orc_forward_token.argtypes = [i32] * 4 + [P] * 17
        L.orc_forward_token.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar format helpers (vectorised by a Python loop; small inputs only) ----
def f2h(v: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(v, dtype=np.float32).ravel()
    return np.array([L.orc_f2h(float(x)) for x in flat], dtype=np.uint16).reshape(np.shape(v))


def h2f(b: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(b, dtype=np.uint16).ravel()
    return np.array([L.orc_h2f(int(x)) for x in flat], dtype=np.float32).reshape(np.shape(b))


def f2bf(v: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(v, dtype=np.float32).ravel()
    return np.array([L.orc_f2bf(float(x)) for x in flat], dtype=np.uint16).reshape(np.shape(v))


# ---- stages ----
def route_sort(expert_idx: np.ndarray, E: int) -> dict:
    ei = _c(expert_idx, np.int32)
    M, top_k = ei.shape
    R = M * top_k
    out = dict(sorted_route=np.empty(R, np.int32), expanded_row_idx=np.empty(R, np.int32),
               tokens_per_expert=np.empty(E, np.int32), expert_offsets=np.empty(E + 1, np.int32),
               expert_cumsum=np.empty(E, np.int32))
    dropped = lib().orc_route_sort(M, top_k, E, _p(ei), _p(out["sorted_route"]),
                                   _p(out["expanded_row_idx"]), _p(out["tokens_per_expert"]),
                                   _p(out["expert_offsets"]), _p(out["expert_cumsum"]))
    out["dropped"] = int(dropped)
    return out


def quant_token(x_row: np.ndarray) -> tuple[np.ndarray, np.float32]:
    xr = _c(x_row, np.float16).view(np.uint16)
    K = xr.shape[0]
    q = np.empty(K, np.int8)
    sc = np.empty(1, np.float32)
    lib().orc_quant_token(K, _p(xr), _p(q), _p(sc))
    return q, sc[0]


def gmm_row(a_row: np.ndarray, w: np.ndarray, scale: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """w: logical [Kred, N] int8 of one expert."""
    a = _c(a_row, np.int8)
    w = _c(w, np.int8)
    s = _c(scale, np.float32)
    Kred, N = w.shape
    acc = np.empty(N, np.int32)
    c = np.empty(N, np.uint16)
    lib().orc_gmm_row(Kred, N, _p(a), _p(w), _p(s), _p(acc), _p(c))
    return acc, c.view(np.float16)


def swiglu_quant_row(c_row: np.ndarray, pts1: float) -> tuple[np.ndarray, np.float32]:
    c = _c(c_row, np.float16).view(np.uint16)
    I = c.shape[0] // 2
    q2 = np.empty(I, np.int8)
    p2 = np.empty(1, np.float32)
    lib().orc_swiglu_quant_row(I, _p(c), ctypes.c_float(pts1), _p(q2), _p(p2))
    return q2, p2[0]


def unpermute_token(eri_t, probs_t, gmm2_out, pts2) -> tuple[np.ndarray, np.ndarray]:
    eri_t = _c(eri_t, np.int32)
    probs_t = _c(probs_t, np.float32)
    g = _c(gmm2_out, np.float16).view(np.uint16)
    p2 = _c(pts2, np.float32)
    K = g.shape[1]
    out = np.empty(K, np.uint16)
    outf = np.empty(K, np.float32)
    lib().orc_unpermute_token(K, eri_t.shape[0], _p(eri_t), _p(probs_t), _p(g), _p(p2), _p(out),
                              _p(outf))
    return out, outf


def forward(inp: dict, E: int | None = None) -> dict:
    """Whole forward with every intermediate.  out is bf16 bits (uint16)."""
    x = _c(inp["x"], np.float16).view(np.uint16)
    ei = _c(inp["expert_idx"], np.int32)
    probs = _c(inp["probs"], np.float32)
    w1 = _c(inp["w1"], np.int8)
    s1 = _c(inp["scale1"], np.float32)
    w2 = _c(inp["w2"], np.int8)
    s2 = _c(inp["scale2"], np.float32)
    M, K = x.shape
    E = w1.shape[0] if E is None else E
    top_k = ei.shape[1]
    N1 = w1.shape[2]
    I = N1 // 2
    R = M * top_k
    o = dict(sorted_route=np.empty(R, np.int32), expanded_row_idx=np.empty(R, np.int32),
             tokens_per_expert=np.empty(E, np.int32), expert_offsets=np.empty(E + 1, np.int32),
             expert_cumsum=np.empty(E, np.int32),
             gmA=np.zeros((R, K), np.int8), pts1=np.zeros(R, np.float32),
             acc1=np.zeros((R, N1), np.int32), gmC=np.zeros((R, N1), np.uint16),
             q2=np.zeros((R, I), np.int8), pts2=np.zeros(R, np.float32),
             acc2=np.zeros((R, K), np.int32), gmm2_out=np.zeros((R, K), np.uint16),
             out=np.empty((M, K), np.uint16), out_f32=np.empty((M, K), np.float32))
    keys = ["sorted_route", "expanded_row_idx", "tokens_per_expert", "expert_offsets",
            "expert_cumsum", "gmA", "pts1", "acc1", "gmC", "q2", "pts2", "acc2", "gmm2_out",
            "out", "out_f32"]
    dropped = lib().orc_forward(M, K, E, top_k, I, _p(x), _p(ei), _p(probs), _p(w1), _p(s1),
                                _p(w2), _p(s2), *[_p(o[k]) for k in keys])
    o["dropped"] = int(dropped)
    o["gmC"] = o["gmC"].view(np.float16)
    o["gmm2_out"] = o["gmm2_out"].view(np.float16)
    return o


def forward_token(inp: dict, t: int) -> dict:
    """One token's forward (no sort); slot rows in slot order."""
    x = _c(inp["x"][t], np.float16).view(np.uint16)
    ei = _c(inp["expert_idx"][t], np.int32)
    probs = _c(inp["probs"][t], np.float32)
    w1, s1, w2, s2 = inp["w1"], inp["scale1"], inp["w2"], inp["scale2"]
    for a in (w1, s1, w2, s2):
        assert a.flags["C_CONTIGUOUS"]
    E, K, N1 = w1.shape
    I = N1 // 2
    top_k = ei.shape[0]
    o = dict(qa=np.empty(K, np.int8), pts1=np.empty(1, np.float32),
             acc1=np.zeros((top_k, N1), np.int32), gmC=np.zeros((top_k, N1), np.uint16),
             q2=np.zeros((top_k, I), np.int8), pts2=np.zeros(top_k, np.float32),
             acc2=np.zeros((top_k, K), np.int32), gmm2_out=np.zeros((top_k, K), np.uint16),
             out=np.empty(K, np.uint16), out_f32=np.empty(K, np.float32))
    keys = ["qa", "pts1", "acc1", "gmC", "q2", "pts2", "acc2", "gmm2_out", "out", "out_f32"]
    lib().orc_forward_token(K, E, top_k, I, _p(x), _p(ei), _p(probs), _p(w1), _p(s1), _p(w2),
                            _p(s2), *[_p(o[k]) for k in keys])
    o["pts1"] = o["pts1"][0]
    o["gmC"] = o["gmC"].view(np.float16)
    o["gmm2_out"] = o["gmm2_out"].view(np.float16)
    return o


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
