"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a library
routine (numpy float16, torch bfloat16, numpy stable argsort, float64 matmul),
a closed form worked by hand from the pto-isa MegaMoE overview page's stage
formulas, an invariant, an error bound, or an independent per-token brute force
(tests/bruteforce.py) that never sorts.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import inputs as W
from oracle import oracle as O
from tests import bruteforce as BF


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def test_h2f_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.h2f(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _halfway_points():
    # every midpoint between consecutive finite positive halves, both signs
    h = np.arange(0, 0x7bff, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2          # exact in float64, and in float32 as well
    mids = mids.astype(np.float32)
    return np.concatenate([mids, -mids])


def test_f2h_vs_numpy_ties_and_random():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        _halfway_points(),
        rng.standard_normal(4000).astype(np.float32) * np.float32(100.0),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-5),   # subnormal range
        np.array([65504, 65519.996, 65520, 65536, 1e9, -65520, 0.0, -0.0, 5.96e-8, 2.98e-8,
                  2.99e-8, np.inf, -np.inf], np.float32),
    ])
    got = O.f2h(vals)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f2bf_vs_torch():
    rng = np.random.default_rng(2)
    base = rng.standard_normal(6000).astype(np.float32) * np.float32(1000.0)
    # exact ties: bf16 value + half of its ulp
    b = torch.from_numpy(base).to(torch.bfloat16).float().numpy()
    ulp_half = np.abs(b) * np.float32(2.0 ** -8)
    ties = (b + np.sign(b) * np.ldexp(np.float32(1.0), np.floor(np.log2(np.abs(b) + 1e-30)).astype(
        np.int32) - 8)).astype(np.float32)
    del ulp_half
    vals = np.concatenate([base, ties, np.array([3.39e38, 3.4e38, -3.4e38, 1e-40, 0.0],
                                                np.float32)])
    got = O.f2bf(vals)
    ref = BF.to_bf16_bits(vals)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------
# FrontReorder: route sort and metadata
# ----------------------------------------------------------------------------
def _check_sort_invariants(ei, E, o):
    flat = ei.ravel()
    R = flat.size
    valid = (flat >= 0) & (flat < E)
    Rv = int(valid.sum())
    sr, eri = o["sorted_route"], o["expanded_row_idx"]
    # bijection between valid routes and rows [0, Rv)
    assert np.all(eri[~valid] == -1)
    assert sorted(eri[valid].tolist()) == list(range(Rv))
    assert np.all(sr[Rv:] == -1)
    assert np.array_equal(eri[sr[:Rv]], np.arange(Rv))
    # counts and prefixes
    cnt = o["tokens_per_expert"]
    assert cnt.sum() == Rv and o["dropped"] == R - Rv
    assert np.array_equal(o["expert_cumsum"], np.cumsum(cnt))
    assert o["expert_offsets"][0] == 0 and np.array_equal(o["expert_offsets"][1:], np.cumsum(cnt))
    # expert-major, ascending route inside each group
    e_sorted = flat[sr[:Rv]]
    assert np.all(np.diff(e_sorted) >= 0)
    for e in range(E):
        grp = sr[o["expert_offsets"][e]:o["expert_offsets"][e + 1]]
        assert np.all(np.diff(grp) > 0)
        assert np.all(flat[grp] == e)


@pytest.mark.parametrize("M,E,top_k,seed", [(1, 1, 1, 0), (16, 4, 2, 0), (37, 8, 3, 1),
                                            (256, 64, 6, 2), (300, 256, 8, 3), (5, 16, 16, 4)])
def test_route_sort_vs_stable_argsort(M, E, top_k, seed):
    rng = np.random.default_rng(seed)
    ei = np.argsort(rng.random((M, E)), axis=1)[:, :top_k].astype(np.int32)
    o = O.route_sort(ei, E)
    ref = np.argsort(ei.ravel(), kind="stable").astype(np.int32)
    assert np.array_equal(o["sorted_route"], ref)
    assert np.array_equal(o["tokens_per_expert"], np.bincount(ei.ravel(), minlength=E))
    _check_sort_invariants(ei, E, o)


def test_route_sort_duplicates_and_skew():
    rng = np.random.default_rng(5)
    ei = rng.integers(0, 3, (50, 4)).astype(np.int32)      # duplicates inside a token allowed
    ei[:, 0] = 1                                           # one hot expert
    o = O.route_sort(ei, 8)                                # experts 3..7 empty
    assert np.array_equal(o["sorted_route"], np.argsort(ei.ravel(), kind="stable"))
    assert np.all(o["tokens_per_expert"][3:] == 0)
    _check_sort_invariants(ei, 8, o)


def test_route_sort_closed_forms():
    # E = 1: identity permutation
    ei = np.zeros((9, 1), np.int32)
    o = O.route_sort(ei, 1)
    assert np.array_equal(o["sorted_route"], np.arange(9))
    # topK = 1, expert(t) = t mod E: rows of expert e are t = e, e+E, ...
    M, E = 23, 5
    ei = (np.arange(M) % E).astype(np.int32)[:, None]
    o = O.route_sort(ei, E)
    cnt = [(M - e + E - 1) // E for e in range(E)]
    for t in range(M):
        e = t % E
        assert o["expanded_row_idx"][t] == sum(cnt[:e]) + t // E


def test_route_sort_invalid_ids_dropped():
    ei = np.array([[0, 7], [-1, 1], [1, 0], [3, 2]], np.int32)  # E=3: ids 7, -1, 3 invalid
    o = O.route_sort(ei, 3)
    assert o["dropped"] == 3
    assert o["expanded_row_idx"].tolist() == [0, -1, -1, 2, 3, 1, -1, 4]
    assert o["sorted_route"].tolist() == [0, 5, 3, 4, 7, -1, -1, -1]
    _check_sort_invariants(ei, 3, o)


# ----------------------------------------------------------------------------
# FrontReorder: per-token dynamic quantisation (CAST_ROUND)
# ----------------------------------------------------------------------------
def test_quant_hand_examples():
    # max 127 -> scale exactly 1.0; halves round away from zero under CAST_ROUND
    x = np.array([127, 0.5, -0.5, 1.5, 2.5, -2.5, 63.5, 0], np.float16)
    q, sc = O.quant_token(x)
    assert sc == np.float32(1.0)
    assert q.tolist() == [127, 1, -1, 2, 3, -3, 64, 0]
    # max 127/32 -> scale exactly 1/32, q = 32 x
    x = np.array([3.96875, -1.0, 0.5, 1.0 / 64, -3.0 / 64], np.float16)
    q, sc = O.quant_token(x)
    assert sc == np.float32(1.0 / 32)
    assert q.tolist() == [127, -32, 16, 1, -2]
    # The page divides by the fp32 scale (TDIV), it does not multiply by 127/max:
    # with max 11 the fp32 scale 11/127 rounds up, so 5.5/scale = 63.4999.. -> 63,
    # whereas 5.5 * fp32(127/11) = 63.5 -> 64.
    q, sc = O.quant_token(np.array([11.0, 5.5], np.float16))
    assert np.float32(5.5) / sc < np.float32(63.5)
    assert q.tolist() == [127, 63]


def test_quant_special_rows():
    q, sc = O.quant_token(np.zeros(64, np.float16))
    assert sc == 0 and np.all(q == 0)
    q, sc = O.quant_token(np.full(64, -0.7, np.float16))
    assert np.all(q == -127)


def test_quant_invariants_random():
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = (rng.standard_normal(512) * rng.uniform(0.01, 100)).astype(np.float16)
        q, sc = O.quant_token(x)
        v = x.astype(np.float64)
        assert np.abs(q).max() <= 127
        assert abs(int(q[np.argmax(np.abs(v))])) == 127
        assert np.all((np.sign(q) == np.sign(v)) | (q == 0))
        assert sc == np.float32(np.float32(np.abs(v).max()) / np.float32(127))
        err = np.abs(q.astype(np.float64) * float(sc) - v)
        assert np.all(err <= float(sc) * (0.5 + 1e-5))
        qb, scb = BF.quant(x)
        assert np.array_equal(q, qb) and sc == scb


# ----------------------------------------------------------------------------
# GMM1 / GMM2 row: exact int32 accumulators + per-channel dequant to half
# ----------------------------------------------------------------------------
def test_gmm_row_hand_example():
    a = np.array([1, 2], np.int8)
    w = np.array([[1, 0, 3], [2, -1, 1]], np.int8)
    scale = np.array([0.5, 1.0, 0.25], np.float32)
    acc, c = O.gmm_row(a, w, scale)
    assert acc.tolist() == [5, -2, 5]
    assert c.tolist() == [2.5, -2.0, 1.25]


def test_gmm_row_exact_vs_float64_matmul():
    rng = np.random.default_rng(4)
    Kred, N = 384, 96
    w = rng.integers(-127, 128, (Kred, N), dtype=np.int8)
    scale = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    for extreme in (False, True):
        a = rng.integers(-127, 128, Kred, dtype=np.int8)
        if extreme:
            a[:] = 127
            w2 = np.full_like(w, -127)
        else:
            w2 = w
        acc, c = O.gmm_row(a, w2, scale)
        ref = a.astype(np.float64) @ w2.astype(np.float64)   # exact: partial sums < 2^53
        assert np.array_equal(acc, ref.astype(np.int32))
        exact = ref * scale.astype(np.float64)
        rel = np.abs(c.astype(np.float64) - exact) / np.abs(exact).clip(1e-30)
        assert np.all(rel <= 2.0 ** -11 + 2.0 ** -23)


def test_gmm_row_one_hot_column():
    rng = np.random.default_rng(6)
    a = rng.integers(-127, 128, 64, dtype=np.int8)
    w = np.zeros((64, 8), np.int8)
    for n in range(8):
        w[(n * 7) % 64, n] = n - 3
    acc, _ = O.gmm_row(a, w, np.ones(8, np.float32))
    assert acc.tolist() == [int(a[(n * 7) % 64]) * (n - 3) for n in range(8)]


# ----------------------------------------------------------------------------
# SwiGLU + dynamic re-quant (CAST_RINT)
# ----------------------------------------------------------------------------
def test_swiglu_hand_example_halves_and_rint():
    # u = 32 makes silu(u) == u exactly in fp32 (exp(-32) vanishes next to 1),
    # so y = 32 * g exactly: y = [127, 2.5, 3.5], maxAbs = 127, multiplier 1.
    c = np.array([32, 32, 32, 127 / 32, 2.5 / 32, 3.5 / 32], np.float16)
    q2, p2 = O.swiglu_quant_row(c, 1.0)
    assert p2 == np.float32(1.0)
    assert q2.tolist() == [127, 2, 4]          # ties to even (CAST_RINT)


def test_swiglu_first_half_is_silu():
    # u = [0, 20, -20, 1], g = [3, 2, 5, 1] -> y = [0, 40, ~-2e-7, 0.731]
    c = np.array([0, 20, -20, 1, 3, 2, 5, 1], np.float16)
    q2, p2 = O.swiglu_quant_row(c, 1.0)
    assert p2 == np.float32(np.float32(40.0) / np.float32(127.0))
    # 0.7310586 * 127/40 = 2.321
    assert q2.tolist() == [0, 127, 0, 2]
    # pts1 is applied before the activation: doubling it is not linear in y
    q2b, p2b = O.swiglu_quant_row(c, 2.0)
    # u' = [0, 40, -40, 2], g' = [6, 4, 10, 2]: y' = [0, 160, ~0, 2*1.7616*...]
    y3 = 2.0 / (1 + np.exp(-2.0)) * 2.0
    assert q2b.tolist() == [0, 127, 0, int(np.rint(y3 * 127 / 160))]


def test_swiglu_invariants_and_bound_random():
    rng = np.random.default_rng(7)
    for _ in range(10):
        I = 256
        c = (rng.standard_normal(2 * I) * 500).astype(np.float16)
        pts1 = np.float32(rng.uniform(0.005, 0.05))
        q2, p2 = O.swiglu_quant_row(c, pts1)
        assert np.abs(q2).max() == 127
        cc = c.astype(np.float64) * float(pts1)
        u, g = cc[:I], cc[I:]
        y = u / (1 + np.exp(-u)) * g
        assert abs(float(p2) - np.abs(y).max() / 127) <= 1e-5 * np.abs(y).max() / 127
        err = np.abs(q2 * float(p2) - y)
        assert np.all(err <= float(p2) * (0.5 + 1e-3))
        qb, pb, _ = BF.swiglu_quant(c, pts1)
        assert pb == p2
        assert np.abs(qb.astype(int) - q2.astype(int)).max() <= 1


def test_swiglu_zero_row():
    q2, p2 = O.swiglu_quant_row(np.zeros(16, np.float16), 0.3)
    assert p2 == 0 and np.all(q2 == 0)


# ----------------------------------------------------------------------------
# Combine dequant + Unpermute
# ----------------------------------------------------------------------------
def test_unpermute_hand_example():
    g = np.array([[1, 2], [3, 4]], np.float16)
    pts2 = np.array([0.5, 2.0], np.float32)
    out, outf = O.unpermute_token(np.array([0, 1], np.int32), np.array([0.25, 0.75], np.float32),
                                  g, pts2)
    # v0 = [0.5, 1], v1 = [6, 8]; 0.25 v0 + 0.75 v1 = [4.625, 6.25]
    assert outf.tolist() == [4.625, 6.25]
    assert O.bf16_to_f32(out).tolist() == [4.625, 6.25]


def test_unpermute_one_hot_zero_and_invalid():
    rng = np.random.default_rng(8)
    g = (rng.standard_normal((5, 64)) * 300).astype(np.float16)
    pts2 = rng.uniform(10, 100, 5).astype(np.float32)
    # one-hot prob: out is the bf16 of that row's dequant
    out, _ = O.unpermute_token(np.array([3, 1, 4], np.int32), np.array([0, 1, 0], np.float32), g,
                               pts2)
    assert np.array_equal(out, BF.to_bf16_bits(g[1].astype(np.float32) * pts2[1]))
    # zero probs -> zero
    out, outf = O.unpermute_token(np.array([3, 1], np.int32), np.zeros(2, np.float32), g, pts2)
    assert np.all(outf == 0)
    # invalid rows are skipped
    out_a, _ = O.unpermute_token(np.array([-1, 2], np.int32), np.array([0.9, 0.1], np.float32), g,
                                 pts2)
    out_b, _ = O.unpermute_token(np.array([2], np.int32), np.array([0.1], np.float32), g, pts2)
    assert np.array_equal(out_a, out_b)


def test_unpermute_linear_in_probs():
    rng = np.random.default_rng(9)
    g = (rng.standard_normal((4, 128)) * 300).astype(np.float16)
    pts2 = rng.uniform(10, 100, 4).astype(np.float32)
    rows = np.array([0, 1, 2, 3], np.int32)
    p = rng.dirichlet(np.ones(4)).astype(np.float32)
    _, outf = O.unpermute_token(rows, p, g, pts2)
    v = BF.to_bf16_f32(g.astype(np.float32) * pts2[:, None]).astype(np.float64)
    ref = (p.astype(np.float64)[:, None] * v).sum(0)
    assert np.all(np.abs(outf - ref) <= 1e-6 * np.abs(v).max() * 4)


# ----------------------------------------------------------------------------
# whole forward
# ----------------------------------------------------------------------------
def _check_forward_vs_bruteforce(inp, o, tokens):
    for t in tokens:
        b = BF.forward_token(inp, t)
        eri = o["expanded_row_idx"][t * inp["expert_idx"].shape[1]:][:inp["expert_idx"].shape[1]]
        for s, d in enumerate(eri):
            sl = b["slots"][s]
            if d < 0:
                assert sl is None
                continue
            assert np.array_equal(o["gmA"][d], b["qa"]) and o["pts1"][d] == b["pts1"]
            assert np.array_equal(o["acc1"][d], sl["acc1"])
            assert np.array_equal(o["gmC"][d].view(np.uint16), sl["gmC"].view(np.uint16))
            assert np.abs(o["q2"][d].astype(int) - sl["q2"].astype(int)).max() <= 1
            assert np.array_equal(o["acc2"][d], sl["acc2"]) or \
                np.abs(o["q2"][d].astype(int) - sl["q2"].astype(int)).max() == 1
        ref = b["out_f32"]
        assert np.abs(o["out_f32"][t] - ref).max() <= 1e-3 * max(np.abs(ref).max(), 1e-6)


def test_forward_tiny_vs_bruteforce():
    w = W.WORKLOADS["tiny"]
    inp = W.generate(w, 0)
    o = O.forward(inp)
    assert o["dropped"] == 0
    _check_sort_invariants(inp["expert_idx"], w.E, o)
    _check_forward_vs_bruteforce(inp, o, range(w.M))
    # out is the bf16 rounding of out_f32
    assert np.array_equal(o["out"], BF.to_bf16_bits(o["out_f32"]))


def test_forward_token_matches_forward():
    w = W.custom(24, 256, 6, 3, 128, routing="zipf")
    inp = W.generate(w, 3)
    o = O.forward(inp)
    for t in (0, 7, 23):
        ot = O.forward_token(inp, t)
        assert np.array_equal(ot["out"], o["out"][t])
        for s in range(w.top_k):
            d = o["expanded_row_idx"][t * w.top_k + s]
            assert np.array_equal(ot["acc1"][s], o["acc1"][d])
            assert np.array_equal(ot["q2"][s], o["q2"][d])


def test_forward_dense_special_case():
    # E = 1, topK = 1, prob 1: the pipeline is a plain dense quantised FFN
    w = W.custom(8, 128, 1, 1, 128)
    inp = W.generate(w, 11)
    inp["probs"][:] = 1.0
    o = O.forward(inp)
    assert np.array_equal(o["sorted_route"], np.arange(8))
    qa = np.stack([BF.quant(inp["x"][t])[0] for t in range(8)])
    acc1 = qa.astype(np.float64) @ inp["w1"][0].astype(np.float64)
    assert np.array_equal(o["acc1"], acc1.astype(np.int32))
    acc2 = o["q2"].astype(np.float64) @ inp["w2"][0].astype(np.float64)
    assert np.array_equal(o["acc2"], acc2.astype(np.int32))
    ref = BF.to_bf16_f32(o["gmm2_out"].astype(np.float32) * o["pts2"][:, None])
    assert np.array_equal(o["out_f32"], ref)


def test_forward_invalid_expert_dropped():
    w = W.custom(6, 128, 4, 2, 128)
    inp = W.generate(w, 12)
    inp["expert_idx"][2, 1] = 9
    inp["expert_idx"][4, 0] = -3
    o = O.forward(inp)
    assert o["dropped"] == 2
    _check_sort_invariants(inp["expert_idx"], w.E, o)
    _check_forward_vs_bruteforce(inp, o, range(w.M))


def test_forward_unquantised_sanity():
    w = W.WORKLOADS["tiny"]
    inp = W.generate(w, 0)
    o = O.forward(inp)
    rel = []
    for t in range(w.M):
        ref = BF.forward_unquantised_f64(inp, t)
        rel.append(np.linalg.norm(o["out_f32"][t] - ref) / np.linalg.norm(ref))
    # int8 activations on both GEMMs: a few percent relative error is expected
    assert max(rel) < 0.08, max(rel)
