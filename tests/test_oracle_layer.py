"""Pins of the oracle's layer steps: router front (top-k with ties to the lower id,
softmax weights), SwiGLU clamp, and the fused (order-free) finalize; plus the general
recipe pipeline against the pinned per-token pipeline."""
import math

import numpy as np
import pytest

import synth
from oracle.formats import bf16_to_f32
from oracle.layer import finalize_fused, router_topk, swiglu_clamp
from oracle.moe import brute_force_moe, dequant_activation, dequant_weights, finalize, prepare_weights, routed_moe
from oracle.quant import dequantize_rows, quantize_input_per_token, quantize_rows_f32
from oracle.recipes import routed_moe_recipe

F32 = np.float32


# ----------------------------------------------------------------------------- router
def _router_brute(logits, k, renorm):
    ids, ws = [], []
    for row in logits:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]
        m = max(float(v) for v in row)
        den = sum(math.exp(float(v) - m) for v in row)
        w = [np.float32(math.exp(float(row[e]) - m) / den) for e in order]
        if renorm:
            s = np.float32(0.0)
            for v in w:
                s = np.float32(s + v)
            w = [np.float32(v / s) for v in w]
        ids.append(order)
        ws.append(w)
    return np.array(ids, np.int32), np.array(ws, F32)


@pytest.mark.parametrize("renorm", [False, True])
def test_router_matches_brute_force(renorm):
    rng = np.random.default_rng(41)
    lg = rng.standard_normal((50, 37)).astype(F32)
    lg[3, [4, 9, 20]] = 5.0                      # ties at the top: lower ids first
    lg[7, :] = 0.0                               # all equal: ids 0..k-1
    lg[11, [2, 30]] = -1e30                      # huge negative logits
    ids, w = router_topk(lg, 5, renorm)
    bi, bw = _router_brute(lg, 5, renorm)
    assert np.array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=2e-7, atol=0)
    assert list(ids[3, :3]) == [4, 9, 20] and list(ids[7]) == [0, 1, 2, 3, 4]
    if renorm:
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_router_topk_of_logits_is_topk_of_probabilities():
    rng = np.random.default_rng(42)
    lg = (rng.standard_normal((40, 64)) * 3).astype(F32)
    ids, _ = router_topk(lg, 6)
    p = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    want = np.argsort(-p, axis=1, kind="stable")[:, :6]
    assert np.array_equal(ids, want)


def test_router_matches_synthetic_inputs_generator():
    """The seeded generator draws its top-k the same way (softmax, descending, lower id)."""
    w = synth.WORKLOADS["ep4_t512"]
    ids, wts = synth.router(w, 64)
    lg = synth.router_logits(w, 64)
    rid, rw = router_topk(lg, w.K, w.renormalize)
    assert np.array_equal(rid, ids)
    np.testing.assert_allclose(rw, wts, rtol=1e-6)


# ----------------------------------------------------------------------------- clamp
def test_swiglu_clamp_values():
    g = np.array([-20, -1, 0, 9.5, 10, 25], F32)
    u = np.array([-30, -10, -9, 0, 11, 10], F32)
    cg, cu = swiglu_clamp(g, u, 10.0)
    assert list(cg) == [-20, -1, 0, 9.5, 10, 10]
    assert list(cu) == [-10, -10, -9, 0, 10, 10]
    ng, nu = swiglu_clamp(g, u, 0.0)
    assert np.array_equal(ng, g) and np.array_equal(nu, u)


# ----------------------------------------------------------------------------- pipelines
def _case(seed, T=12, H=64, I=32, E=4, K=2, act="swiglu", scale=1.0):
    rng = np.random.default_rng(seed)
    x = synth._bf16_np((rng.standard_normal((T, H)) * scale).astype(F32))
    N1 = 2 * I if act == "swiglu" else I
    w1 = synth._bf16_np((rng.standard_normal((E, N1, H)) * 0.3).astype(F32))
    w2 = synth._bf16_np((rng.standard_normal((E, H, I)) * 0.05).astype(F32))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    wts = rng.dirichlet(np.ones(K), T).astype(F32)
    return x, w1, w2, ids, wts


@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_general_pipeline_equals_pinned_per_token(act):
    x, w1, w2, ids, wts = _case(43, act=act)
    q = quantize_input_per_token(x)
    W = prepare_weights(w1, w2)
    a = routed_moe(*q, ids, wts, W, act)
    b = routed_moe_recipe("per_token", q, ids, wts, W, act)
    for f in ("out", "h", "hq", "h_sf", "z"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert np.array_equal(routed_moe_recipe("per_token", q, ids, wts, W, act, swiglu_limit=1e30).out, a.out)


def _qh(h):
    q, s, g = quantize_rows_f32(np.asarray(h, F32))
    return dequantize_rows(q, s, g).astype(np.float64)


def test_clamped_pipeline_equals_brute_force():
    x, w1, w2, ids, wts = _case(44, scale=4.0)
    q = quantize_input_per_token(x)
    W = prepare_weights(w1, w2)
    limit = 2.0
    res = routed_moe_recipe("per_token", q, ids, wts, W, "swiglu", swiglu_limit=limit)
    y_gate = res.h  # sanity: the clamp changes the result on these inputs
    assert not np.array_equal(res.out, routed_moe_recipe("per_token", q, ids, wts, W, "swiglu").out)
    bf = brute_force_moe(bf16_to_f32(x), ids, wts, bf16_to_f32(w1), bf16_to_f32(w2), "swiglu",
                         quantize=(dequant_activation, dequant_weights, dequant_weights, _qh),
                         swiglu_limit=limit)
    got = bf16_to_f32(res.out).astype(np.float64)
    for t in range(got.shape[0]):
        assert np.abs(got[t] - bf[t]).max() <= 1e-2 * np.abs(bf[t]).max()
    assert y_gate.shape[0] == ids.size


def test_fused_finalize_equals_exact_sum_of_fp32_terms():
    rng = np.random.default_rng(45)
    T, K, H, R = 9, 3, 32, 20
    zf = (rng.standard_normal((R, H)) * 10).astype(F32)
    rr = rng.permutation(T * K)[: T * K].astype(np.int32) % R
    rr[rng.random(T * K) < 0.2] = -1
    w = rng.random((T, K)).astype(F32)
    got = bf16_to_f32(finalize_fused(zf, rr, w, T, K))
    for t in range(T):
        acc = 0.0
        for j in range(K):
            r = rr[t * K + j]
            if r >= 0:
                acc += np.float64(np.float32(w[t, j] * zf[r]))   # exact products, any order
        want = bf16_to_f32(synth._bf16_np(np.asarray(acc, F32)))
        assert np.array_equal(got[t], want)


def test_fused_finalize_closed_form_on_exact_terms():
    """Integer z values and weights 1 or 2: every product and every partial
    sum is an integer of magnitude at most 64, exact in FP32 and in BF16, so
    the order-free finalize must return the integer sums themselves (computed
    here with Python integers), skip invalid routes, and give +0 for a token
    with none."""
    rng = np.random.default_rng(47)
    T, K, H, R = 6, 4, 16, 12
    zi = rng.integers(-8, 9, (R, H))
    wi = rng.integers(1, 3, (T, K))
    rr = rng.integers(0, R, T * K).astype(np.int32)
    rr[[1, 6, 7]] = -1
    rr[4 * K:5 * K] = -1                                 # token 4: no valid route
    got = bf16_to_f32(finalize_fused(zi.astype(np.float32), rr, wi.astype(np.float32), T, K))
    for t in range(T):
        want = [0] * H
        for j in range(K):
            r = int(rr[t * K + j])
            if r >= 0:
                want = [want[n] + int(wi[t, j]) * int(zi[r, n]) for n in range(H)]
        assert got[t].tolist() == [float(v) for v in want], t
    assert not np.signbit(got[4]).any() and not got[4].any()


def test_fused_pipeline_close_to_ordered_and_brute_force():
    x, w1, w2, ids, wts = _case(46, T=16, act="relu2")
    q = quantize_input_per_token(x)
    W = prepare_weights(w1, w2)
    o = routed_moe_recipe("per_token", q, ids, wts, W, "relu2")
    f = routed_moe_recipe("per_token", q, ids, wts, W, "relu2", finalize_mode="fused")
    go, gf = (bf16_to_f32(r.out).astype(np.float64) for r in (o, f))
    # the two finalizes differ only by the BF16 rounding of z and the sum's rounding
    assert np.all(np.abs(gf - go) <= 2 ** -7 * np.abs(go).max(axis=1, keepdims=True))
    bf = brute_force_moe(bf16_to_f32(x), ids, wts, bf16_to_f32(w1), bf16_to_f32(w2), "relu2",
                         quantize=(dequant_activation, dequant_weights, dequant_weights, _qh))
    for t in range(gf.shape[0]):
        assert np.abs(gf[t] - bf[t]).max() <= 1e-2 * np.abs(bf[t]).max()
