"""Pins of the oracle's per-tensor and weight-only (W4A16) recipes.

per_tensor : the static-scale quantizer equals the pinned per-token quantizer
             whenever the two row scales coincide, is exact on values it can
             represent, is power-of-two equivariant and saturates as E4M3 / E2M1
             do; folded alphas reduce to the unfolded ones at a = 1 and invert
             w_scale * a to rounding; the pipeline equals a per-token brute
             force on dequantized tensors.
weight_only: on weights NVFP4 represents exactly, the pipeline is the textbook
             MoE with a BF16 intermediate (brute force, no quantization); on
             general weights it equals the brute force on dequantized weights.
"""
import numpy as np
import pytest

import synth
from oracle.formats import bf16_to_f32, e4m3_decode, f32_to_bf16_rne, unpack_nibbles
from oracle.moe import (bf16_reference_moe, brute_force_moe, dequant_weights, prepare_weights,
                        routed_moe)
from oracle.quant import (dequantize_blocks, quantize_input_per_token, quantize_rows_f32,
                          quantize_weights, weight_global_scale)
from oracle.recipes import (dequant_static, fold_input_scale, prepare_weights_per_tensor,
                            quantize_input_per_tensor, quantize_rows_static, routed_moe_recipe,
                            static_row_scale)

F32 = np.float32
E2M1_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _bf16(x):
    return synth._bf16_np(np.asarray(x, F32))


def _scale_for(g):
    """A float32 a with fp32(1/a) == g, or None."""
    a0 = F32(F32(1.0) / g)
    for a in (a0, np.nextafter(a0, F32(0)), np.nextafter(a0, F32(np.inf))):
        if static_row_scale(a) == g:
            return F32(a)
    return None


# ----------------------------------------------------------------------------- static quantizer
def test_static_equals_per_token_when_row_scales_coincide():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal((40, 256)),
                        np.exp(rng.uniform(-12, 12, (10, 256))) * rng.choice([-1, 1], (10, 256))]).astype(F32)
    q, sf, g = quantize_rows_f32(x)
    hits = 0
    for r in range(x.shape[0]):
        a = _scale_for(g[r])
        if a is None:
            continue
        hits += 1
        qs, ss = quantize_rows_static(x[r:r + 1], a)
        assert np.array_equal(qs[0], q[r]) and np.array_equal(ss[0], sf[r])
    assert hits >= 40


def _representable_rows(rng, R, L, m):
    """Rows whose every 16-block is grid * s * 2^m with block max 6 and E4M3 s; one block s = 448."""
    nb = L // 16
    s_vals = e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    rows = np.empty((R, L), np.float64)
    for r in range(R):
        s = rng.choice(s_vals, nb)
        s[rng.integers(nb)] = 448.0
        v = rng.choice(E2M1_GRID, (nb, 16)) * rng.choice([-1, 1], (nb, 16))
        v[np.arange(nb), rng.integers(0, 16, nb)] = 6.0
        rows[r] = (v * s[:, None]).reshape(-1) * 2.0 ** m
    return rows.astype(F32)


@pytest.mark.parametrize("m", [-20, -9, 0, 7])
def test_static_quantizer_exact_on_representable_values(m):
    """a = 2^-m: every block scale and code is exact, so dequant(quant(x)) == x bit for bit."""
    rng = np.random.default_rng(22 + m)
    x = _representable_rows(rng, 6, 128, m)
    a = F32(2.0 ** -m)
    q, sf = quantize_rows_static(x, a)
    xh = (dequantize_blocks(q, sf).astype(F32) * static_row_scale(a)).astype(F32)
    assert np.array_equal(xh, x)


def test_static_quantizer_power_of_two_equivariance():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((8, 128)).astype(F32)
    a = F32(2688.0 / 3.7)
    q0, s0 = quantize_rows_static(x, a)
    for m in (-15, -2, 3, 25):
        q1, s1 = quantize_rows_static((x * F32(2.0 ** m)).astype(F32), F32(a * F32(2.0 ** -m)))
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_static_quantizer_saturates_beyond_its_range():
    """With a calibrated for amax A, blocks above A saturate: scale 448, max code 6."""
    rng = np.random.default_rng(24)
    x = rng.standard_normal((4, 256)).astype(F32)
    a = F32(2688.0 / 0.5)                       # calibrated far below the real amax
    q, sf = quantize_rows_static(x, a)
    codes = unpack_nibbles(q).reshape(4, 16, 16)
    g = np.float64(static_row_scale(a))
    amax_b = np.abs(x.astype(np.float64)).reshape(4, 16, 16).max(axis=2)
    hot = amax_b / 6 / g > 448
    assert hot.any()
    assert np.all(sf[hot] == 0x7E)
    big = np.abs(x.reshape(4, 16, 16)) > 6 * 448 * g * (1 + 1e-6)
    assert np.all((codes[big] & 7) == 7)        # clipped to +-6
    xh = dequantize_blocks(q, sf) * g
    assert np.abs(xh).max() <= 6 * 448 * g * (1 + 1e-6)


def test_static_quantizer_roundtrip_bound_when_calibrated():
    rng = np.random.default_rng(25)
    x = (rng.standard_normal((20, 256)) * rng.uniform(0.1, 3, (20, 1))).astype(F32)
    a = F32(F32(2688.0) / F32(np.abs(x).max()))
    q, sf = quantize_rows_static(x, a)
    g = static_row_scale(a)
    xh = (dequantize_blocks(q, sf).astype(F32) * g).astype(np.float64)
    e = np.repeat((e4m3_decode(sf).astype(F32) * g).astype(np.float64), 16, axis=1)
    assert np.all(np.abs(x - xh) <= e * (1 + 2.0 ** -19))


def test_per_tensor_input_quantizer_reads_bf16():
    rng = np.random.default_rng(26)
    xb = _bf16(rng.standard_normal((3, 64)))
    a = F32(1000.0)
    q, s = quantize_input_per_tensor(xb, a)
    q2, s2 = quantize_rows_static(bf16_to_f32(xb), a)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ----------------------------------------------------------------------------- folding
def test_fold_input_scale():
    rng = np.random.default_rng(27)
    w = _bf16(rng.standard_normal((5, 32, 64)) * rng.uniform(0.01, 2, (5, 1, 1)))
    _, _, alpha = quantize_weights(w)
    assert np.array_equal(fold_input_scale(w, F32(1.0)), alpha)          # a = 1: unchanged
    for a in (F32(3.0), F32(2688.0 / 7.3), F32(1e-3)):
        got = fold_input_scale(w, a).astype(np.float64)
        for e in range(5):
            _, w_scale = weight_global_scale(bf16_to_f32(w[e]))
            assert abs(got[e] * float(w_scale) * float(a) - 1.0) <= 3 * 2.0 ** -24
    z = np.zeros((1, 32, 64), np.uint16)
    assert fold_input_scale(z, F32(5.0))[0] == 0.0                        # all-zero expert


def test_prepare_per_tensor_keeps_codes():
    rng = np.random.default_rng(28)
    w1 = _bf16(rng.standard_normal((3, 64, 64)) * 0.05)
    w2 = _bf16(rng.standard_normal((3, 64, 32)) * 0.05)
    P = prepare_weights(w1, w2)
    Q = prepare_weights_per_tensor(w1, w2, F32(50.0), F32(70.0))
    for f in ("w1q", "w1sf", "w2q", "w2sf"):
        assert np.array_equal(getattr(P, f), getattr(Q, f))
    assert np.array_equal(Q.a1, fold_input_scale(w1, F32(50.0)))
    assert np.array_equal(Q.a2, fold_input_scale(w2, F32(70.0)))


# ----------------------------------------------------------------------------- pipelines
def _case(T, H, I, E, K, act, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)) * rng.uniform(0.3, 2, (T, 1)))
    N1 = 2 * I if act == "swiglu" else I
    w1 = _bf16(rng.standard_normal((E, N1, H)) * 0.05)
    w2 = _bf16(rng.standard_normal((E, H, I)) * 0.05)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    wts = rng.dirichlet(np.ones(K), T).astype(F32)
    return x, w1, w2, ids, wts


def _close_per_token(got_bits, want, tol, med):
    got = bf16_to_f32(got_bits).astype(np.float64)
    for t in range(got.shape[0]):
        assert np.abs(got[t] - want[t]).max() <= tol * np.abs(want[t]).max() + 1e-30
    rel = np.abs(got - want) / (np.abs(want).max(axis=1, keepdims=True) + 1e-30)
    assert np.median(rel) < med


@pytest.mark.parametrize("T,H,I,E,K,act", [(3, 32, 16, 2, 2, "relu2"), (5, 64, 32, 3, 2, "swiglu"),
                                           (16, 256, 128, 4, 2, "relu2")])
def test_per_tensor_pipeline_equals_brute_force(T, H, I, E, K, act):
    x, w1, w2, ids, wts = _case(T, H, I, E, K, act, seed=T + H)
    a1 = F32(F32(2688.0) / F32(np.abs(bf16_to_f32(x)).max()))
    a2 = F32(2688.0 / 0.02)
    xq, xs = quantize_input_per_tensor(x, a1)
    W = prepare_weights_per_tensor(w1, w2, a1, a2)
    res = routed_moe_recipe("per_tensor", (xq, xs), ids, wts, W, act, a2=a2)
    bf = brute_force_moe(bf16_to_f32(x), ids, wts, bf16_to_f32(w1), bf16_to_f32(w2), act,
                         quantize=(lambda v: dequant_static(v, a1), dequant_weights, dequant_weights,
                                   lambda h: dequant_static(h, a2)))
    _close_per_token(res.out, bf, 1e-2, 3e-3)


@pytest.mark.parametrize("T,H,I,E,K,act", [(3, 32, 16, 2, 2, "relu2"), (5, 64, 32, 3, 2, "swiglu"),
                                           (16, 256, 128, 4, 2, "relu2")])
def test_weight_only_pipeline_equals_brute_force(T, H, I, E, K, act):
    x, w1, w2, ids, wts = _case(T, H, I, E, K, act, seed=T * 3 + H)
    res = routed_moe_recipe("weight_only", x, ids, wts, prepare_weights(w1, w2), act)
    to_bf16 = lambda h: bf16_to_f32(f32_to_bf16_rne(np.asarray(h, F32))).astype(np.float64)
    bf = brute_force_moe(bf16_to_f32(x), ids, wts, bf16_to_f32(w1), bf16_to_f32(w2), act,
                         quantize=(lambda v: np.asarray(v, np.float64), dequant_weights, dequant_weights,
                                   to_bf16))
    _close_per_token(res.out, bf, 1e-2, 1e-3)


def _representable_weights(rng, E, N, K, m):
    w = np.stack([_representable_rows(rng, N, K, m) for _ in range(E)])
    assert np.all(np.abs(w).max(axis=(1, 2)) == F32(2688.0 * 2.0 ** m))   # so alpha = 2^m exactly
    return w


def test_weight_only_is_textbook_moe_on_representable_weights():
    """Weights NVFP4 holds exactly: W4A16 == the BF16-intermediate MoE with no quantization."""
    rng = np.random.default_rng(29)
    T, H, I, E, K = 6, 64, 32, 3, 2
    for act in ("relu2", "swiglu"):
        N1 = 2 * I if act == "swiglu" else I
        w1 = _representable_weights(rng, E, N1, H, -14)
        w2 = _representable_weights(rng, E, H, I, -13)
        w1b, w2b = _bf16(w1), _bf16(w2)
        assert np.array_equal(bf16_to_f32(w1b), w1)              # exact in BF16
        W = prepare_weights(w1b, w2b)
        assert np.array_equal(dequant_weights(w1), w1.astype(np.float64))
        x = _bf16(rng.standard_normal((T, H)))
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        wts = rng.dirichlet(np.ones(K), T).astype(F32)
        res = routed_moe_recipe("weight_only", x, ids, wts, W, act)
        to_bf16 = lambda h: bf16_to_f32(f32_to_bf16_rne(np.asarray(h, F32))).astype(np.float64)
        bf = brute_force_moe(bf16_to_f32(x), ids, wts, w1, w2, act,
                             quantize=(lambda v: np.asarray(v, np.float64), lambda w: w, lambda w: w,
                                       to_bf16))
        _close_per_token(res.out, bf, 1e-2, 1e-3)


def test_recipes_batch_invariance_and_plausibility():
    """Batch invariance of both recipes; per-token cosine to the unquantized MoE at the
    pages' bar (mean > 0.97, min > 0.95), with weight_only closer than per_token since
    it keeps BF16 activations."""
    w = synth.WORKLOADS["tiny"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    w1, w2 = synth.all_weights(w)
    ref = bf16_reference_moe(x, ids, wts, w1, w2, w.act)

    def cosine(bits):
        got = bf16_to_f32(bits).astype(np.float64)
        return np.sum(got * ref, 1) / (np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1))

    P = prepare_weights(w1, w2)
    xq, xs, xg = quantize_input_per_token(x)
    token_run = routed_moe(xq, xs, xg, ids, wts, P, w.act)
    cos_token = cosine(token_run.out)
    # calibrated static scales: 2688 / amax of the FC1 input and of the intermediate
    a1 = F32(F32(2688.0) / F32(np.abs(bf16_to_f32(x)).max()))
    a2 = F32(F32(2688.0) / F32(np.abs(token_run.h).max()))
    runs = {
        "weight_only": (lambda xs_, i, wt: routed_moe_recipe("weight_only", xs_, i, wt, P, w.act)),
        "per_tensor": (lambda xs_, i, wt: routed_moe_recipe(
            "per_tensor", quantize_input_per_tensor(xs_, a1), i, wt,
            prepare_weights_per_tensor(w1, w2, a1, a2), w.act, a2=a2)),
    }
    for name, run in runs.items():
        full = run(x, ids, wts).out
        for t in (0, 9):
            assert np.array_equal(run(x[t:t + 1], ids[t:t + 1], wts[t:t + 1]).out[0], full[t])
        cos = cosine(full)
        assert cos.mean() > 0.97 and cos.min() > 0.95, (name, cos.mean(), cos.min())
        if name == "weight_only":
            assert cos.mean() > cos_token.mean() and cos.min() > cos_token.min()


def test_recipe_rejects_unknown_and_mismatch():
    x, w1, w2, ids, wts = _case(2, 32, 16, 2, 1, "relu2", seed=1)
    with pytest.raises(ValueError):
        routed_moe_recipe("mxfp8", x, ids, wts, prepare_weights(w1, w2), "relu2")
    with pytest.raises(ValueError):
        routed_moe_recipe("weight_only", x, ids, wts, prepare_weights(w1, w2), "swiglu")
