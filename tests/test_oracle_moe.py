"""Pins of the oracle's MoE pipeline: gating, routing, exact GEMM sums, finalize order,
brute-force MoE agreement and plausibility against the unquantized MoE."""
import zlib

import numpy as np
import pytest

import synth
from oracle.formats import bf16_to_f32, f32_to_bf16_rne, e2m1_decode, e4m3_decode, unpack_nibbles
from oracle.moe import (Weights, activation, bf16_reference_moe, brute_force_moe, dequant_activation,
                        dequant_weights, detect_gating, fc, finalize, prepare_weights, route, routed_moe)
from oracle.quant import dequantize_rows, quantize_input_per_token, quantize_rows_f32

F32 = np.float32


# ----------------------------------------------------------------------------- gating
@pytest.mark.parametrize("n1,i,want", [(256, 128, True), (128, 128, False), (96, 48, True), (48, 48, False)])
def test_gating_accepts(n1, i, want):
    assert detect_gating(n1, i) is want


@pytest.mark.parametrize("n1,i,h1,h2", [(272, 128, 64, 64), (64, 128, 64, 64), (0, 0, 64, 64),
                                        (256, 128, 64, 32), (100, 0, 64, 64)])
def test_gating_rejects(n1, i, h1, h2):
    with pytest.raises(ValueError):
        detect_gating(n1, i, h1, h2)


# ----------------------------------------------------------------------------- routing
def _route_brute(ids, E, off):
    T, K = ids.shape
    rows = []
    for e in range(E):                      # experts in order, then flat routes in order
        for f in range(T * K):
            if ids.reshape(-1)[f] - off == e:
                rows.append(f)
    r_of = np.full(T * K, -1, np.int32)
    for r, f in enumerate(rows):
        r_of[f] = r
    counts = np.array([sum(1 for f in range(T * K) if ids.reshape(-1)[f] - off == e) for e in range(E)])
    return np.array(rows, np.int64), r_of, counts


@pytest.mark.parametrize("case", ["random", "one_expert", "empty_experts", "invalid", "offset", "int64"])
def test_routing_brute_force(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    T, K, E, off = 37, 4, 8, 0
    ids = rng.integers(0, E, (T, K))
    if case == "one_expert":
        ids[:] = 5
    elif case == "empty_experts":
        ids = rng.choice([1, 6], (T, K))
    elif case == "invalid":
        ids[rng.random((T, K)) < 0.3] = -1
        ids[0, 0] = E + 3
    elif case == "offset":
        off = 16
        ids = rng.integers(0, 40, (T, K))
    ids = ids.astype(np.int64 if case == "int64" else np.int32)
    rt = route(ids, E, off)
    rows, r_of, counts = _route_brute(ids, E, off)
    assert np.array_equal(rt.route_of_row, rows)
    assert np.array_equal(rt.row_of_route, r_of)
    assert np.array_equal(rt.counts, counts)
    valid = r_of >= 0
    assert sorted(r_of[valid].tolist()) == list(range(valid.sum()))      # bijection on valid routes
    assert np.array_equal(rt.offsets[1:] - rt.offsets[:-1], counts)


# ----------------------------------------------------------------------------- GEMM
def test_fc_equals_exact_integer_sum():
    """Decoded values are integers times 2^-10; an int64 matmul gives the exact sum."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((33, 512)) * np.exp(rng.uniform(-3, 3, (33, 1)))).astype(F32)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(F32)
    xq, xs, xg = quantize_rows_f32(x)
    from oracle.quant import quantize_weight_matrix
    wq, ws, wa = quantize_weight_matrix(synth._bf16_np(w))
    y = fc(xq, xs, xg, wq, ws, wa)

    def ints(q, s):
        v = e2m1_decode(unpack_nibbles(q)).reshape(q.shape[0], -1, 16) * e4m3_decode(s)[:, :, None]
        i = np.rint(v * 1024).astype(np.int64)
        assert np.array_equal(i / 1024.0, v)
        return i.reshape(q.shape[0], -1)

    exact = ints(xq, xs) @ ints(wq, ws).T                                  # exact, units of 2^-20
    acc = (exact.astype(np.float64) * 2.0 ** -20).astype(F32)             # one rounding (|exact| < 2^53)
    want = (acc * (xg * F32(wa)).astype(F32)[:, None]).astype(F32)
    assert np.mean(y == want) > 0.9999
    assert np.all(np.abs(y - want) <= np.spacing(np.abs(want)) + 0)


# ----------------------------------------------------------------------------- activation
def test_activation_values():
    y = np.array([[-2.0, 0.0, 3.0, -0.0]], F32)
    assert activation(y, "relu2", 4).tolist() == [[0.0, 0.0, 9.0, 0.0]]
    g = np.array([[0.0, 1.0, -100.0]], F32)
    u = np.array([[5.0, 2.0, 3.0]], F32)
    h = activation(np.concatenate([g, u], axis=1), "swiglu", 3)
    assert h[0, 0] == 0.0
    assert abs(h[0, 1] - 2.0 / (1 + np.exp(-1.0))) < 1e-6
    assert h[0, 2] == F32(-100.0 / (1 + np.exp(100.0)) * 3.0) or abs(h[0, 2]) < 1e-30


# ----------------------------------------------------------------------------- finalize
def _z(vals):
    return f32_to_bf16_rne(np.array(vals, F32))


def test_finalize_slot_order():
    """Slot order [2^24, 1, -2^24] gives 0 (2^24 + 1 rounds back to 2^24); expert order would give 1."""
    z = _z([[2.0 ** 24], [1.0], [-2.0 ** 24]])
    # rows stored in expert order C, B, A; the token's slots point at A, B, C
    z_rows = z[[2, 1, 0]]
    row_of_route = np.array([2, 1, 0], np.int32)
    out = finalize(z_rows, row_of_route, np.ones((1, 3), F32), 1, 3)
    assert out.tolist() == [[0]]
    out_rev = finalize(z_rows, np.array([0, 1, 2], np.int32), np.ones((1, 3), F32), 1, 3)
    assert bf16_to_f32(out_rev).tolist() == [[1.0]]


def test_finalize_no_fused_multiply_add():
    """w1*z1 = 1 + 2^-7 + 2^-20 + 2^-27 rounds to drop 2^-27; a fused op would leave 2^-27."""
    w = np.array([[1 + 2.0 ** -7 + 2.0 ** -20, 1 + 2.0 ** -20]], F32)
    z = _z([[-1.0], [1 + 2.0 ** -7]])
    out = finalize(z, np.array([0, 1], np.int32), w, 1, 2)
    assert out.tolist() == [[0x0000]]


def test_finalize_invalid_routes_and_sign_of_zero():
    z = _z([[-0.0, 3.0]])
    out = finalize(z, np.array([-1, 0, -1, -1], np.int32), np.array([[9.0, 1.0], [1.0, 1.0]], F32), 2, 2)
    assert out[0].tolist() == [0x0000, 0x4040]           # +0 + (-0) = +0
    assert out[1].tolist() == [0x0000, 0x0000]           # no valid route -> +0


# ----------------------------------------------------------------------------- whole MoE
def _small_case(T, H, I, E, K, act, seed, offset=0, invalid=0.0):
    rng = np.random.default_rng(seed)
    x = synth._bf16_np((rng.standard_normal((T, H)) * rng.uniform(0.1, 3, (T, 1))).astype(F32))
    N1 = 2 * I if act == "swiglu" else I
    w1 = synth._bf16_np((rng.standard_normal((E, N1, H)) * 0.05).astype(F32))
    w2 = synth._bf16_np((rng.standard_normal((E, H, I)) * 0.05).astype(F32))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32) + offset
    ids[rng.random((T, K)) < invalid] = -1
    wts = rng.dirichlet(np.ones(K), T).astype(F32)
    return x, w1, w2, ids, wts


def _run_oracle(x, w1, w2, ids, wts, act, offset=0):
    xq, xs, xg = quantize_input_per_token(x)
    W = prepare_weights(w1, w2)
    return routed_moe(xq, xs, xg, ids, wts, W, act, offset)


def _qh(h):
    q, s, g = quantize_rows_f32(np.asarray(h, F32))
    return dequantize_rows(q, s, g).astype(np.float64)


@pytest.mark.parametrize("T,H,I,E,K,act", [(1, 32, 16, 2, 1, "relu2"), (3, 32, 16, 2, 2, "relu2"),
                                           (3, 32, 16, 2, 2, "swiglu"), (16, 256, 128, 4, 2, "relu2"),
                                           (9, 64, 32, 3, 2, "swiglu"), (6, 128, 64, 5, 3, "relu2")])
def test_pipeline_equals_brute_force(T, H, I, E, K, act):
    x, w1, w2, ids, wts = _small_case(T, H, I, E, K, act, seed=T * 100 + H + K)
    res = _run_oracle(x, w1, w2, ids, wts, act)
    got = bf16_to_f32(res.out).astype(np.float64)
    bf = brute_force_moe(bf16_to_f32(x), ids, wts, bf16_to_f32(w1), bf16_to_f32(w2), act,
                         quantize=(dequant_activation, dequant_weights, dequant_weights, _qh))
    for t in range(T):
        scale = np.abs(bf[t]).max()
        assert np.abs(got[t] - bf[t]).max() <= 1e-2 * scale + 1e-30
    rel = np.abs(got - bf) / (np.abs(bf).max(axis=1, keepdims=True) + 1e-30)
    assert np.median(rel) < 3e-3


def test_brute_force_is_textbook_moe():
    """With identity quantization the brute force equals an independent einsum formulation."""
    T, H, I, E, K = 5, 32, 16, 3, 2
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, H))
    for act in ("relu2", "swiglu"):
        N1 = 2 * I if act == "swiglu" else I
        w1 = rng.standard_normal((E, N1, H)) * 0.1
        w2 = rng.standard_normal((E, H, I)) * 0.1
        ids = np.array([[0, 2], [1, 1], [2, 0], [1, 0], [0, -1]])
        wts = rng.random((T, K))
        for limit in ((0.0, 0.3) if act == "swiglu" else (0.0,)):
            got = brute_force_moe(x, ids, wts, w1, w2, act, swiglu_limit=limit)
            want = np.zeros((T, H))
            for j in range(K):
                e = np.clip(ids[:, j], 0, E - 1)
                y = np.einsum("tnh,th->tn", w1[e], x)
                if act == "relu2":
                    h = np.maximum(y, 0) ** 2
                else:
                    g, u = y[:, :I], y[:, I:]
                    if limit:
                        g, u = np.where(g > limit, limit, g), np.where(u > limit, limit,
                                                                        np.where(u < -limit, -limit, u))
                    h = g * (1 / (1 + np.exp(-g))) * u
                z = np.einsum("thi,ti->th", w2[e], h)
                want += np.where(ids[:, j:j + 1] >= 0, wts[:, j:j + 1] * z, 0)
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
            if limit:
                assert not np.allclose(got, brute_force_moe(x, ids, wts, w1, w2, act))  # clamp bites


def test_expert_offset_and_invalid_routes():
    x, w1, w2, ids, wts = _small_case(12, 64, 32, 4, 2, "relu2", seed=5, offset=40, invalid=0.25)
    res = _run_oracle(x, w1, w2, ids, wts, "relu2", offset=40)
    res0 = _run_oracle(x, w1, w2, np.where(ids >= 0, ids - 40, -1).astype(np.int32), wts, "relu2", 0)
    assert np.array_equal(res.out, res0.out)
    dead = np.all(ids < 0, axis=1)
    assert np.all(res.out[dead] == 0)


def test_oracle_batch_invariance_and_token_subset():
    w = synth.WORKLOADS["tiny"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    w1, w2 = synth.all_weights(w)
    xq, xs, xg = quantize_input_per_token(x)
    W = prepare_weights(w1, w2)
    full = routed_moe(xq, xs, xg, ids, wts, W, "relu2").out
    for t in (0, 7, 15):
        alone = routed_moe(xq[t:t + 1], xs[t:t + 1], xg[t:t + 1], ids[t:t + 1], wts[t:t + 1], W, "relu2").out
        assert np.array_equal(alone[0], full[t])
    sub = routed_moe(xq, xs, xg, ids, wts, W, "relu2", tokens=[3, 9]).out
    assert np.array_equal(sub[[3, 9]], full[[3, 9]])


@pytest.mark.parametrize("name", ["tiny", "swiglu"])
def test_plausibility_against_bf16_moe(name):
    """Per-token cosine to the unquantized MoE: mean > 0.97 and min > 0.95."""
    w = synth.WORKLOADS[name]
    T = min(w.T, 64)
    x = synth.activations(w, T)
    ids, wts = synth.router(w, T)
    w1, w2 = synth.all_weights(w)
    xq, xs, xg = quantize_input_per_token(x)
    res = routed_moe(xq, xs, xg, ids, wts, prepare_weights(w1, w2), w.act)
    ref = bf16_reference_moe(x, ids, wts, w1, w2, w.act)
    got = bf16_to_f32(res.out).astype(np.float64)
    cos = np.sum(got * ref, 1) / (np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1))
    assert cos.mean() > 0.97 and cos.min() > 0.95
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0.03 < rel < 0.35


def test_act_mismatch_rejected():
    x, w1, w2, ids, wts = _small_case(2, 32, 16, 2, 1, "relu2", seed=1)
    with pytest.raises(ValueError):
        _run_oracle(x, w1, w2, ids, wts, "swiglu")
