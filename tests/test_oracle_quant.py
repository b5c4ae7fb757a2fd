"""Pins of the oracle's quantizers: worked example, invariants, round-trip bounds, weight scale."""
import json
import os

import numpy as np

from oracle.formats import e2m1_decode, e4m3_decode, unpack_nibbles
from oracle.quant import (RECIPE_CONST, block_quantize, dequantize_blocks, dequantize_rows,
                          per_row_scale, quantize_input_per_token, quantize_rows_f32,
                          quantize_weight_matrix, weight_global_scale)

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _bf16(x):
    import synth
    return synth._bf16_np(np.asarray(x, F32))


def test_recipe_constant_is_fp32_of_one_over_2688():
    assert RECIPE_CONST == F32(1.0 / (448 * 6))
    assert float(RECIPE_CONST).hex() == "0x1.8618620000000p-12"


def test_worked_example_h32():
    g = json.load(open(os.path.join(GOLD, "worked_example_h32.json")))
    x = np.array([g["x"]], F32)
    xq, sf, scale = quantize_input_per_token(_bf16(x))
    assert xq[0].tobytes().hex().upper() == g["xq_hex"]
    assert sf[0].tolist() == g["x_sf"]
    assert float(scale[0]).hex() == float.fromhex(g["x_scale_hex"]).hex()
    # dequantization of the example is exact
    assert np.array_equal(dequantize_blocks(xq, sf)[0] * float(scale[0]) / float(scale[0]),
                          dequantize_blocks(xq, sf)[0])
    e = e4m3_decode(np.array(g["x_sf"])) * float(scale[0])
    assert np.float32(e[0]) == 1.0 and np.float32(e[1]) == 0.5


def _logspace_rows(rng, R, L):
    mags = np.exp(rng.uniform(np.log(1e-6), np.log(1e6), (R, L)))
    return (mags * rng.choice([-1.0, 1.0], (R, L))).astype(F32)


def test_invariants_on_rows():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal((20, 256)).astype(F32), _logspace_rows(rng, 20, 256),
                        np.zeros((1, 256), F32)])
    q, sf, g = quantize_rows_f32(x)
    codes = unpack_nibbles(q)
    assert sf.max() <= 0x7E
    for r in range(x.shape[0]):
        if not np.any(x[r]):
            assert g[r] == 0 and not q[r].any() and not sf[r].any()
            continue
        i = np.argmax(np.abs(x[r]))
        assert codes[r, i] & 7 == 7                            # the row max lands on +-6
        assert sf[r, i // 16] == 0x7E                            # in a block scaled by 448
        assert (codes[r, i] >> 3) == (1 if x[r, i] < 0 else 0)


def test_power_of_two_equivariance():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((8, 128)).astype(F32)
    q0, s0, g0 = quantize_rows_f32(x)
    for m in (-20, -3, 5, 30):
        q1, s1, g1 = quantize_rows_f32((x * F32(2.0 ** m)).astype(F32))
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
        assert np.array_equal(g1, (g0 * F32(2.0 ** m)).astype(F32))


def test_roundtrip_bound():
    """|x - x_hat| <= e_b (1 + 2^-19) elementwise, and the block step bound (closed form)."""
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal((30, 512)).astype(F32), _logspace_rows(rng, 30, 512)])
    q, sf, g = quantize_rows_f32(x)
    xh = dequantize_rows(q, sf, g).astype(np.float64)
    e = (e4m3_decode(sf).astype(F32) * g[:, None]).astype(np.float64)
    eb = np.repeat(e, 16, axis=1)
    assert np.all(np.abs(x.astype(np.float64) - xh) <= eb * (1 + 2.0 ** -19))
    amax_b = np.abs(x.astype(np.float64)).reshape(60, 32, 16).max(axis=2)
    normal = sf >= 0x08
    assert np.all(e[normal] <= (amax_b[normal] / 6) * (17 / 16) * (1 + 2.0 ** -22))
    sub = (~normal) & (sf > 0)
    gg = np.repeat(g[:, None].astype(np.float64), 32, axis=1)
    assert np.all(e[sub] <= amax_b[sub] / 6 + gg[sub] * 2.0 ** -10)


def test_block_formula_by_hand_loop():
    """Element-by-element scalar loop of the block steps (independent of the vectorized code)."""
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((3, 64)) * [[1e-3], [1.0], [300.0]]).astype(F32)
    codes, sf = block_quantize(x, per_row_scale(x))
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for r in range(3):
        g = F32(F32(np.max(np.abs(x[r]))) * RECIPE_CONST)
        for b in range(4):
            blk = x[r, 16 * b:16 * b + 16]
            v = F32(F32(F32(np.max(np.abs(blk))) / F32(6)) / g)
            # e4m3 by scanning every byte for the nearest value (ties to even byte)
            best = min(range(0x7F), key=lambda c: (abs(float(e4m3_decode(c)) - min(float(v), 448.0)), c % 2))
            assert sf[r, b] == best
            e = F32(F32(e4m3_decode(best)) * g)
            for i in range(16):
                qv = F32(blk[i] / e)
                a = abs(float(qv))
                c = min(range(8), key=lambda k: (abs(grid[k] - a), k % 2)) if a <= 6 else 7
                c |= 8 if np.signbit(qv) else 0
                assert codes[r, 16 * b + i] == c


def test_weight_scale_and_invariants():
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(F32)
    wb = _bf16(w)
    q, sf, alpha = quantize_weight_matrix(wb)
    wf = (wb.astype(np.uint32) << 16).view(F32)
    amax = np.abs(wf).max()
    assert abs(float(alpha) * 2688.0 - float(amax)) <= 2 * np.spacing(np.float32(amax))
    codes = unpack_nibbles(q)
    i, j = np.unravel_index(np.argmax(np.abs(wf)), wf.shape)
    assert codes[i, j] & 7 == 7 and sf[i, j // 16] == 0x7E
    a0, s0 = weight_global_scale(np.zeros((4, 16), F32))
    assert a0 == 0 and s0 == np.inf
    qz, sfz, az = quantize_weight_matrix(np.zeros((4, 32), np.uint16))
    assert az == 0 and not qz.any() and not sfz.any()


def test_weight_scale_exact_at_powers_of_two():
    """Where amax / 2688 is a power of two, w_scale = 2688 / amax and its
    reciprocal are exact under any rounding, so alpha must equal amax / 2688
    bit for bit: pins the recipe constant 2688 = 448 * 6 and the reciprocal
    structure of the per-expert scale (not only to within 2 ulp)."""
    for k in range(-40, 41, 5):
        amax = np.float32(2688.0 * 2.0 ** k)
        w = np.zeros((2, 32), F32)
        w[1, 17] = amax
        w[0, 3] = -amax * np.float32(0.25)
        a, s = weight_global_scale(w)
        assert np.float32(a) == np.float32(2.0 ** k), (k, a)
        assert np.float32(s) == np.float32(2.0 ** -k), (k, s)
        # the element at amax encodes as code 6 (0x7) under the top block scale 448
        q, sf, alpha = quantize_weight_matrix(_bf16(w))
        assert np.float32(alpha) == np.float32(2.0 ** k)
        assert sf[1, 1] == 0x7E and unpack_nibbles(q)[1, 17] == 0x7


def test_weight_dequant_error_small():
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((128, 512)) * 0.02).astype(F32)
    q, sf, alpha = quantize_weight_matrix(_bf16(w))
    wh = dequantize_blocks(q, sf) * float(alpha)
    wf = (_bf16(w).astype(np.uint32) << 16).view(F32).astype(np.float64)
    rel = np.linalg.norm(wh - wf) / np.linalg.norm(wf)
    assert 0.05 < rel < 0.15                       # NVFP4's expected few-percent-to-10% error
