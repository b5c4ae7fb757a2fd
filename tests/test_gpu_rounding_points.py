"""Quantizers at the rounding points of the block scale and of the codes.

The kernels take a block's E4M3 scale from one multiply by a per-row
reciprocal and fall back to the two IEEE divisions only when the product lies
within a few ulp of a point where the E4M3 rounding changes; likewise the
E2M1 codes come from a multiply by fp32(1/e) unless a value sits next to a code
boundary. These inputs are built so that many blocks land exactly on, or a few
ulp either side of, those points (E4M3 midpoints of the normal range,
half-steps of the subnormal grid, the saturation region; E2M1 boundaries
0.25 ... 5), and the results must match the oracle's divisions byte for byte:
the FP32 row quantizer (the requant of h), the BF16 per-token quantizer and
the weight preparation.
"""
import numpy as np
import pytest

import synth
from helpers import dev, dev_bf16
from oracle import moe as om
from oracle import quant as oq
from test_gpu_kernels import _check_prepared

pytestmark = pytest.mark.gpu

F32 = np.float32
K_RECIPE = F32(1.0) / F32(2688.0)


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


def _sync():
    import torch
    torch.cuda.synchronize()


def scale_rounding_points():
    """Values where E4M3 rounding (RNE, saturating at 448) changes: midpoints of
    the normal range (2^E * (1 + (2j + 1) / 16)) and half-steps (k + 1/2) * 2^-9
    of the subnormal grid."""
    pts = [(k + 0.5) / 512 for k in range(8)]
    for E in range(-6, 9):
        for j in range(8):
            m = 2.0 ** E * (1 + (2 * j + 1) / 16)
            if m < 464:
                pts.append(m)
    return np.array(pts, np.float64)


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(F32)


def block_scale_value(a, g):
    """fp32(fp32(a / 6) / g), the value the block scale byte encodes."""
    return (F32(a) / F32(6)).astype(F32) / F32(g)


def near_point(z, ulps):
    """z within `ulps` of a value whose low 19 mantissa bits are zero."""
    b = np.asarray(z, F32).view(np.uint32).astype(np.int64)
    r = b & 0x7FFFF
    return (r <= ulps) | (r >= 0x80000 - ulps)


def f32_amaxes_near_points(g, spread=24):
    """FP32 block amaxes a whose scale value lands on or within `spread` ulp of
    every rounding point (all float32 neighbours of point * 6 * g)."""
    out = []
    for p in scale_rounding_points():
        a0 = F32(p * 6.0 * float(g))
        bits = a0.view(np.uint32).astype(np.int64) + np.arange(-spread, spread + 1)
        out.append(bits.astype(np.uint32).view(F32))
    return np.concatenate(out)


def code_boundary_elements(a, g, rng, n):
    """n values of magnitude below a at or next to E2M1 code boundaries of the
    block whose amax is a (y = x / e near 0.25, 0.75, ..., 5), plus noise."""
    from oracle.formats import e4m3_decode, e4m3_encode_sat
    sf = e4m3_encode_sat(np.array([block_scale_value(a, g)], F32))
    e = F32(e4m3_decode(sf)[0]) * F32(g)
    b = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], n) * rng.choice([-1, 1], n)
    x = (b * float(e)).astype(F32)
    x = (x.view(np.uint32).astype(np.int64) + rng.integers(-3, 4, n)).astype(np.uint32).view(F32)
    x = np.where(np.abs(x) < a, x, F32(0.5) * a)
    return x


def f32_rows(rng, g_row_amax, L):
    """Rows of length L whose row amax is g_row_amax; each 16-block has its own
    crafted amax and code-boundary elements."""
    g = F32(g_row_amax) * K_RECIPE
    amaxes = f32_amaxes_near_points(g)
    amaxes = amaxes[amaxes < g_row_amax]
    nblk = L // 16
    rows = []
    for start in range(0, len(amaxes), nblk - 1):
        row = np.zeros(L, F32)
        row[0] = g_row_amax
        for j, a in enumerate(amaxes[start:start + nblk - 1]):
            blk = code_boundary_elements(a, g, rng, 16)
            blk[rng.integers(0, 16)] = a * rng.choice([-1, 1])
            row[16 * (j + 1):16 * (j + 2)] = blk
        rows.append(row)
    return np.array(rows, F32), amaxes, g


@pytest.mark.parametrize("R", [1.0, 3.7e-3, 2.9e4])
def test_requant_rows_at_rounding_points(pm, R):
    rng = np.random.default_rng(int(R * 1000) % 97)
    h, _, _ = f32_rows(rng, R, 3072)
    hq, hs, hg = pm.quantize_rows_f32(dev(h))
    _sync()
    q, s, g = oq.quantize_rows_f32(h)
    assert np.array_equal(hq.cpu().numpy(), q)
    assert np.array_equal(hs.cpu().numpy(), s)
    assert np.array_equal(hg.cpu().numpy().view(np.uint32), g.view(np.uint32))


def bf16_rows_with_ties(rng, L):
    """BF16 rows of amax 2688, so g = fp32(2688 * fp32(1/2688)) (1 or a neighbour
    of it): block amaxes 6 * m (m a scale rounding point with few significant
    bits) are exact in BF16 and put fp32(a/6) on the point itself, and their
    BF16 neighbours land next to it."""
    pts = scale_rounding_points()
    a = synth._bf16_np((6.0 * pts).astype(F32))
    nb = np.concatenate([a, a + 1, a - 1]).astype(np.uint16)   # BF16 neighbours
    vals = bf16_to_f32(nb)
    vals = vals[(vals > 0) & (vals < 2688)]
    nblk = L // 16
    g = F32(2688.0) * K_RECIPE
    rows = []
    for start in range(0, len(vals), nblk - 1):
        row = np.zeros(L, F32)
        row[0] = 2688.0
        for j, av in enumerate(vals[start:start + nblk - 1]):
            blk = code_boundary_elements(av, g, rng, 16)
            blk[rng.integers(0, 16)] = av
            row[16 * (j + 1):16 * (j + 2)] = blk
        rows.append(row)
    return synth._bf16_np(np.array(rows, F32))


def test_input_quantizer_at_rounding_points(pm):
    rng = np.random.default_rng(5)
    x = bf16_rows_with_ties(rng, 1024)
    xq, xs, xg = pm.quantize_input_per_token(dev_bf16(x))
    _sync()
    q, s, g = oq.quantize_input_per_token(x)
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy(), s)
    assert np.array_equal(xg.cpu().numpy().view(np.uint32), g.view(np.uint32))


def test_prepare_weights_at_rounding_points(pm):
    """Experts whose amax is 2688 (alpha = 1) with blocks at the scale's
    rounding points, and one expert of arbitrary alpha with FP32-searched
    block amaxes rounded to BF16."""
    rng = np.random.default_rng(9)
    E, I, H = 3, 128, 512
    w1 = np.zeros((E, 2 * I, H), F32)
    w2 = np.zeros((E, H, I), F32)
    rows1 = bf16_to_f32(bf16_rows_with_ties(rng, H))
    rows2 = bf16_to_f32(bf16_rows_with_ties(rng, I))
    for e in range(2):
        w1[e, :min(2 * I, len(rows1))] = rows1[:2 * I]
        w2[e, :min(H, len(rows2))] = rows2[:H]
    hr, _, _ = f32_rows(rng, 7.25, H)
    w1[2, :min(2 * I, len(hr))] = hr[:2 * I]
    w2[2] = rng.standard_normal((H, I)).astype(F32) * 0.01
    b1, b2 = synth._bf16_np(w1), synth._bf16_np(w2)
    P = pm.prepare_weights(dev_bf16(b1), dev_bf16(b2))
    _sync()
    _check_prepared(P, om.prepare_weights(b1, b2), E, 2 * I, H, I, range(E))


@pytest.mark.parametrize("a1", [1.0, 0.37])
def test_static_scale_quantizer_at_rounding_points(pm, a1):
    """The per-tensor recipe's static scale a (g = fp32(1 / a); a = 1 puts the
    blocks of amax 6 m exactly on the points)."""
    import torch
    from oracle import recipes as orc
    rng = np.random.default_rng(11)
    x = bf16_rows_with_ties(rng, 1024)
    a = torch.tensor([a1], dtype=torch.float32, device="cuda")
    xq, xs = pm.quantize_input_per_tensor(dev_bf16(x), a)
    _sync()
    q, s = orc.quantize_input_per_tensor(x, np.float32(a1))[:2]
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy(), s)
