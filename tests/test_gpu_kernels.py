"""GPU parity of the single-step kernels against the oracle: bit-exact bytes,
scales and integer maps (quantizers, weight preparation, routing, finalize)."""
import json
import os
import zlib

import numpy as np
import pytest

import synth
from helpers import oracle_weights, bf16_bits, canonical_from_prepared, dev, dev_bf16
from oracle import moe as om
from oracle import quant as oq
from oracle.formats import f32_to_bf16_rne

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


def _sync():
    import torch
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- quantizer
def _check_quant_bf16(pm, x_bits):
    xq, xs, xg = pm.quantize_input_per_token(dev_bf16(x_bits))
    _sync()
    oq_, os_, og_ = oq.quantize_input_per_token(x_bits)
    assert np.array_equal(xq.cpu().numpy(), oq_)
    assert np.array_equal(xs.cpu().numpy(), os_)
    assert np.array_equal(xg.cpu().numpy().view(np.uint32), og_.view(np.uint32))


def test_quantize_worked_example(pm):
    g = json.load(open(os.path.join(GOLD, "worked_example_h32.json")))
    x = np.zeros((1, 64), np.float32)
    x[0, :32] = g["x"]
    xq, xs, xg = pm.quantize_input_per_token(dev_bf16(synth._bf16_np(x)))
    _sync()
    assert xq.cpu().numpy()[0, :16].tobytes().hex().upper() == g["xq_hex"]
    assert xs.cpu().numpy()[0, :2].tolist() == g["x_sf"]
    assert float(xg.cpu().numpy()[0]).hex() == float.fromhex(g["x_scale_hex"]).hex()


def test_quantize_edge_rows(pm):
    rng = np.random.default_rng(1)
    L = 320
    rows = [np.zeros(L), rng.standard_normal(L),
            np.exp(rng.uniform(np.log(1e-6), np.log(1e6), L)) * rng.choice([-1, 1], L),
            np.full(L, -0.0), np.r_[np.zeros(L - 1), 1e-38], np.r_[np.zeros(L - 1), -3e38],
            np.tile([6, -0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5], L // 8),
            rng.standard_normal(L) * 1e-30]
    x = synth._bf16_np(np.array(rows, np.float32))
    _check_quant_bf16(pm, x)


@pytest.mark.parametrize("name", ["tiny", "swiglu", "relu2", "ep4_t1024", "large"])
def test_quantize_workload_activations(pm, name):
    w = synth.WORKLOADS[name]
    _check_quant_bf16(pm, synth.activations(w, T=min(w.T, 1024)))


def test_quantize_rows_f32(pm):
    rng = np.random.default_rng(2)
    L = 3072
    h = np.concatenate([
        np.maximum(rng.standard_normal((40, L)), 0) ** 2,
        rng.standard_normal((40, L)) * np.exp(rng.uniform(-20, 20, (40, 1))),
        np.exp(rng.uniform(np.log(1e-30), np.log(1e30), (8, L))) * rng.choice([-1, 1], (8, L)),
        np.zeros((2, L)), rng.standard_normal((2, L)) * 1e-40,
    ]).astype(np.float32)
    hq, hs, hg = pm.quantize_rows_f32(dev(h))
    _sync()
    q, s, g = oq.quantize_rows_f32(h)
    assert np.array_equal(hq.cpu().numpy(), q)
    assert np.array_equal(hs.cpu().numpy(), s)
    assert np.array_equal(hg.cpu().numpy().view(np.uint32), g.view(np.uint32))


# ----------------------------------------------------------------------------- weights
def _check_prepared(P, oW, E, N1, H, I, experts):
    gated = N1 == 2 * I
    c1, s1 = canonical_from_prepared(P.w1_codes.cpu().numpy(), P.w1_scales.cpu().numpy(), E, N1, H,
                                     I if gated else 0)
    c2, s2 = canonical_from_prepared(P.w2_codes.cpu().numpy(), P.w2_scales.cpu().numpy(), E, H, I, 0)
    a1 = P.w1_alpha.cpu().numpy()
    a2 = P.w2_alpha.cpu().numpy()
    for e in experts:
        w1q, w1s, al1, w2q, w2s, al2 = oW.expert(e)
        assert np.array_equal(c1[e], w1q), f"FC1 codes, expert {e}"
        assert np.array_equal(s1[e], w1s), f"FC1 scales, expert {e}"
        assert np.array_equal(c2[e], w2q), f"FC2 codes, expert {e}"
        assert np.array_equal(s2[e], w2s), f"FC2 scales, expert {e}"
        assert a1[e].view(np.uint32) == np.float32(al1).view(np.uint32)
        assert a2[e].view(np.uint32) == np.float32(al2).view(np.uint32)


@pytest.mark.parametrize("name", ["tiny", "swiglu", "relu2"])
def test_prepare_weights_small(pm, name):
    w = synth.WORKLOADS[name]
    w1, w2 = synth.all_weights(w, device="cuda")
    P = pm.prepare_weights(w1, w2)
    _sync()
    oW = oracle_weights(w)
    experts = range(w.E) if w.E <= 4 else [0, 1, w.E // 2, w.E - 1]
    _check_prepared(P, oW, w.E, w.N1, w.H, w.I, experts)


def test_prepare_weights_edge_values(pm):
    """All-zero expert, a tiny-magnitude expert (subnormal E4M3 scales), one huge outlier."""
    import torch
    E, I, H = 3, 64, 128
    rng = np.random.default_rng(3)
    w1 = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    w1[0] = 0
    w2[1] *= np.exp(rng.uniform(-12, 0, (H, I)))
    w1[2, 5, 7] = 300.0
    b1, b2 = synth._bf16_np(w1), synth._bf16_np(w2)
    P = pm.prepare_weights(dev_bf16(b1), dev_bf16(b2))
    _sync()
    _check_prepared(P, om.prepare_weights(b1, b2), E, 2 * I, H, I, range(E))
    assert P.w1_alpha.cpu().numpy()[0] == 0


def test_prepare_weights_ep4_sampled_and_refresh(pm):
    """Full ep4 stacks generated on the GPU; sampled experts checked; in-place refresh."""
    import torch
    w = synth.WORKLOADS["ep4_t512"]
    w1, w2 = synth.all_weights(w, device="cuda")
    P = pm.prepare_weights(w1, w2)
    _sync()
    ptrs = [t.data_ptr() for t in (P.w1_codes, P.w1_scales, P.w1_alpha, P.w2_codes, P.w2_scales, P.w2_alpha)]
    sample = [0, 47, 95]
    oW = oracle_weights(w)
    _check_prepared(P, oW, w.E, w.N1, w.H, w.I, sample)
    w_new = w.with_(weight_epoch=1)
    n1, n2 = synth.all_weights(w_new, device="cuda")
    P2 = pm.prepare_weights(n1, n2, out=P)
    _sync()
    assert P2 is P and ptrs == [t.data_ptr() for t in (P.w1_codes, P.w1_scales, P.w1_alpha, P.w2_codes,
                                                      P.w2_scales, P.w2_alpha)]
    oW2 = oracle_weights(w_new)
    _check_prepared(P, oW2, w.E, w.N1, w.H, w.I, [48])
    del w1, w2, n1, n2
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- routing
def _route_case(name, rng):
    if name == "random":
        return rng.integers(0, 32, (300, 4)), 32, 0
    if name == "one_expert":
        return np.full((100, 2), 3), 8, 0
    if name == "invalid_and_offset":
        ids = rng.integers(0, 200, (500, 6))
        ids[rng.random(ids.shape) < 0.2] = -1
        return ids, 96, 96
    if name == "skewed_large":
        ids = np.where(rng.random((4096, 8)) < 0.5, rng.integers(0, 2, (4096, 8)), rng.integers(0, 256, (4096, 8)))
        return ids, 256, 0
    if name == "many_experts":
        return rng.integers(0, 1024, (700, 8)), 1024, 0
    if name == "single":
        return np.array([[5, 1]]), 6, 0
    if name == "one_launch_limit":        # 8192 routes: the largest one-workgroup routing
        ids = rng.integers(0, 64, (1024, 8))
        ids[::7, 3] = -1
        return ids, 64, 0
    if name == "skewed_one_launch":       # hot experts inside the one-workgroup routing
        ids = np.where(rng.random((1000, 8)) < 0.5, rng.integers(0, 2, (1000, 8)),
                       rng.integers(0, 96, (1000, 8)))
        return ids, 96, 0
    if name == "past_one_launch":         # 8200 routes: the three-kernel routing
        return rng.integers(0, 64, (1025, 8)), 64, 0
    raise KeyError(name)


@pytest.mark.parametrize("case", ["random", "one_expert", "invalid_and_offset", "skewed_large",
                                  "many_experts", "single", "one_launch_limit", "skewed_one_launch",
                                  "past_one_launch"])
@pytest.mark.parametrize("ids_dtype", [np.int32, np.int64])
def test_routing_matches_oracle(pm, case, ids_dtype):
    """Row maps and expert offsets of routed_moe's workspace equal the oracle's stable routing."""
    import torch
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    ids, E, off = _route_case(case, rng)
    ids = ids.astype(ids_dtype)
    T, K = ids.shape
    H, I = 64, 64
    # Minimal weights: zeros (the maps do not depend on them).
    W = pm.prepare_weights(torch.zeros((E, I, H), dtype=torch.bfloat16, device="cuda"),
                           torch.zeros((E, H, I), dtype=torch.bfloat16, device="cuda"))
    xq, xs, xg = pm.quantize_input_per_token(torch.zeros((T, H), dtype=torch.bfloat16, device="cuda"))
    ws = torch.zeros(pm.moe_workspace_bytes(T, K, E, H, I, pm.ACT_RELU2), dtype=torch.uint8, device="cuda")
    wts = torch.ones((T, K), dtype=torch.float32, device="cuda")
    pm.routed_moe(xq, xs, xg, dev(ids), wts, W, expert_offset=off, workspace=ws)
    _sync()
    v = pm.workspace_views(ws, T, K, E, H, I, pm.ACT_RELU2)
    rt = om.route(ids, E, off)
    R = rt.route_of_row.size
    assert np.array_equal(v["row_of_route"].cpu().numpy(), rt.row_of_route)
    assert np.array_equal(v["route_of_row"].cpu().numpy()[:R], rt.route_of_row)
    assert np.array_equal(v["expert_offsets"].cpu().numpy(), rt.offsets)
    assert v["counters"].cpu().numpy()[0] == R


# ----------------------------------------------------------------------------- finalize
def _finalize_gpu(pm, z_bits, rows, w):
    out = pm.finalize(dev_bf16(z_bits), dev(rows.astype(np.int32)), dev(w.astype(np.float32)))
    _sync()
    return bf16_bits(out)


def test_finalize_hand_cases(pm):
    # slot order: 2^24 + 1 rounds back to 2^24, then -2^24 -> 0
    z = f32_to_bf16_rne(np.array([[2.0 ** 24] * 8, [1.0] * 8, [-2.0 ** 24] * 8], np.float32))
    got = _finalize_gpu(pm, z[[2, 1, 0]], np.array([2, 1, 0]), np.ones((1, 3), np.float32))
    assert got.tolist() == [[0] * 8]
    # no fused multiply-add
    w = np.array([[1 + 2.0 ** -7 + 2.0 ** -20, 1 + 2.0 ** -20]], np.float32)
    z = f32_to_bf16_rne(np.array([[-1.0] * 8, [1 + 2.0 ** -7] * 8], np.float32))
    assert _finalize_gpu(pm, z, np.array([0, 1]), w).tolist() == [[0] * 8]
    # invalid routes and +0
    z = f32_to_bf16_rne(np.array([[-0.0] * 8], np.float32))
    got = _finalize_gpu(pm, z, np.array([-1, 0, -1, -1]), np.ones((2, 2), np.float32))
    assert got.tolist() == [[0] * 8, [0] * 8]


@pytest.mark.parametrize("T,K,H", [(1, 1, 8), (37, 6, 7168), (300, 8, 2048), (64, 2, 2056)])
def test_finalize_random(pm, T, K, H):
    rng = np.random.default_rng(T * K)
    R = T * K
    z = f32_to_bf16_rne((rng.standard_normal((R, H)) * np.exp(rng.uniform(-5, 5, (R, 1)))).astype(np.float32))
    rows = rng.permutation(R).astype(np.int32)
    rows[rng.random(R) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    got = _finalize_gpu(pm, z, rows, w)
    assert np.array_equal(got, om.finalize(z, rows, w, T, K))
