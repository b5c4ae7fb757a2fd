"""GPU parity at widths that are multiples of 16 but not of 64 (H = 2064) or 32 (I = 1040).

The library pads every reduction to whole 64-element chunks with zero codes and zero
block scales and drops the padding columns of the last column block on output; the
interface keeps the canonical, unpadded arrays. Checked against the oracle (which
knows nothing of the padding): prepared weights bit-exact, the whole path element by
element within the per-token tolerance (1e-2 of each token's / row's max), the
requantized intermediate bit-exact given the GPU's own FP32 h, and the one-call
forward (internal quantizer writing padded rows) bit-equal to quantize + routed_moe
(canonical rows re-laid inside the library).
"""
import numpy as np
import pytest

import synth
from helpers import bf16_bits, canonical_from_prepared, dev, dev_bf16, oracle_weights
from oracle import moe as om
from oracle import quant as oq
from oracle import recipes as orc
from oracle.formats import bf16_to_f32

pytestmark = pytest.mark.gpu
REL_TOL = 1e-2


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


def _sync():
    import torch
    torch.cuda.synchronize()


def _rows_close(got_bits, want_bits, what):
    got = bf16_to_f32(got_bits).astype(np.float64)
    want = bf16_to_f32(want_bits).astype(np.float64)
    err = np.abs(got - want).max(axis=1)
    scale = np.abs(want).max(axis=1)
    bad = np.nonzero(err > REL_TOL * scale)[0]
    assert bad.size == 0, f"{what}: rows {bad[:8]} rel err {(err / np.maximum(scale, 1e-30))[bad[:8]]}"
    cos = np.sum(got * want) / (np.linalg.norm(got) * np.linalg.norm(want) + 1e-300)
    assert cos >= 0.999, f"{what}: cosine {cos}"


@pytest.mark.parametrize("name", ["odd_swiglu", "odd_relu2"])
def test_prepare_weights_odd_widths(pm, name):
    w = synth.WORKLOADS[name]
    w1, w2 = synth.all_weights(w)
    P = pm.prepare_weights(dev_bf16(w1), dev_bf16(w2))
    _sync()
    W = om.prepare_weights(w1, w2)
    gI = w.I if w.gated else 0
    c1, s1 = canonical_from_prepared(P.w1_codes.cpu().numpy(), P.w1_scales.cpu().numpy(), w.E, w.N1,
                                     w.H, gI)
    c2, s2 = canonical_from_prepared(P.w2_codes.cpu().numpy(), P.w2_scales.cpu().numpy(), w.E, w.H,
                                     w.I)
    assert np.array_equal(c1, W.w1q) and np.array_equal(s1, W.w1sf)
    assert np.array_equal(c2, W.w2q) and np.array_equal(s2, W.w2sf)
    assert np.array_equal(P.w1_alpha.cpu().numpy(), W.a1) and np.array_equal(P.w2_alpha.cpu().numpy(), W.a2)


@pytest.mark.parametrize("name", ["odd_swiglu", "odd_relu2"])
def test_moe_odd_widths(pm, name):
    import torch
    w = synth.WORKLOADS[name]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    xb = dev_bf16(x)
    xq, xs, xg = pm.quantize_input_per_token(xb)
    ws = torch.empty(pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, P.act), dtype=torch.uint8,
                     device="cuda")
    out = pm.routed_moe(xq, xs, xg, dev(ids), dev(wts), P, workspace=ws)
    _sync()
    v = pm.workspace_views(ws, w.T, w.K, w.E, w.H, w.I, P.act)
    # the canonical quantizer output is the oracle's, bit for bit
    oxq, oxs, oxg = oq.quantize_input_per_token(x)
    assert np.array_equal(xq.cpu().numpy(), oxq) and np.array_equal(xs.cpu().numpy(), oxs)
    res = om.routed_moe(oxq, oxs, oxg, ids, wts, oracle_weights(w, range(w.E)), w.act)
    R = res.routing.route_of_row.size
    assert np.array_equal(v["row_of_route"].cpu().numpy(), res.routing.row_of_route)
    h = v["h"].cpu().numpy()[:R]
    assert np.all(np.abs(h - res.h).max(axis=1) <= 1e-4 * np.abs(res.h).max(axis=1) + 1e-30)
    # requant of the GPU's own h: bit-exact, and the padding of each row is zero
    q, sf, g = oq.quantize_rows_f32(h)
    assert np.array_equal(v["hq"].cpu().numpy()[:R], q) and np.array_equal(v["h_sf"].cpu().numpy()[:R], sf)
    assert np.array_equal(v["h_scale"].cpu().numpy()[:R].view(np.uint32), g.view(np.uint32))
    assert not v["hq_padded"][:R, w.I // 2:].any() and not v["h_sf_padded"][:R, w.I // 16:].any()
    _rows_close(bf16_bits(v["z"])[:R], res.z, "z")
    _rows_close(bf16_bits(out), res.out, "out")
    # the one-call forward (padded rows written by the internal quantizer) gives the same bits
    fwd = pm.moe_forward(xb, dev(ids), dev(wts), P)
    _sync()
    assert torch.equal(fwd.view(torch.int16), out.view(torch.int16))
    # and so do both finalize layouts of the fused (order-free) mode, to tolerance
    fused = pm.moe_forward(xb, dev(ids), dev(wts), P, finalize="fused")
    _sync()
    _rows_close(bf16_bits(fused), res.out, "fused out")


@pytest.mark.parametrize("name", ["odd_swiglu", "odd_relu2"])
def test_w4a16_odd_widths(pm, name):
    import torch
    w = synth.WORKLOADS[name]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    ws = torch.empty(pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, P.act), dtype=torch.uint8,
                     device="cuda")
    out = pm.routed_moe_w4a16(dev_bf16(x), dev(ids), dev(wts), P, workspace=ws)
    _sync()
    v = pm.workspace_views(ws, w.T, w.K, w.E, w.H, w.I, P.act)
    res = orc.routed_moe_recipe("weight_only", x, ids, wts, oracle_weights(w, range(w.E)), w.act)
    R = res.routing.route_of_row.size
    _rows_close(v["h_bf16"].cpu().numpy().view(np.uint16)[:R], res.h_bf16, "h (BF16)")
    _rows_close(bf16_bits(v["z"])[:R], res.z, "z")
    _rows_close(bf16_bits(out), res.out, "out")


def test_per_tensor_odd_widths(pm):
    import torch
    F32 = np.float32
    w = synth.WORKLOADS["odd_relu2"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    a1 = F32(F32(2688.0) / F32(np.abs(bf16_to_f32(x)).max()))
    a2 = F32(2688.0 / 3.0)
    sc = lambda v: torch.tensor([float(v)], dtype=torch.float32, device="cuda")
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"), input_scales=(sc(a1), sc(a2)))
    xq, xs = pm.quantize_input_per_tensor(dev_bf16(x), sc(a1))
    out = pm.routed_moe_per_tensor(xq, xs, dev(ids), dev(wts), P, sc(a2))
    _sync()
    W = orc.LazyWeightsPerTensor(lambda e: synth.expert_weights(w, e), w.E, w.N1, w.H, w.I, a1, a2)
    res = orc.routed_moe_recipe("per_tensor", orc.quantize_input_per_tensor(x, a1), ids, wts, W,
                                w.act, a2=a2)
    _rows_close(bf16_bits(out), res.out, "out")
