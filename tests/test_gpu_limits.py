"""GPU parity at the limits: rows of 16384 elements for both quantizers
(bit-exact); the routed path with the longest reduction (H = 16384) and the
widest FC1 (SwiGLU with I = 16384, N1 = 32768); and degenerate expert sets
(one expert, two experts split over two streams, every route on one expert so
that one stream's part is empty). End-to-end results against the oracle to
the per-token tolerance (1e-2 of the token's max)."""
import numpy as np
import pytest

import synth
from helpers import bf16_bits, dev, dev_bf16
from oracle import moe as om
from oracle import quant as oq
from oracle import recipes as orc
from oracle.formats import bf16_to_f32

pytestmark = pytest.mark.gpu
MAX_ROW = 16384


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


def _sync():
    import torch
    torch.cuda.synchronize()


def test_quantize_longest_rows(pm):
    rng = np.random.default_rng(16384)
    x = rng.standard_normal((7, MAX_ROW)).astype(np.float32)
    x[1, ::97] *= 50.0                                  # outliers
    x[2] = 0.0                                          # an all-zero row
    xb = synth._bf16_np(x)
    xq, xs, xg = pm.quantize_input_per_token(dev_bf16(xb))
    h = (rng.standard_normal((5, MAX_ROW)) * np.exp(rng.uniform(-8, 8, (5, 1)))).astype(np.float32)
    hq, hs, hg = pm.quantize_rows_f32(dev(h))
    _sync()
    for got, want in zip((xq, xs, xg, hq, hs, hg),
                         oq.quantize_input_per_token(xb) + oq.quantize_rows_f32(h)):
        got = got.cpu().numpy()
        assert got.shape == want.shape and np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("H,I,act", [(MAX_ROW, 64, "relu2"), (64, MAX_ROW, "swiglu")])
def test_moe_largest_dims(pm, H, I, act):
    rng = np.random.default_rng(H + I)
    T, K, E = 9, 2, 3
    N1 = 2 * I if act == "swiglu" else I
    w1 = synth._bf16_np(rng.standard_normal((E, N1, H)).astype(np.float32) * 0.02)
    w2 = synth._bf16_np(rng.standard_normal((E, H, I)).astype(np.float32) * 0.02)
    x = synth._bf16_np(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    P = pm.prepare_weights(dev_bf16(w1), dev_bf16(w2))
    out = pm.moe_forward(dev_bf16(x), dev(ids), dev(wts), P)
    _sync()
    xq, xs, xg = oq.quantize_input_per_token(x)
    res = om.routed_moe(xq, xs, xg, ids, wts, om.prepare_weights(w1, w2), act)
    got = bf16_to_f32(bf16_bits(out)).astype(np.float64)
    want = bf16_to_f32(res.out).astype(np.float64)
    err = np.abs(got - want).max(axis=1)
    assert np.all(err <= 1e-2 * np.abs(want).max(axis=1)), err / np.abs(want).max(axis=1)


def _moe_case(pm, rng, T, K, E, H, I, act, ids):
    N1 = 2 * I if act == "swiglu" else I
    w1 = synth._bf16_np(rng.standard_normal((E, N1, H)).astype(np.float32) * 0.02)
    w2 = synth._bf16_np(rng.standard_normal((E, H, I)).astype(np.float32) * 0.02)
    x = synth._bf16_np(rng.standard_normal((T, H)).astype(np.float32))
    wts = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    P = pm.prepare_weights(dev_bf16(w1), dev_bf16(w2))
    return w1, w2, x, wts, P


@pytest.mark.parametrize("case", ["one_expert", "two_experts_split", "all_on_one_of_16"])
def test_expert_count_edges(pm, case):
    """Degenerate expert sets, with and without the two-stream split: E = 1;
    E = 2 split into one expert per stream; every route on one expert of 16, so
    one of the two parts is empty. Bit-equal across stream counts, and equal to
    the oracle to the per-token tolerance."""
    import torch
    rng = np.random.default_rng(len(case))
    H, I, act = 256, 128, "swiglu"
    if case == "one_expert":
        T, K, E = 300, 1, 1
        ids = np.zeros((T, K), np.int32)
    elif case == "two_experts_split":
        T, K, E = 1200, 2, 2
        ids = np.tile(np.array([[0, 1]], np.int32), (T, 1))
        ids[::3] = ids[::3, ::-1]
    else:
        T, K, E = 4096, 1, 16
        ids = np.full((T, K), 5, np.int32)
    w1, w2, x, wts, P = _moe_case(pm, rng, T, K, E, H, I, act, ids)
    outs = [pm.moe_forward(dev_bf16(x), dev(ids), dev(wts), P, streams=s) for s in (1, 2, 0)]
    _sync()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    toks = np.arange(T) if T <= 300 else np.array([0, 1, 2, T // 2, T - 1])
    xq, xs, xg = oq.quantize_input_per_token(x)
    res = om.routed_moe(xq, xs, xg, ids, wts, om.prepare_weights(w1, w2), act, tokens=toks)
    got = bf16_to_f32(bf16_bits(outs[0])[toks]).astype(np.float64)
    want = bf16_to_f32(res.out[toks]).astype(np.float64)
    err = np.abs(got - want).max(axis=1)
    assert np.all(err <= 1e-2 * np.abs(want).max(axis=1)), err / np.abs(want).max(axis=1)


@pytest.mark.parametrize("H,I", [(16, 16), (64, 48), (128, 96), (192, 64)])
@pytest.mark.parametrize("act", ["relu2", "swiglu"])
@pytest.mark.parametrize("recipe", ["per_token", "w4a16", "per_token_fused"])
def test_short_reductions(pm, H, I, act, recipe):
    """Reductions of one, two and three 64-element chunks (fewer chunks than
    the weight register ring holds, so every prefetch past the end is clamped
    to the last chunk): 2048 routes, run on one stream (whole launches) and
    split over two (half launches), NVFP4 and W4A16, and the order-free
    finalize (whose FC2 refills its ring the other way); bit-equal across the
    two (ordered finalize), and equal to the oracle to the per-token tolerance
    for every token."""
    import torch
    rng = np.random.default_rng(H * 1000 + I + (act == "swiglu"))
    T, K, E = 1024, 2, 8
    ids = np.argsort(rng.standard_normal((T, E)), axis=1)[:, :K].astype(np.int32)
    w1, w2, x, wts, P = _moe_case(pm, rng, T, K, E, H, I, act, ids)
    fused = recipe == "per_token_fused"
    kw = dict(recipe="per_token", finalize="fused") if fused else dict(recipe=recipe)
    outs = [pm.moe_forward(dev_bf16(x), dev(ids), dev(wts), P, streams=s, **kw) for s in (1, 2)]
    _sync()
    if not fused:  # the atomic adds of the fused finalize land in any order
        assert torch.equal(outs[1].view(torch.int16), outs[0].view(torch.int16))
    W = om.prepare_weights(w1, w2)
    if recipe == "w4a16":
        res = orc.routed_moe_recipe("weight_only", x, ids, wts, W, act)
    else:
        xq, xs, xg = oq.quantize_input_per_token(x)
        res = om.routed_moe(xq, xs, xg, ids, wts, W, act)
    want = bf16_to_f32(res.out).astype(np.float64)
    for o in outs:
        got = bf16_to_f32(bf16_bits(o)).astype(np.float64)
        err = np.abs(got - want).max(axis=1)
        assert np.all(err <= 1e-2 * np.abs(want).max(axis=1)), err / np.abs(want).max(axis=1)


@pytest.mark.parametrize("T", [2048, 2049])
def test_forward_route_quantize_boundary(pm, T):
    """The one-call forward routes and quantizes its BF16 input in one launch
    up to 8192 routes (T = 2048, K = 4) and in separate launches on two streams
    above (T = 2049): both give the bits of the separate quantize call followed
    by pmoe_routed_moe, with int32 and int64 ids."""
    import torch
    rng = np.random.default_rng(T)
    K, E, H, I = 4, 16, 256, 128
    ids = np.argsort(rng.standard_normal((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[7] = -1                                          # a token without routes
    w1, w2, x, wts, P = _moe_case(pm, rng, T, K, E, H, I, "swiglu", ids)
    xd = dev_bf16(x)
    xq, xs, xg = pm.quantize_input_per_token(xd)
    ref = pm.routed_moe(xq, xs, xg, dev(ids), dev(wts), P)
    for idt in (np.int32, np.int64):
        got = pm.moe_forward(xd, dev(ids.astype(idt)), dev(wts), P)
        _sync()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), idt
    assert not bf16_bits(ref)[7].any()


@pytest.mark.parametrize("recipe", ["per_token", "per_tensor"])
@pytest.mark.parametrize("streams", [1, 2])
def test_requant_bytes_in_the_path(pm, streams, recipe):
    """The intermediate's requantization inside the routed path, bit for bit:
    hq, h_sf (and h_scale, per-token) that the path leaves in its workspace
    equal the oracle's quantization of the FP32 h it left beside them -- per
    row, or with the static scale a2 -- for every routed row. One stream runs
    one workgroup per row over all rows; two streams run each expert half's
    rows one wave per row over a looping grid (a ragged 132-block row: some
    lanes hold 3 blocks, others 2)."""
    import torch
    rng = np.random.default_rng(2112 + streams)
    T, K, E, H, I, act = 1024, 4, 16, 256, 2112, "relu2"
    ids = np.argsort(rng.standard_normal((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.05] = -1
    w1, w2, x, wts, P = _moe_case(pm, rng, T, K, E, H, I, act, ids)
    xd = dev_bf16(x)
    ws = torch.zeros(pm.moe_workspace_bytes(T, K, E, H, I, P.act), dtype=torch.uint8, device="cuda")
    if recipe == "per_token":
        xq, xs, xg = pm.quantize_input_per_token(xd)
        pm.routed_moe_ex(xq, xs, xg, dev(ids), dev(wts), P, workspace=ws, streams=streams)
    else:
        a1 = torch.tensor([float(2688.0 / np.abs(bf16_to_f32(x)).max())], device="cuda")
        a2_host = np.float32(2688.0 / 0.75)
        a2 = torch.tensor([float(a2_host)], dtype=torch.float32, device="cuda")
        P = pm.prepare_weights(dev_bf16(w1), dev_bf16(w2), input_scales=(a1, a2))
        xq, xs = pm.quantize_input_per_tensor(xd, a1)
        pm.routed_moe_ex(xq, xs, None, dev(ids), dev(wts), P, recipe="per_tensor", a2=a2,
                         workspace=ws, streams=streams)
    _sync()
    v = pm.workspace_views(ws, T, K, E, H, I, P.act)
    R = int(v["counters"][0].item())
    assert R == int((ids >= 0).sum())
    h = v["h"][:R].cpu().numpy()
    if recipe == "per_token":
        q, s, g = oq.quantize_rows_f32(h)
        assert np.array_equal(v["h_scale"][:R].cpu().numpy().view(np.uint32), g.view(np.uint32))
    else:
        q, s = orc.quantize_rows_static(h, a2_host)
    assert np.array_equal(v["hq"][:R].cpu().numpy(), q)
    assert np.array_equal(v["h_sf"][:R].cpu().numpy(), s)
