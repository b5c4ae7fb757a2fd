"""GPU parity of the layer steps: the router front, the SwiGLU clamp, the fused
(order-free) finalize, and pmoe_routed_moe_ex.

Bit-exact: router ids; pmoe_routed_moe_ex with default options equals
pmoe_routed_moe. Tolerance: router weights to 1e-5 relative (expf and the sum
order differ from the oracle's float64 softmax); MoE outputs per token
max |gpu - oracle| <= 1e-2 * max |oracle| and global cosine >= 0.999.
"""
import numpy as np
import pytest

import synth
from helpers import oracle_weights, bf16_bits, dev, dev_bf16
from oracle import layer as ol
from oracle import moe as om
from oracle import quant as oq
from oracle import recipes as orc
from oracle.formats import bf16_to_f32

pytestmark = pytest.mark.gpu
REL_TOL = 1e-2
F32 = np.float32


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


def _sync():
    import torch
    torch.cuda.synchronize()


def _assert_rows_close(got_bits, want_bits, what):
    got = bf16_to_f32(got_bits).astype(np.float64)
    want = bf16_to_f32(want_bits).astype(np.float64)
    scale = np.abs(want).max(axis=1)
    err = np.abs(got - want).max(axis=1)
    bad = np.nonzero(err > REL_TOL * scale)[0]
    assert bad.size == 0, f"{what}: rows {bad[:8]} rel err {(err / np.maximum(scale, 1e-30))[bad[:8]]}"
    cos = np.sum(got * want) / (np.linalg.norm(got) * np.linalg.norm(want) + 1e-300)
    assert cos >= 0.999, f"{what}: cosine {cos}"


# ----------------------------------------------------------------------------- router
def _router_cases():
    rng = np.random.default_rng(51)
    cases = []
    for name in ("tiny", "swiglu", "ep4_t1024", "large"):
        w = synth.WORKLOADS[name]
        cases.append((name, synth.router_logits(w), w.K, w.renormalize))
    lg = rng.standard_normal((300, 1024)).astype(F32)
    lg[:50, ::7] = 2.5                            # many exact ties at the top
    lg[50:60] = 0.0                               # all equal
    cases.append(("E1024_K32_ties", lg, 32, False))
    cases.append(("E5_K5", rng.standard_normal((33, 5)).astype(F32), 5, True))
    cases.append(("E65_K1", rng.standard_normal((257, 65)).astype(F32), 1, False))
    return cases


@pytest.mark.parametrize("case", _router_cases(), ids=lambda c: c[0])
def test_router_topk(pm, case):
    _, lg, K, renorm = case
    ids, w = pm.router_topk(dev(lg), K, renorm)
    _sync()
    oid, ow = ol.router_topk(lg, K, renorm)
    assert np.array_equal(ids.cpu().numpy(), oid)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-30)


def test_router_feeds_the_path(pm):
    """Router front + per-token path on the EP4 share: same routing as the seeded inputs."""
    w = synth.WORKLOADS["ep4_t512"]
    ids, wts = pm.router_topk(dev(synth.router_logits(w)), w.K, w.renormalize)
    _sync()
    sid, swt = synth.router(w)
    assert np.array_equal(ids.cpu().numpy(), sid)
    np.testing.assert_allclose(wts.cpu().numpy(), swt, rtol=1e-5)


# ----------------------------------------------------------------------------- options
class ExRun:
    def __init__(self, pm, w, recipe="per_token", finalize="ordered", limit=0.0, P=None):
        import torch
        self.x = synth.activations(w)
        self.ids, self.wts = synth.router(w)
        self.P = P or pm.prepare_weights(*synth.all_weights(w, device="cuda"))
        K = self.ids.shape[1]
        self.ws = torch.empty(pm.moe_workspace_bytes(w.T, K, w.E, w.H, w.I, self.P.act),
                              dtype=torch.uint8, device="cuda")
        xd = dev_bf16(self.x)
        if recipe == "per_token":
            xq, xs, xg = pm.quantize_input_per_token(xd)
        else:
            xq, xs, xg = xd, None, None
        self.out = pm.routed_moe_ex(xq, xs, xg, dev(self.ids), dev(self.wts), self.P, recipe=recipe,
                                    finalize=finalize, swiglu_limit=limit, workspace=self.ws)
        _sync()
        self.views = pm.workspace_views(self.ws, w.T, K, w.E, w.H, w.I, self.P.act)


def _oracle(w, x, ids, wts, recipe="per_token", **kw):
    W = oracle_weights(w)
    xin = oq.quantize_input_per_token(x) if recipe == "per_token" else x
    return orc.routed_moe_recipe(recipe, xin, ids, wts, W, w.act, **kw)


def test_ex_defaults_equal_routed_moe(pm):
    import torch
    w = synth.WORKLOADS["swiglu"]
    run = ExRun(pm, w)
    xq, xs, xg = pm.quantize_input_per_token(dev_bf16(run.x))
    ref = pm.routed_moe(xq, xs, xg, dev(run.ids), dev(run.wts), run.P)
    _sync()
    assert torch.equal(ref.view(torch.int16), run.out.view(torch.int16))


@pytest.mark.parametrize("name,limit", [("swiglu", 0.05), ("ep4_t512", 0.5)])
def test_swiglu_clamp(pm, name, limit):
    w = synth.WORKLOADS[name]
    run = ExRun(pm, w, limit=limit)
    experts = None if name == "swiglu" else [0, 17]
    res = _oracle(w, run.x, run.ids, run.wts, swiglu_limit=limit, experts=experts)
    rows = np.nonzero(res.computed_rows)[0]
    h = run.views["h"].cpu().numpy()[rows]
    assert np.abs(h).max() <= max(limit, 0.2785) * limit * (1 + 1e-5)   # |silu(min(g,L))| * L
    assert np.all(np.abs(h - res.h[rows]).max(axis=1) <= 1e-4 * np.abs(res.h[rows]).max(axis=1) + 1e-30)
    _assert_rows_close(bf16_bits(run.views["z"])[rows], res.z[rows], "z")
    unclamped = _oracle(w, run.x, run.ids, run.wts, experts=experts)
    assert not np.array_equal(unclamped.z[rows], res.z[rows])       # the clamp bites here
    if experts is None:
        _assert_rows_close(bf16_bits(run.out), res.out, "out")


@pytest.mark.parametrize("name,recipe", [("tiny", "per_token"), ("swiglu", "per_token"),
                                         ("swiglu", "w4a16"), ("relu2", "per_token")])
def test_fused_finalize(pm, name, recipe):
    w = synth.WORKLOADS[name]
    run = ExRun(pm, w, recipe=recipe, finalize="fused")
    orecipe = "weight_only" if recipe == "w4a16" else recipe
    toks = None if w.T <= 256 else [0, 1, 500, w.T - 1]
    res = _oracle(w, run.x, run.ids, run.wts, recipe=orecipe, finalize_mode="fused", tokens=toks)
    got = bf16_bits(run.out)
    if toks is None:
        _assert_rows_close(got, res.out, "out (fused)")
    else:
        _assert_rows_close(got[toks], res.out[toks], "out (fused)")
    ordered = ExRun(pm, w, recipe=recipe, P=run.P).out
    _assert_rows_close(got, bf16_bits(ordered), "fused vs ordered")


@pytest.mark.parametrize("name,recipe", [("relu2", "per_token"), ("ep4_t1024", "per_token"),
                                         ("ep4_t512", "w4a16")])
def test_two_streams_same_bits(pm, name, recipe):
    """The two expert halves on two streams give exactly the one-stream result."""
    import torch
    w = synth.WORKLOADS[name]
    x = dev_bf16(synth.activations(w))
    ids, wts = (dev(a) for a in synth.router(w))
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    if recipe == "per_token":
        xin = pm.quantize_input_per_token(x)
    else:
        xin = (x, None, None)
    outs = [pm.routed_moe_ex(*xin, ids, wts, P, recipe=recipe, streams=s) for s in (1, 2, 0, 2)]
    _sync()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    del P
    torch.cuda.empty_cache()


@pytest.mark.parametrize("recipe,finalize", [("per_token", "ordered"), ("per_token", "fused"),
                                             ("per_tensor", "ordered"), ("w4a16", "ordered"),
                                             ("w4a16", "fused")])
def test_edges_offsets_invalid_routes(pm, recipe, finalize):
    """expert_offset with int64 ids and -1 fills; a token whose routes are all outside the
    shard gets +0; results match the same call on shifted int32 ids with offset 0."""
    import torch
    w = synth.WORKLOADS["swiglu"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    ids = ids.astype(np.int64) + 40
    ids[5, :] = -1                                  # token 5: no route at all
    ids[9, :] = 7                                   # token 9: every id below the shard
    ids[12, 1] = 40 + w.E                           # one id just past the shard
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    a2 = torch.tensor([2688.0 / 0.5], dtype=torch.float32, device="cuda")
    xd = dev_bf16(x)
    if recipe == "per_token":
        xin = pm.quantize_input_per_token(xd)
    elif recipe == "per_tensor":
        a1 = torch.tensor([float(2688.0 / np.abs(bf16_to_f32(x)).max())], device="cuda")
        P = pm.prepare_weights(*synth.all_weights(w, device="cuda"), input_scales=(a1, a2))
        xin = pm.quantize_input_per_tensor(xd, a1) + (None,)
    else:
        xin = (xd, None, None)
    kw = dict(recipe=recipe, finalize=finalize, a2=a2 if recipe == "per_tensor" else None)
    got = pm.routed_moe_ex(*xin, dev(ids), dev(wts), P, expert_offset=40, **kw)
    shifted = np.where((ids >= 40) & (ids < 40 + w.E), ids - 40, -1).astype(np.int32)
    ref = pm.routed_moe_ex(*xin, dev(shifted), dev(wts), P, **kw)
    _sync()
    g, r = bf16_bits(got), bf16_bits(ref)
    assert not g[5].any() and not g[9].any()
    if finalize == "ordered":
        assert np.array_equal(g, r)
    else:
        _assert_rows_close(np.delete(g, [5, 9], 0), np.delete(r, [5, 9], 0), "fused with offset")


def test_edges_single_token_and_router_k_equals_e(pm):
    import torch
    w = synth.WORKLOADS["tiny"]
    x = synth.activations(w, 1)
    ids, wts = synth.router(w, 1)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    out = pm.routed_moe_ex(dev_bf16(x), None, None, dev(ids), dev(wts), P, recipe="w4a16")
    _sync()
    res = _oracle(w, x, ids, wts, recipe="weight_only")
    _assert_rows_close(bf16_bits(out), res.out, "T=1 W4A16")
    lg = synth.router_logits(w, 33)
    rid, rw = pm.router_topk(dev(lg), w.E, True)
    _sync()
    oid, ow = ol.router_topk(lg, w.E, True)
    assert np.array_equal(rid.cpu().numpy(), oid)
    np.testing.assert_allclose(rw.cpu().numpy(), ow, rtol=1e-5)
    np.testing.assert_allclose(rw.cpu().numpy().sum(axis=1), 1.0, rtol=1e-5)


# ----------------------------------------------------------------------------- BF16 forward
@pytest.mark.parametrize("name,recipe,finalize", [
    ("tiny", "per_token", "ordered"), ("swiglu", "per_tensor", "ordered"),
    ("swiglu", "w4a16", "ordered"), ("relu2", "per_token", "fused"),
    ("ep4_t1024", "per_token", "ordered"), ("ep4_t512", "per_tensor", "ordered")])
def test_forward_equals_quantize_then_path(pm, name, recipe, finalize):
    """pmoe_moe_forward (quantize overlapped with routing) gives the bits of the
    separate quantize call followed by pmoe_routed_moe_ex; ordered finalize
    bit for bit, the fused one to its tolerance."""
    import torch
    w = synth.WORKLOADS[name]
    x = synth.activations(w)
    ids, wts = (dev(a) for a in synth.router(w))
    xd = dev_bf16(x)
    a1 = torch.tensor([float(2688.0 / np.abs(bf16_to_f32(x)).max())], device="cuda")
    a2 = torch.tensor([2688.0 / 0.5], dtype=torch.float32, device="cuda")
    scales = (a1, a2) if recipe == "per_tensor" else None
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"), input_scales=scales)
    kw = dict(recipe=recipe, finalize=finalize, a2=a2 if recipe == "per_tensor" else None)
    if recipe == "per_token":
        xin = pm.quantize_input_per_token(xd)
    elif recipe == "per_tensor":
        xin = pm.quantize_input_per_tensor(xd, a1) + (None,)
    else:
        xin = (xd, None, None)
    ref = pm.routed_moe_ex(*xin, ids, wts, P, **kw)
    outs = [pm.moe_forward(xd, ids, wts, P, a1=a1 if recipe == "per_tensor" else None,
                           streams=s, **kw) for s in (0, 1, 2)]
    _sync()
    for got in outs:
        if finalize == "ordered":
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        else:
            _assert_rows_close(bf16_bits(got), bf16_bits(ref), "forward (fused)")
    del P
    torch.cuda.empty_cache()


def test_forward_matches_oracle(pm):
    w = synth.WORKLOADS["swiglu"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    got = pm.moe_forward(dev_bf16(x), dev(ids), dev(wts), P)
    _sync()
    _assert_rows_close(bf16_bits(got), _oracle(w, x, ids, wts).out, "forward")


@pytest.mark.parametrize("recipe", ["per_token", "per_tensor", "w4a16"])
def test_forward_edges(pm, recipe):
    """pmoe_moe_forward with int64 ids, an expert offset and -1 fills, and with T = 1,
    bit for bit against the separate quantize + pmoe_routed_moe_ex path."""
    import torch
    w = synth.WORKLOADS["swiglu"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    ids = ids.astype(np.int64) + 40
    ids[3, :] = -1
    ids[7, 2] = 40 + w.E
    xd = dev_bf16(x)
    a1 = torch.tensor([float(2688.0 / np.abs(bf16_to_f32(x)).max())], device="cuda")
    a2 = torch.tensor([2688.0 / 0.5], dtype=torch.float32, device="cuda")
    scales = (a1, a2) if recipe == "per_tensor" else None
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"), input_scales=scales)
    kw = dict(recipe=recipe, a2=a2 if recipe == "per_tensor" else None, expert_offset=40)
    fa1 = a1 if recipe == "per_tensor" else None
    for rows in (slice(None), slice(5, 6)):
        xs = xd[rows].contiguous()
        if recipe == "per_token":
            xin = pm.quantize_input_per_token(xs)
        elif recipe == "per_tensor":
            xin = pm.quantize_input_per_tensor(xs, a1) + (None,)
        else:
            xin = (xs, None, None)
        i_d, w_d = dev(ids[rows]), dev(wts[rows])
        ref = pm.routed_moe_ex(*xin, i_d, w_d, P, **kw)
        got = pm.moe_forward(xs, i_d, w_d, P, a1=fa1, **kw)
        _sync()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    full = pm.moe_forward(xd, dev(ids), dev(wts), P, a1=fa1, **kw)
    _sync()
    assert not bf16_bits(full)[3].any()            # a token without valid routes gets +0


def test_forward_batch_invariance_across_stream_split(pm):
    """A token alone (one stream, one M-tile per expert) gives the same BF16 bits as
    inside the full ep4_t1024 batch (two streams, split expert set, hot experts
    spanning many M-tiles)."""
    import torch
    w = synth.WORKLOADS["ep4_t1024"]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    full = pm.moe_forward(dev_bf16(x), dev(ids), dev(wts), P)
    toks = [0, int(np.nonzero((ids == 0).any(axis=1))[0][0]), 700, w.T - 1]
    alone = [pm.moe_forward(dev_bf16(x[t:t + 1]), dev(ids[t:t + 1]), dev(wts[t:t + 1]), P) for t in toks]
    _sync()
    fb = bf16_bits(full)
    for t, a in zip(toks, alone):
        assert np.array_equal(bf16_bits(a)[0], fb[t]), f"token {t}"
    del P
    torch.cuda.empty_cache()


def test_forward_repeat_determinism_full_size(pm):
    """Race check: the one-call forward at ep4_t1024 (two streams, forked
    quantization) gives identical bits over repeated calls, with other work on
    the same workspace in between (a fused-finalize call and a W4A16 call)."""
    import torch
    w = synth.WORKLOADS["ep4_t1024"]
    x = dev_bf16(synth.activations(w))
    ids, wts = (dev(a) for a in synth.router(w))
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    ws = torch.empty(pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, P.act), dtype=torch.uint8,
                     device="cuda")
    ref = pm.moe_forward(x, ids, wts, P, workspace=ws).clone()
    for i in range(4):
        if i % 2:
            pm.moe_forward(x, ids, wts, P, finalize="fused", workspace=ws)
        else:
            pm.moe_forward(x, ids, wts, P, recipe="w4a16", workspace=ws)
        out = pm.moe_forward(x, ids, wts, P, workspace=ws)
        _sync()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"repeat {i}"
    del P, ws
    torch.cuda.empty_cache()


def test_side_stream_with_allocator_churn(pm):
    """Calls on a stream other than torch's current one: inputs produced on the current stream
    right before the call are waited for, and the temporaries the binding allocates (workspace,
    output, contiguous copies) are not handed out again by the caching allocator while the
    call's kernels still use them, even when the current stream frees and refills memory at
    once."""
    import torch
    w = synth.WORKLOADS["swiglu"]
    x = dev_bf16(synth.activations(w))
    ids, wts = synth.router(w)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    ref = pm.moe_forward(x, dev(ids), dev(wts), P)
    xq, xs, xg = pm.quantize_input_per_token(x)
    ref2 = pm.routed_moe(xq, xs, xg, dev(ids), dev(wts), P)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for i in range(6):
        xi = x.clone()                                           # made on the current stream
        ids_nc = dev(ids.astype(np.int64).T.copy()).t()          # non-contiguous: copied inside
        if i % 2 == 0:
            o = pm.moe_forward(xi, ids_nc, dev(wts), P, stream=side)
        else:
            q = pm.quantize_input_per_token(xi, stream=side)
            o = pm.routed_moe(*q, ids_nc, dev(wts), P, stream=side)
            del q
        del xi, ids_nc
        junk = [torch.full((1 << 18,), -1, dtype=torch.int32, device="cuda") for _ in range(48)]
        del junk
        outs.append(o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        want = ref if i % 2 == 0 else ref2
        assert torch.equal(o.view(torch.int16), want.view(torch.int16)), i
