"""GPU parity of the per-tensor NVFP4 and W4A16 (weight-only) recipes against the oracle.

Bit-exact: the static-scale quantizer's bytes, the folded alphas, the prepared
codes (identical to the per-token preparation) and the routing maps.
Tolerance (floating-point steps), per token: max |gpu - oracle| <= 1e-2 * max
|oracle| on the output and on every sampled FC2 row z, and a global cosine
>= 0.999. Batch invariance: a token alone gives the same BF16 bits as inside
its batch. Static scales are inputs: a1 from the activations' amax, a2 from
the oracle's intermediate on the sampled rows.
"""
import numpy as np
import pytest

import synth
from helpers import (bf16_bits, dev, dev_bf16, oracle_weights, oracle_weights_per_tensor,
                     sample_experts, sample_tokens, split_expert)
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


def _scalar(v):
    import torch
    return torch.tensor([float(v)], dtype=torch.float32, device="cuda")


def _assert_rows_close(got_bits, want_bits, what):
    got = bf16_to_f32(got_bits).astype(np.float64)
    want = bf16_to_f32(want_bits).astype(np.float64)
    scale = np.abs(want).max(axis=1)
    err = np.abs(got - want).max(axis=1)
    bad = np.nonzero(err > REL_TOL * scale)[0]
    assert bad.size == 0, f"{what}: rows {bad[:8]} rel err {(err / np.maximum(scale, 1e-30))[bad[:8]]}"
    cos = np.sum(got * want) / (np.linalg.norm(got) * np.linalg.norm(want) + 1e-300)
    assert cos >= 0.999, f"{what}: cosine {cos}"


def _a1(x_bits):
    return F32(F32(2688.0) / F32(np.abs(bf16_to_f32(x_bits)).max()))


def _a2_from_oracle(w, x, ids, wts, experts=None):
    """Calibrate the FC2 input scale on the oracle's per-token intermediate."""
    xq, xs, xg = oq.quantize_input_per_token(x)
    W = oracle_weights(w, experts if experts is not None else ())
    res = om.routed_moe(xq, xs, xg, ids, wts, W, w.act, experts=experts)
    return F32(F32(2688.0) / F32(np.abs(res.h[res.computed_rows]).max()))


# ----------------------------------------------------------------------------- per-tensor pieces
@pytest.mark.parametrize("name", ["tiny", "swiglu", "relu2", "ep4_t1024"])
def test_quantize_per_tensor_bit_exact(pm, name):
    w = synth.WORKLOADS[name]
    x = synth.activations(w)
    for a in (_a1(x), F32(_a1(x) * 8)):          # calibrated, and one that saturates large values
        xq, xs = pm.quantize_input_per_tensor(dev_bf16(x), _scalar(a))
        _sync()
        wq, ws = orc.quantize_input_per_tensor(x, a)
        assert np.array_equal(xq.cpu().numpy(), wq) and np.array_equal(xs.cpu().numpy(), ws)


def test_prepare_per_tensor_folds_alphas(pm):
    import torch
    w = synth.WORKLOADS["swiglu"]
    w1, w2 = synth.all_weights(w)
    a1, a2 = F32(61.25), F32(1234.5)
    P = pm.prepare_weights(dev_bf16(w1), dev_bf16(w2))
    Q = pm.prepare_weights(dev_bf16(w1), dev_bf16(w2), input_scales=(_scalar(a1), _scalar(a2)))
    _sync()
    for f in ("w1_codes", "w1_scales", "w2_codes", "w2_scales"):
        assert torch.equal(getattr(P, f), getattr(Q, f))
    assert np.array_equal(Q.w1_alpha.cpu().numpy(), orc.fold_input_scale(w1, a1))
    assert np.array_equal(Q.w2_alpha.cpu().numpy(), orc.fold_input_scale(w2, a2))


# ----------------------------------------------------------------------------- per-tensor pipeline
class PerTensorRun:
    def __init__(self, pm, w, a1, a2, T=None, x=None, ids=None, wts=None, P=None):
        import torch
        self.T = w.T if T is None else T
        self.x = synth.activations(w, self.T) if x is None else x
        if ids is None:
            ids, wts = synth.router(w, self.T)
        self.ids, self.wts = ids, wts
        self.P = P or pm.prepare_weights(*synth.all_weights(w, device="cuda"),
                                         input_scales=(_scalar(a1), _scalar(a2)))
        xq, xs = pm.quantize_input_per_tensor(dev_bf16(self.x), _scalar(a1))
        K = ids.shape[1]
        self.ws = torch.empty(pm.moe_workspace_bytes(self.T, K, w.E, w.H, w.I, self.P.act),
                              dtype=torch.uint8, device="cuda")
        self.out = pm.routed_moe_per_tensor(xq, xs, dev(ids), dev(wts), self.P, _scalar(a2),
                                            workspace=self.ws)
        _sync()
        self.views = pm.workspace_views(self.ws, self.T, K, w.E, w.H, w.I, self.P.act)


def _oracle_per_tensor(w, x, ids, wts, a1, a2, need=(), **kw):
    W = oracle_weights_per_tensor(w, a1, a2, need)
    return orc.routed_moe_recipe("per_tensor", orc.quantize_input_per_tensor(x, a1), ids, wts, W,
                                 w.act, a2=a2, **kw)


@pytest.mark.parametrize("name", ["tiny", "swiglu"])
def test_per_tensor_moe_small(pm, name):
    w = synth.WORKLOADS[name]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    a1, a2 = _a1(x), _a2_from_oracle(w, x, ids, wts)
    run = PerTensorRun(pm, w, a1, a2)
    res = _oracle_per_tensor(w, x, ids, wts, a1, a2)
    R = res.routing.route_of_row.size
    assert np.array_equal(run.views["row_of_route"].cpu().numpy(), res.routing.row_of_route)
    h = run.views["h"].cpu().numpy()[:R]
    assert np.all(np.abs(h - res.h).max(axis=1) <= 1e-4 * np.abs(res.h).max(axis=1) + 1e-30)
    assert np.mean(run.views["hq"].cpu().numpy()[:R] == res.hq) > 0.999
    _assert_rows_close(bf16_bits(run.views["z"])[:R], res.z, "z")
    _assert_rows_close(bf16_bits(run.out), res.out, "out")


def _sample(w, views, ids):
    """Experts on both streams (split sides, hot, first, last) and 8 tokens, three of them
    routed only to experts of the second stream; plus every expert those need."""
    offs = views["expert_offsets"].cpu().numpy()
    split = split_expert(offs, views["counters"].cpu().numpy())
    experts = sample_experts(np.diff(offs), split)
    tokens, need = sample_tokens(ids, split, experts, n=8, E=w.E)
    return experts, tokens, need


def _check_sampled(w, run_z, run_out, views, res, res_t, experts, tokens):
    offs = views["expert_offsets"].cpu().numpy()
    z = bf16_bits(run_z)
    for e in experts:
        rows = np.arange(offs[e], offs[e + 1])
        rows = rows[res.computed_rows[rows]]
        assert rows.size > 0, e
        _assert_rows_close(z[rows], res.z[rows], f"z of expert {e}")
    _assert_rows_close(bf16_bits(run_out)[tokens], res_t.out[tokens], f"out of tokens {tokens}")


@pytest.mark.parametrize("name", ["relu2", "ep4_t1024", "large"])
def test_per_tensor_moe_sampled(pm, name):
    import torch
    w = synth.WORKLOADS[name]
    x = synth.activations(w)
    ids, wts = synth.router(w)
    a1, a2 = _a1(x), _a2_from_oracle(w, x, ids, wts, experts=[0, 17])
    run = PerTensorRun(pm, w, a1, a2)
    experts, tokens, need = _sample(w, run.views, ids)
    res = _oracle_per_tensor(w, x, ids, wts, a1, a2, need=need, experts=experts)
    res_t = _oracle_per_tensor(w, x, ids, wts, a1, a2, tokens=tokens)
    _check_sampled(w, run.views["z"], run.out, run.views, res, res_t, experts, tokens)
    del run
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- W4A16
class W4A16Run:
    def __init__(self, pm, w, T=None, x=None, ids=None, wts=None, P=None):
        import torch
        self.T = w.T if T is None else T
        self.x = synth.activations(w, self.T) if x is None else x
        if ids is None:
            ids, wts = synth.router(w, self.T)
        self.ids, self.wts = ids, wts
        self.P = P or pm.prepare_weights(*synth.all_weights(w, device="cuda"))
        K = ids.shape[1]
        self.ws = torch.empty(pm.moe_workspace_bytes(self.T, K, w.E, w.H, w.I, self.P.act),
                              dtype=torch.uint8, device="cuda")
        self.out = pm.routed_moe_w4a16(dev_bf16(self.x), dev(ids), dev(wts), self.P, workspace=self.ws)
        _sync()
        self.views = pm.workspace_views(self.ws, self.T, K, w.E, w.H, w.I, self.P.act)


def _oracle_w4a16(w, x, ids, wts, need=(), **kw):
    W = oracle_weights(w, need)
    return orc.routed_moe_recipe("weight_only", x, ids, wts, W, w.act, **kw)


@pytest.mark.parametrize("name", ["tiny", "swiglu"])
def test_w4a16_moe_small(pm, name):
    w = synth.WORKLOADS[name]
    run = W4A16Run(pm, w)
    res = _oracle_w4a16(w, run.x, run.ids, run.wts)
    R = res.routing.route_of_row.size
    assert np.array_equal(run.views["row_of_route"].cpu().numpy(), res.routing.row_of_route)
    hb = run.views["h_bf16"].cpu().numpy().view(np.uint16)[:R]
    _assert_rows_close(hb, res.h_bf16, "h (BF16)")
    # h is one BF16 rounding of an FP32 value that differs only in summation order
    agree = np.mean(hb == res.h_bf16)
    assert agree > 0.99, agree
    _assert_rows_close(bf16_bits(run.views["z"])[:R], res.z, "z")
    _assert_rows_close(bf16_bits(run.out), res.out, "out")


@pytest.mark.parametrize("name", ["relu2", "ep4_t512", "ep4_t1024", "large"])
def test_w4a16_moe_sampled(pm, name):
    import torch
    w = synth.WORKLOADS[name]
    run = W4A16Run(pm, w)
    experts, tokens, need = _sample(w, run.views, run.ids)
    res = _oracle_w4a16(w, run.x, run.ids, run.wts, need=need, experts=experts)
    res_t = _oracle_w4a16(w, run.x, run.ids, run.wts, tokens=tokens)
    _check_sampled(w, run.views["z"], run.out, run.views, res, res_t, experts, tokens)
    del run
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- invariance
def test_recipes_batch_invariance(pm):
    """A token alone gives the same bits as inside a batch of 1024 (swiglu and relu2 shapes)."""
    for name in ("relu2", "ep4_t1024"):
        w = synth.WORKLOADS[name]
        x = synth.activations(w)
        ids, wts = synth.router(w)
        P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
        full = W4A16Run(pm, w, x=x, ids=ids, wts=wts, P=P).out
        for t in (0, 513, w.T - 1):
            alone = W4A16Run(pm, w, T=1, x=x[t:t + 1], ids=ids[t:t + 1], wts=wts[t:t + 1], P=P).out
            assert np.array_equal(bf16_bits(alone)[0], bf16_bits(full)[t])
        a1, a2 = _a1(x), F32(2688.0 / 4.0)
        Q = pm.prepare_weights(*synth.all_weights(w, device="cuda"),
                               input_scales=(_scalar(a1), _scalar(a2)))
        full = PerTensorRun(pm, w, a1, a2, x=x, ids=ids, wts=wts, P=Q).out
        for t in (0, 513, w.T - 1):
            alone = PerTensorRun(pm, w, a1, a2, T=1, x=x[t:t + 1], ids=ids[t:t + 1], wts=wts[t:t + 1],
                                 P=Q).out
            assert np.array_equal(bf16_bits(alone)[0], bf16_bits(full)[t])
        del P, Q
