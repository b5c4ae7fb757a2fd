"""pmoe_routed_moe_static -- the routed path on the library's static scratch, for callers
that cannot allocate device memory -- against pmoe_routed_moe with a workspace, through
the C ABI: bit-identical outputs on two calls in a row, the second with fewer tokens (the
scratch keeps the first call's contents, which must not leak into the second), at a shape
whose reductions are padded inside the library and at the EP4 width; and a clear
PMOE_ERR_WORKSPACE, with the output untouched, for sizes beyond the scratch."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import dev, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


def _static(pm, q, ids, wts, P, out):
    """The C call itself (no binding logic in between)."""
    T, K = ids.shape
    return pm.lib().pmoe_routed_moe_static(
        pm._ptr(q[0]), pm._ptr(q[1]), pm._ptr(q[2]), pm._ptr(ids), pm.IDS_INT32, pm._ptr(wts), T, K,
        P.E, P.H, P.I, P.N1, 0, pm._ptr(P.w1_codes), pm._ptr(P.w1_scales), pm._ptr(P.w1_alpha),
        pm._ptr(P.w2_codes), pm._ptr(P.w2_scales), pm._ptr(P.w2_alpha), P.act, pm._ptr(out),
        pm._stream())


@pytest.mark.parametrize("name,T_first,T_second", [("swiglu", 256, 100), ("odd_swiglu", 600, 37),
                                                    ("ep4_t512", 300, 64)])
def test_static_scratch_equals_workspace_path(pm, name, T_first, T_second):
    import torch
    w = synth.WORKLOADS[name]
    x = synth.activations(w, T_first)
    ids, wts = synth.router(w, T_first)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    for T in (T_first, T_second):                       # the second call is smaller
        q = pm.quantize_input_per_token(dev_bf16(x[:T]))
        i_d, w_d = dev(ids[:T].astype(np.int32)), dev(wts[:T])
        want = pm.routed_moe(*q, i_d, w_d, P)
        got = torch.full((T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
        rc = _static(pm, q, i_d, w_d, P, got)
        assert rc == 0, pm.lib().pmoe_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (name, T)
    del P
    torch.cuda.empty_cache()


def test_static_scratch_rejects_sizes_beyond_it(pm):
    import torch
    w = synth.WORKLOADS["ep4_t1024"]            # T*K = 6144 routes at H=7168, I=3072
    need = pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, pm.ACT_SWIGLU)
    assert need > pm.STATIC_SCRATCH_BYTES
    small = synth.WORKLOADS["swiglu"]
    P = pm.prepare_weights(*synth.all_weights(small, device="cuda"))
    T = 8192                                    # T*K = 32768 routes at H=2048, I=768
    assert pm.moe_workspace_bytes(T, small.K, small.E, small.H, small.I, P.act) > pm.STATIC_SCRATCH_BYTES
    x = synth.activations(small, 16)
    q = pm.quantize_input_per_token(dev_bf16(np.tile(x, (T // 16, 1))))
    ids, wts = synth.router(small, 16)
    i_d = dev(np.tile(ids, (T // 16, 1)).astype(np.int32))
    w_d = dev(np.tile(wts, (T // 16, 1)))
    out = torch.full((T, small.H), 3.0, dtype=torch.bfloat16, device="cuda")
    rc = _static(pm, q, i_d, w_d, P, out)
    msg = pm.lib().pmoe_last_error().decode()
    assert rc == 5 and "static scratch" in msg, (rc, msg)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    # and the entry point still works right after (a size that fits)
    want = pm.routed_moe(q[0][:16], q[1][:16], q[2][:16], i_d[:16], w_d[:16], P)
    got = torch.empty_like(want)
    assert _static(pm, (q[0][:16], q[1][:16], q[2][:16]), i_d[:16], w_d[:16], P, got) == 0
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
