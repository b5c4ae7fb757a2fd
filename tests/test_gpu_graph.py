"""Graph capture: the one-call forward (routing and input quantization in one
launch, the two expert halves on two streams, the finalize),
captured in a HIP graph through torch.cuda.graph, replays to the eager result
several times, with eager work and synchronizations between the replays
(workspace and output overwritten in between): bit for bit with the ordered
finalize; with the order-free (atomic) finalize, whose FP32 sums depend on
the order of the adds, to the per-token tolerance (1e-2 of the token's max)."""
import numpy as np
import pytest

import synth
from helpers import bf16_bits, dev, dev_bf16
from oracle.formats import bf16_to_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pm():
    import torch
    import precision_moe_amd as pm
    assert torch.cuda.is_available()
    return pm


@pytest.mark.parametrize("name,recipe,finalize", [("ep4_t512", "per_token", "ordered"),
                                                  ("relu2", "per_token", "fused"),
                                                  ("swiglu", "w4a16", "ordered")])
def test_forward_graph_replay_equals_eager(pm, name, recipe, finalize):
    import torch
    w = synth.WORKLOADS[name]
    x = dev_bf16(synth.activations(w))
    ids, wts = (dev(a) for a in synth.router(w))
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    ws = torch.empty(pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, P.act), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    kw = dict(recipe=recipe, finalize=finalize, workspace=ws, out=out)
    pm.moe_forward(x, ids, wts, P, **kw)
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up on a side stream before capture
        pm.moe_forward(x, ids, wts, P, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pm.moe_forward(x, ids, wts, P, **kw)
    torch.cuda.synchronize()
    for i in range(4):
        ws.fill_(0xA5 if i % 2 else 0)     # eager work that overwrites what the graph reads back
        out.fill_(float(i + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if finalize == "ordered":
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        else:
            got = bf16_to_f32(bf16_bits(out)).astype(np.float64)
            want = bf16_to_f32(bf16_bits(eager)).astype(np.float64)
            err = np.abs(got - want).max(axis=1)
            assert np.all(err <= 1e-2 * np.abs(want).max(axis=1)), f"replay {i}"
    del g
    torch.cuda.synchronize()
