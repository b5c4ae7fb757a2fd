"""End-to-end GPU parity of routed_moe against the oracle, plus batch invariance.

Tolerance (floating-point steps): per token, max_n |gpu - oracle| <= 1e-2 * max_n
|oracle| on the finalized output and on every per-route FC2 row z, and a global
cosine >= 0.999; the FP32 activation output h agrees to 1e-4 of each row's max
(only the FP32 accumulation order and expf differ). Routing maps, quantized
activations and the finalize order are checked bit-exactly elsewhere.
"""
import numpy as np
import pytest

import synth
from helpers import (bf16_bits, dev, dev_bf16, oracle_weights, sample_experts, sample_tokens,
                     split_expert)
from oracle import moe as om
from oracle import quant as oq
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


def _assert_rows_close(got_bits, want_bits, what):
    got = bf16_to_f32(got_bits).astype(np.float64)
    want = bf16_to_f32(want_bits).astype(np.float64)
    scale = np.abs(want).max(axis=1)
    err = np.abs(got - want).max(axis=1)
    bad = np.nonzero(err > REL_TOL * scale)[0]
    assert bad.size == 0, f"{what}: rows {bad[:8]} rel err {(err / np.maximum(scale, 1e-30))[bad[:8]]}"
    cos = np.sum(got * want) / (np.linalg.norm(got) * np.linalg.norm(want) + 1e-300)
    assert cos >= 0.999, f"{what}: cosine {cos}"
    return float(np.median(err / np.maximum(scale, 1e-30)))


class GpuCase:
    """Inputs on the GPU, the prepared weights, and one routed_moe run."""

    def __init__(self, pm, w, T=None, ids=None, wts=None, x=None, weights=None, offset=0, ids64=False):
        import torch
        self.pm, self.w = pm, w
        self.T = w.T if T is None else T
        self.x = synth.activations(w, self.T) if x is None else x
        if ids is None:
            ids, wts = synth.router(w, self.T)
        self.ids, self.wts = ids, wts
        self.P = weights if weights is not None else pm.prepare_weights(*synth.all_weights(w, device="cuda"))
        self.offset = offset
        self.xq, self.xs, self.xg = pm.quantize_input_per_token(dev_bf16(self.x))
        K = ids.shape[1]
        self.ws = torch.empty(pm.moe_workspace_bytes(self.T, K, w.E, w.H, w.I, self.P.act),
                              dtype=torch.uint8, device="cuda")
        self.ids_dev = dev(ids.astype(np.int64 if ids64 else np.int32))
        self.out = pm.routed_moe(self.xq, self.xs, self.xg, self.ids_dev, dev(wts), self.P,
                                 expert_offset=offset, workspace=self.ws)
        _sync()
        self.views = pm.workspace_views(self.ws, self.T, K, w.E, w.H, w.I, self.P.act)

    def out_bits(self):
        return bf16_bits(self.out)


def _oracle(w, x, ids, wts, tokens=None, experts=None, weights=None):
    xq, xs, xg = oq.quantize_input_per_token(x)
    W = weights or oracle_weights(w)
    return om.routed_moe(xq, xs, xg, ids, wts, W, w.act, tokens=tokens, experts=experts)


def _sampled_parity(w, run, n_tokens=8):
    """z rows of every sampled expert (first, ordinary, both sides of the two-stream split,
    the hot ones, the last) and the outputs of n_tokens tokens (three of them routed only to
    experts of the second stream) against the oracle. Returns (experts, tokens)."""
    v = run.views
    offs = v["expert_offsets"].cpu().numpy()
    split = split_expert(offs, v["counters"].cpu().numpy())
    assert 0 < split < w.E, split
    experts = sample_experts(np.diff(offs), split)
    tokens, need = sample_tokens(run.ids, split, experts, n=n_tokens, E=w.E)
    W = oracle_weights(w, need)
    res = _oracle(w, run.x, run.ids, run.wts, experts=experts, weights=W)
    z = bf16_bits(v["z"])
    for e in experts:
        rows = np.arange(offs[e], offs[e + 1])
        rows = rows[res.computed_rows[rows]]
        assert rows.size > 0, e
        _assert_rows_close(z[rows], res.z[rows], f"z of expert {e}")
    res_t = _oracle(w, run.x, run.ids, run.wts, tokens=tokens, weights=W)
    _assert_rows_close(run.out_bits()[tokens], res_t.out[tokens], f"out of tokens {tokens}")
    assert any((run.ids[t] >= split).all() for t in tokens)
    return experts, tokens


# ----------------------------------------------------------------------------- small: everything
@pytest.mark.parametrize("name", ["tiny", "swiglu", "nemo_swiglu", "nemo_relu2"])
def test_moe_matches_oracle_small(pm, name):
    w = synth.WORKLOADS[name]
    run = GpuCase(pm, w)
    res = _oracle(w, run.x, run.ids, run.wts)
    R = res.routing.route_of_row.size
    v = run.views
    assert np.array_equal(v["row_of_route"].cpu().numpy(), res.routing.row_of_route)
    # FP32 activation output
    h = v["h"].cpu().numpy()[:R]
    err = np.abs(h - res.h).max(axis=1)
    assert np.all(err <= 1e-4 * np.abs(res.h).max(axis=1) + 1e-30)
    # requantized intermediate: nearly all codes identical (a code may flip where h sits on a boundary)
    assert np.mean(v["hq"].cpu().numpy()[:R] == res.hq) > 0.999
    _assert_rows_close(bf16_bits(v["z"])[:R], res.z, "z")
    med = _assert_rows_close(run.out_bits(), res.out, "out")
    assert med < 2e-3


def test_moe_relu2_sampled(pm):
    """relu2 workload (T=1024, H=4096, I=2048, E=64, top-6): z rows of experts on both
    streams and the outputs of 8 tokens."""
    w = synth.WORKLOADS["relu2"]
    run = GpuCase(pm, w)
    _sampled_parity(w, run)


def test_fc1_accumulation_within_summation_bound(pm):
    """The GPU's FP32 accumulation of FC1 stays within the worst-case error of any
    summation order: |acc_gpu - acc_exact| <= gamma_K * sum_k |a_k b_k| with
    gamma_K = K u / (1 - K u) (Higham), u = 2^-23 (twice the unit roundoff, for
    the matrix core's internal rounding). relu2 workload, K = H = 4096, every row
    of two experts: the FP32 h = fp32(y^2), y = fp32(acc * s), is compared with
    the exact y^2 through that bound, plus the two FP32 roundings."""
    w = synth.WORKLOADS["relu2"]
    run = GpuCase(pm, w)
    xq, xs, xg = oq.quantize_input_per_token(run.x)
    W = oracle_weights(w)
    rt = om.route(run.ids, w.E)
    h_gpu = run.views["h"].cpu().numpy()
    u = 2.0 ** -23
    gamma = w.H * u / (1 - w.H * u)
    for e in (0, 37):
        rows = np.arange(rt.offsets[e], rt.offsets[e + 1])
        tok = rt.route_of_row[rows] // w.K
        A = oq.dequantize_blocks(xq[tok], xs[tok])            # exact decoded values, float64
        w1q, w1sf, al1 = W.expert(e)[:3]
        B = oq.dequantize_blocks(w1q, w1sf)
        s = (xg[tok].astype(np.float32) * np.float32(al1)).astype(np.float64)[:, None]
        y = (A @ B.T) * s                                      # exact up to float64 rounding
        dy = gamma * (np.abs(A) @ np.abs(B).T) * s * (1 + 2.0 ** -20) + u * np.abs(y)
        h = h_gpu[rows].astype(np.float64)
        bound = (2 * np.abs(y) + dy) * dy + (np.abs(y) + dy) ** 2 * u
        ok = np.where(y > 0, np.abs(h - y * y) <= bound, h <= dy * dy * (1 + u))
        bad = np.argwhere(~ok)
        assert bad.size == 0, f"expert {e}: {len(bad)} entries outside the bound, first {bad[:4].tolist()}"


# ----------------------------------------------------------------------------- full size
@pytest.mark.parametrize("name", ["ep4_t512", "ep4_t1024"])
def test_moe_ep4_sampled(pm, name):
    """The EP4 one-GPU share (E=96, H=7168, I=3072, top-6, two hot experts), in the launch
    configuration the bench times (two streams): z rows of experts on both streams --
    including both sides of the split and the hot expert of the second stream -- and
    the outputs of 8 tokens."""
    import torch
    w = synth.WORKLOADS[name]
    run = GpuCase(pm, w)
    counts = np.diff(run.views["expert_offsets"].cpu().numpy())
    assert counts[0] > 5 * np.median(counts)                         # a hot expert spans many M-tiles
    experts, _ = _sampled_parity(w, run)
    assert 48 in experts and w.E - 1 in experts
    del run
    torch.cuda.empty_cache()


def test_large_batch_invariance_and_refresh(pm):
    """T=4096, E=256, H=7168, I=2048, top-8: T=1 vs T=4096 bitwise, sampled z rows and 8
    tokens against the oracle, then an in-place refresh with new weights tracks the oracle
    of the new weights."""
    import torch
    w = synth.WORKLOADS["large"]
    run = GpuCase(pm, w)
    full = run.out_bits()
    for t in (0, 2047, 4095):
        one = GpuCase(pm, w, T=1, x=run.x[t:t + 1], ids=run.ids[t:t + 1], wts=run.wts[t:t + 1], weights=run.P)
        assert np.array_equal(one.out_bits()[0], full[t]), f"token {t}"
    experts, _ = _sampled_parity(w, run)
    assert max(experts) >= 114
    # in-place refresh
    w2 = w.with_(weight_epoch=1)
    ptr = run.P.w1_codes.data_ptr()
    pm.prepare_weights(*synth.all_weights(w2, device="cuda"), out=run.P)
    again = GpuCase(pm, w, x=run.x, ids=run.ids, wts=run.wts, weights=run.P)
    assert run.P.w1_codes.data_ptr() == ptr
    assert not np.array_equal(again.out_bits(), full)
    res2 = _oracle(w2, run.x, run.ids, run.wts, experts=[5, 200], weights=oracle_weights(w2, [5, 200]))
    rows = np.nonzero(res2.computed_rows)[0]
    _assert_rows_close(bf16_bits(again.views["z"])[rows], res2.z[rows], "z after refresh")
    del run, again
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["ep4_t1024", "large"])
def test_plausibility_against_bf16_moe(pm, name):
    """The GPU output of 8 sampled tokens against the unquantized MoE on the same BF16
    inputs and weights (float64, the oracle's bf16_reference_moe, one token at a time over
    that token's experts): per-token cosine mean > 0.97 and min > 0.95, relative error in
    the band expected of 4-bit weights and activations."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from helpers import oracle_threads
    w = synth.WORKLOADS[name]
    run = GpuCase(pm, w)
    tokens, need = sample_tokens(run.ids, 0, (), n=8, n_part2=0, E=w.E)
    bf16_w = {}

    def gen(e):
        bf16_w[e] = synth.expert_weights(w, e)

    with ThreadPoolExecutor(oracle_threads()) as ex:
        list(ex.map(gen, need))

    def ref_token(t):
        ex_t = [int(e) for e in run.ids[t]]
        w1 = np.stack([bf16_w[e][0] for e in ex_t])
        w2 = np.stack([bf16_w[e][1] for e in ex_t])
        local = np.arange(len(ex_t), dtype=np.int32)[None]
        return om.bf16_reference_moe(run.x[t:t + 1], local, run.wts[t:t + 1], w1, w2, w.act)[0]

    with ThreadPoolExecutor(max(1, oracle_threads() // 4)) as ex:
        ref = np.stack(list(ex.map(ref_token, tokens)))
    got = bf16_to_f32(run.out_bits()[tokens]).astype(np.float64)
    cos = np.sum(got * ref, 1) / (np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"{name}: cosine mean {cos.mean():.4f} min {cos.min():.4f}, relative error {rel:.3f}")
    assert cos.mean() > 0.97 and cos.min() > 0.95, cos
    assert 0.03 < rel < 0.35, rel
    del run
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- invariance
def test_batch_invariance_with_large_cotokens(pm):
    """A target batch alone vs inside 193- and 1024-token batches whose other tokens are
    100x larger and routed to the same experts: bitwise identical outputs."""
    w = synth.WORKLOADS["swiglu"]
    rng = np.random.default_rng(4)
    target = 8
    x = synth.activations(w, 1024)
    ids, wts = synth.router(w, 1024)
    P = pm.prepare_weights(*synth.all_weights(w, device="cuda"))
    alone = GpuCase(pm, w, T=target, x=x[:target], ids=ids[:target], wts=wts[:target], weights=P).out_bits()
    xf = bf16_to_f32(x)
    for total in (193, 1024):
        xb = xf[:total].copy()
        xb[target:] *= 100.0
        xb = synth._bf16_np(xb)
        xb[:target] = x[:target]
        ib = ids[:total].copy()
        ib[target:] = ids[rng.integers(0, target, total - target)]       # same experts as the target
        big = GpuCase(pm, w, T=total, x=xb, ids=ib, wts=wts[:total], weights=P).out_bits()
        assert np.array_equal(big[:target], alone), f"batch of {total}"


def test_expert_offset_int64_and_repeat(pm):
    w = synth.WORKLOADS["tiny"]
    base = GpuCase(pm, w)
    again = GpuCase(pm, w, weights=base.P)
    assert np.array_equal(base.out_bits(), again.out_bits())
    assert np.array_equal(bf16_bits(base.views["z"]), bf16_bits(again.views["z"]))
    ids_shift = base.ids + 40
    ids_shift[1, 0] = -1
    ids_shift[2, 1] = 39                     # another rank's expert
    shifted = GpuCase(pm, w, ids=ids_shift, wts=base.wts, weights=base.P, offset=40, ids64=True)
    ref = base.ids.copy()
    ref[1, 0] = -1
    ref[2, 1] = -1
    masked = GpuCase(pm, w, ids=ref, wts=base.wts, weights=base.P)
    assert np.array_equal(shifted.out_bits(), masked.out_bits())
    res = _oracle(w, base.x, ref, base.wts)
    _assert_rows_close(masked.out_bits(), res.out, "out with invalid routes")


def test_all_routes_invalid_gives_zero(pm):
    w = synth.WORKLOADS["tiny"]
    ids = np.full((5, 2), -1, np.int32)
    run = GpuCase(pm, w, T=5, ids=ids, wts=np.ones((5, 2), np.float32))
    assert not run.out_bits().any()


def test_act_mismatch_is_rejected(pm):
    import pytest as _pt
    w = synth.WORKLOADS["tiny"]
    run = GpuCase(pm, w)
    with _pt.raises(pm.PmoeError) as ei:
        pm.routed_moe(run.xq, run.xs, run.xg, run.ids_dev, dev(run.wts), run.P, act=pm.ACT_SWIGLU)
    assert ei.value.code == 3 or ei.value.code == 4


def test_pointer_and_workspace_errors_leave_output_untouched(pm):
    """Host validation on a GPU: a host, a misaligned and a null pointer are
    PMOE_ERR_POINTER, a workspace one byte short is PMOE_ERR_WORKSPACE, and in
    every case nothing was launched: the output keeps its previous contents."""
    import torch
    w = synth.WORKLOADS["tiny"]
    run = GpuCase(pm, w)
    ids, wts = run.ids_dev, dev(run.wts)
    out = torch.full((w.T, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
    before = out.clone()

    def expect(code, **kw):
        args = dict(xq=run.xq, x_sf=run.xs, x_scale=run.xg, ws=run.ws)
        args.update(kw)
        with pytest.raises(pm.PmoeError) as ei:
            pm.routed_moe(args["xq"], args["x_sf"], args["x_scale"], ids, wts, run.P,
                          workspace=args["ws"], out=out)
        assert ei.value.code == code, (code, str(ei.value))

    expect(2, xq=run.xq.cpu())                                         # host memory
    raw = torch.empty(run.xq.numel() + 16, dtype=torch.uint8, device="cuda")
    expect(2, xq=raw[4:4 + run.xq.numel()].view(run.xq.shape))         # not 16-byte aligned
    expect(2, x_scale=None)                                            # null
    wsb = torch.empty(run.ws.numel() + 256, dtype=torch.uint8, device="cuda")
    expect(2, ws=wsb[16:16 + run.ws.numel()])                          # ws 16- but not 256-byte aligned
    raw64 = torch.zeros(ids.numel() * 2 + 2, dtype=torch.int32, device="cuda")
    ids64 = raw64[1:1 + ids.numel() * 2]                               # int64 ids 4- but not 8-byte aligned
    rc = pm.lib().pmoe_routed_moe(pm._ptr(run.xq), pm._ptr(run.xs), pm._ptr(run.xg), pm._ptr(ids64),
                                  pm.IDS_INT64, pm._ptr(wts), w.T, w.K, w.E, w.H, w.I, run.P.N1, 0,
                                  pm._ptr(run.P.w1_codes), pm._ptr(run.P.w1_scales),
                                  pm._ptr(run.P.w1_alpha), pm._ptr(run.P.w2_codes),
                                  pm._ptr(run.P.w2_scales), pm._ptr(run.P.w2_alpha), run.P.act,
                                  pm._ptr(run.ws), run.ws.numel(), pm._ptr(out), pm._stream())
    assert rc == 2 and "8-byte" in pm.lib().pmoe_last_error().decode()
    need = pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, run.P.act)
    expect(5, ws=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))
    _sync()
    assert torch.equal(out.view(torch.int16), before.view(torch.int16))
    pm.routed_moe(run.xq, run.xs, run.xg, ids, wts, run.P, workspace=run.ws, out=out)
    _sync()
    assert torch.equal(out.view(torch.int16), run.out.view(torch.int16))  # and the same call succeeds
