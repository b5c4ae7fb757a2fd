"""Routed-MoE expert path of the per-token NVFP4 recipe, as a plain CPU pipeline.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Steps (each function names its reading):
  gating       -- SwiGLU iff FC1 has twice FC2's input width
                  [Megatron-LM #8262 . What is added]
  route        -- stable expert-sorted permutation of the valid routes
  fc1          -- exact decoded products summed in float64, rounded once to
                  FP32, then the FP32 factor g_token * alpha1 [FlashInfer #5019 .
                  Tensor and numerical contract, 'Compute order']
  activation   -- squared ReLU or SwiGLU (gate rows first), in FP32
  requant      -- per routed row, from FP32 (quant.quantize_rows_f32)
  fc2          -- as fc1 with g_row * alpha2, rounded to BF16 per route
  finalize     -- per token, slot order, FP32 products and sums, one BF16
                  rounding; routing weights applied here, after FC2
                  [Megatron-LM #8262 . What is tested, 4. Train-gen parity;
                  FlashInfer #5019 . Tensor and numerical contract]
"""
from dataclasses import dataclass

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16_rne
from .quant import dequantize_blocks, dequantize_rows, quantize_rows_f32, quantize_weights

F32 = np.float32
ACTS = ("relu2", "swiglu")


# ----------------------------------------------------------------------------- gating
def detect_gating(n1, i, h_fc1=None, h_fc2=None):
    """Return True for a gated (SwiGLU) FC1, False for non-gated (squared ReLU).

    FC1 is [E, N1, H] and FC2 is [E, H, I]: N1 == 2*I is gated, N1 == I is not,
    anything else is rejected; both must agree on H [Megatron-LM #8262 . What
    is added]. Gate rows come first, then up rows (reading R12;
    [FlashInfer #5019 . Tensor and numerical contract, 'gate-then-up']).
    """
    if i <= 0 or n1 <= 0:
        raise ValueError("FC1/FC2 widths must be positive")
    if h_fc1 is not None and h_fc2 is not None and h_fc1 != h_fc2:
        raise ValueError("FC1 and FC2 disagree on the hidden size")
    if n1 == 2 * i:
        return True
    if n1 == i:
        return False
    raise ValueError(f"FC1 width {n1} is neither I={i} nor 2I={2 * i}")


# ----------------------------------------------------------------------------- routing
@dataclass
class Routing:
    row_of_route: np.ndarray   # int32 [T*K], -1 for an invalid route
    route_of_row: np.ndarray   # int64 [R], flat route index f = t*K + j of each row
    counts: np.ndarray         # int64 [E]
    offsets: np.ndarray        # int64 [E+1], exclusive scan of counts


def route(topk_ids, num_experts, expert_offset=0):
    """Expert-contiguous permutation of the routes.

    Route f = t*K + j is valid iff expert_offset <= id < expert_offset + E
    (local expert slice; invalid ids such as -1 contribute nothing). Rows are
    the valid routes sorted by local expert, ties by ascending f (reading R13).
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    flat = ids.reshape(-1)
    local = flat - int(expert_offset)
    valid = (local >= 0) & (local < num_experts)
    f_valid = np.nonzero(valid)[0]
    order = np.argsort(local[f_valid], kind="stable")
    route_of_row = f_valid[order]
    row_of_route = np.full(flat.shape, -1, dtype=np.int32)
    row_of_route[route_of_row] = np.arange(route_of_row.size, dtype=np.int32)
    counts = np.bincount(local[f_valid], minlength=num_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return Routing(row_of_route, route_of_row.astype(np.int64), counts, offsets)


# ----------------------------------------------------------------------------- GEMMs
def fc(aq, a_sf, a_scale, wq_e, w_sf_e, alpha_e):
    """One expert's grouped-GEMM rows: fp32( fp32(sum_k a_hat*w_hat) * fp32(g * alpha) ).

    a_hat, w_hat are the exactly decoded E2M1 x E4M3 values (no per-row or
    per-expert FP32 factor); the float64 matmul stands in for the exact sum and
    is rounded once to FP32 (reading R14: one combined multiplier applied after
    accumulation).
    """
    A = dequantize_blocks(aq, a_sf)
    B = dequantize_blocks(wq_e, w_sf_e)
    acc = (A @ B.T).astype(F32)
    s = (np.asarray(a_scale, F32) * F32(alpha_e)).astype(F32)
    return (acc * s[:, None]).astype(F32)


def activation(y, act, inter):
    """FP32 activation of FC1 outputs [n, N1] -> h [n, I].

    relu2:  h = fp32(r * r), r = max(y, 0)                (non-gated)
    swiglu: h = fp32(silu(gate) * up), silu(g) = fp32(g / fp32(1 + exp(-g))),
            gate = y[:, :I], up = y[:, I:]; no clamp, no offset
            [Megatron-LM #8262 . What is added].
    """
    y = np.asarray(y, F32)
    if act == "relu2":
        r = np.maximum(y, F32(0.0)).astype(F32)
        return (r * r).astype(F32)
    if act == "swiglu":
        gate = y[:, :inter]
        up = y[:, inter:]
        with np.errstate(over="ignore"):
            den = (1.0 + np.exp(-gate.astype(np.float64))).astype(F32)
        silu = (gate / den).astype(F32)
        return (silu * up).astype(F32)
    raise ValueError(act)


def finalize(z_bf16, row_of_route, topk_w, T, K):
    """Deterministic finalize: out[t] = bf16( sum_j fp32(w[t,j] * z[row(t,j)]) ).

    Accumulation starts at +0.0 in FP32 and walks the top-k slots in order
    j = 0..K-1 (reading R17), skipping invalid routes; every product and sum
    is rounded to FP32 separately, no fused multiply-add (reading R18); the
    sum is rounded to BF16 once.
    """
    z = bf16_to_f32(z_bf16)
    H = z.shape[1] if z.ndim == 2 and z.shape[0] > 0 else None
    rr = np.asarray(row_of_route).reshape(T, K)
    w = np.asarray(topk_w, F32).reshape(T, K)
    if H is None:
        raise ValueError("z must be [R, H] with R > 0; use finalize_empty for no routes")
    acc = np.zeros((T, H), F32)
    for j in range(K):
        r = rr[:, j]
        v = r >= 0
        term = (w[v, j][:, None] * z[r[v]]).astype(F32)
        acc[v] = (acc[v] + term).astype(F32)
    return f32_to_bf16_rne(acc)


# ----------------------------------------------------------------------------- weights
@dataclass
class Weights:
    """Canonical quantized expert weights (gate-then-up FC1, blocks along K)."""
    w1q: np.ndarray    # uint8 [E, N1, H/2]
    w1sf: np.ndarray   # uint8 [E, N1, H/16]
    a1: np.ndarray     # float32 [E]
    w2q: np.ndarray    # uint8 [E, H, I/2]
    w2sf: np.ndarray   # uint8 [E, H, I/16]
    a2: np.ndarray     # float32 [E]

    @property
    def shape(self):
        E, N1, h2 = self.w1q.shape
        return E, N1, 2 * h2, 2 * self.w2q.shape[2]

    def expert(self, e):
        return (self.w1q[e], self.w1sf[e], self.a1[e], self.w2q[e], self.w2sf[e], self.a2[e])


def prepare_weights(w1_bf16, w2_bf16):
    """BF16 stacks FC1 [E, N1, H], FC2 [E, H, I] -> canonical quantized Weights."""
    w1_bf16 = np.asarray(w1_bf16, np.uint16)
    w2_bf16 = np.asarray(w2_bf16, np.uint16)
    detect_gating(w1_bf16.shape[1], w2_bf16.shape[2], w1_bf16.shape[2], w2_bf16.shape[1])
    return Weights(*quantize_weights(w1_bf16), *quantize_weights(w2_bf16))


class LazyWeights:
    """Weights quantized per expert on first use, for stacks too large to hold.

    `source(e)` returns (w1_bf16 [N1, H], w2_bf16 [H, I]) of expert e.
    `cache` (optional) is the dict that keeps the quantized experts, so several
    instances over the same source can share one.
    """

    def __init__(self, source, E, N1, H, I, cache=None):
        self._source, self._cache = source, ({} if cache is None else cache)
        self._shape = (E, N1, H, I)
        detect_gating(N1, I)

    @property
    def shape(self):
        return self._shape

    def expert(self, e):
        if e not in self._cache:
            w1, w2 = self._source(e)
            p1 = quantize_weights(np.asarray(w1, np.uint16)[None])
            p2 = quantize_weights(np.asarray(w2, np.uint16)[None])
            self._cache[e] = (p1[0][0], p1[1][0], p1[2][0], p2[0][0], p2[1][0], p2[2][0])
        return self._cache[e]


# ----------------------------------------------------------------------------- pipeline
@dataclass
class MoeResult:
    out: np.ndarray            # uint16 BF16 [T, H]
    routing: Routing
    h: np.ndarray              # float32 [R, I] (rows not computed stay 0)
    hq: np.ndarray             # uint8 [R, I/2]
    h_sf: np.ndarray           # uint8 [R, I/16]
    h_scale: np.ndarray        # float32 [R]
    z: np.ndarray              # uint16 BF16 [R, H]
    computed_rows: np.ndarray  # bool [R]


def routed_moe(xq, x_sf, x_scale, topk_ids, topk_w, weights, act, expert_offset=0,
               tokens=None, experts=None):
    """S2..S6 of the path on per-token-quantized activations.

    `weights` is a Weights or LazyWeights. `tokens` (optional) restricts the
    computation to a subset of tokens; every token's result depends only on
    its own row and routes, so the subset is exact and the other outputs are 0.
    `experts` (optional) restricts the per-route rows (h, hq, z) to the given
    local experts; the finalized output is then not computed (zeros).
    """
    E, N1, H, I = weights.shape
    gated = detect_gating(N1, I)
    if act not in ACTS or gated != (act == "swiglu"):
        raise ValueError(f"activation {act!r} does not match the FC1 shape")
    ids = np.asarray(topk_ids)
    T, K = ids.shape
    rt = route(ids, E, expert_offset)
    R = rt.route_of_row.size
    tok_of_row = rt.route_of_row // K
    want = np.ones(T, bool) if tokens is None else np.isin(np.arange(T), np.asarray(tokens))
    row_on = want[tok_of_row] if R else np.zeros(0, bool)
    if experts is not None and R:
        exp_of_row = np.repeat(np.arange(E), rt.counts)
        row_on &= np.isin(exp_of_row, np.asarray(experts))

    h = np.zeros((R, I), F32)
    for e in range(E):
        rows = np.arange(rt.offsets[e], rt.offsets[e + 1])
        rows = rows[row_on[rows]] if rows.size else rows
        if rows.size == 0:
            continue
        w1q, w1sf, a1, _, _, _ = weights.expert(e)
        t = tok_of_row[rows]
        y = fc(xq[t], x_sf[t], x_scale[t], w1q, w1sf, a1)
        h[rows] = activation(y, act, I)

    hq = np.zeros((R, I // 2), np.uint8)
    h_sf = np.zeros((R, I // 16), np.uint8)
    h_scale = np.zeros((R,), F32)
    if row_on.any():
        q, s, g = quantize_rows_f32(h[row_on])
        hq[row_on], h_sf[row_on], h_scale[row_on] = q, s, g

    z = np.zeros((R, H), np.uint16)
    for e in range(E):
        rows = np.arange(rt.offsets[e], rt.offsets[e + 1])
        rows = rows[row_on[rows]] if rows.size else rows
        if rows.size == 0:
            continue
        _, _, _, w2q, w2sf, a2 = weights.expert(e)
        zf = fc(hq[rows], h_sf[rows], h_scale[rows], w2q, w2sf, a2)
        z[rows] = f32_to_bf16_rne(zf)

    if R and experts is None:
        out = finalize(z, rt.row_of_route, topk_w, T, K)
    else:
        out = np.zeros((T, H), np.uint16)
    if tokens is not None:
        out[~want] = 0
    return MoeResult(out, rt, h, hq, h_sf, h_scale, z, row_on)


# ----------------------------------------------------------------------------- references
def _act64(y, act, inter, swiglu_limit=0.0):
    if act == "relu2":
        r = np.maximum(y, 0.0)
        return r * r
    gate, up = y[..., :inter], y[..., inter:]
    if swiglu_limit:
        gate = np.minimum(gate, swiglu_limit)
        up = np.clip(up, -swiglu_limit, swiglu_limit)
    return gate / (1.0 + np.exp(-gate)) * up


def brute_force_moe(x_f32, topk_ids, topk_w, w1, w2, act, expert_offset=0, quantize=None,
                    swiglu_limit=0.0):
    """Per-token, per-slot float64 MoE with no sorting or grouping.

    x_f32 [T, H]; w1 [E, N1, H], w2 [E, H, I] as float arrays. With
    quantize=None this is the textbook routed MoE
        out[t] = sum_j w[t,j] * FC2_e( act( FC1_e(x[t]) ) ),  e = id[t,j] - offset.
    With `quantize` = (qx, qw1, qw2, qh), callables returning dequantized float64
    arrays, the same loop runs on dequantized tensors, requantizing the FP32
    intermediate with qh. swiglu_limit > 0 clamps the SwiGLU inputs (gate from
    above, up on both sides).
    """
    x = np.asarray(x_f32, np.float64)
    T, K = np.asarray(topk_ids).shape
    E, N1, H = w1.shape
    I = w2.shape[2]
    if quantize is not None:
        qx, qw1, qw2, qh = quantize
        x = qx(x)
        w1 = qw1(w1)
        w2 = qw2(w2)
    out = np.zeros((T, H), np.float64)
    for t in range(T):
        for j in range(K):
            e = int(topk_ids[t][j]) - expert_offset
            if not (0 <= e < E):
                continue
            y = w1[e] @ x[t]
            h = _act64(y, act, I, swiglu_limit)
            if quantize is not None:
                h = qh(h[None].astype(np.float32))[0]
            out[t] += float(topk_w[t][j]) * (w2[e] @ h)
    return out


def bf16_reference_moe(x_bf16, topk_ids, topk_w, w1_bf16, w2_bf16, act, expert_offset=0):
    """Unquantized MoE on the BF16 inputs and weights (float64), for plausibility checks."""
    return brute_force_moe(bf16_to_f32(x_bf16), topk_ids, topk_w,
                           bf16_to_f32(w1_bf16).astype(np.float64),
                           bf16_to_f32(w2_bf16).astype(np.float64), act, expert_offset)


def dequant_activation(x):
    """float -> per-token quantized and dequantized float64 (for brute_force_moe)."""
    q, s, g = quantize_rows_f32(np.asarray(x, F32))
    return dequantize_rows(q, s, g).astype(np.float64)


def dequant_weights(w):
    """[E, N, K] float -> NVFP4-quantized and dequantized float64 (for brute_force_moe)."""
    from .quant import block_quantize, weight_global_scale
    from .formats import pack_nibbles
    w = np.asarray(w, F32)
    out = np.empty(w.shape, np.float64)
    for e in range(w.shape[0]):
        alpha, _ = weight_global_scale(w[e])
        codes, sf = block_quantize(w[e], np.full(w.shape[1], alpha, F32))
        out[e] = dequantize_rows(pack_nibbles(codes), sf, np.full(w.shape[1], alpha, F32))
    return out
