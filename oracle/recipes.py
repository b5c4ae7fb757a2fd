"""Two further precision recipes of the routed-MoE path, on the CPU.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The extension table of [Megatron-LM #8262 . How to extend] lists, beside the
per-token recipe:

  per_tensor   (w4a4)  FC1 input quantized with a fixed, calibrated scale a1;
                       no per-token scale; fc1_alpha = 1/(w_scale * a1),
                       fc2_alpha = 1/(w_scale * a2); the FC2 input is
                       quantized with the fixed scale a2. Packed weights and
                       block scales are those of the per-token recipe.
  weight_only  (w4a16) BF16 activations, not quantized; alphas = 1/w_scale;
                       weights unchanged.

Readings (continuing the numbering of the per-token recipe):
  R20  A static input scale a follows the weights' global-scale convention
       (a = 2688 / calibrated amax): the quantizer runs the per-token block
       steps with the row scale g = fp32(1 / a) for every row, exactly as the
       weight quantizer does with g = alpha = fp32(1 / w_scale).
  R21  Folding: alpha' = fp32( 1 / fp32(w_scale * a) ), w_scale = fp32(2688 /
       amax_e) of the expert matrix; the GEMM applies y = fp32(acc * alpha').
  R22  W4A16: y = fp32( fp32(sum_k x_k * w_hat_k) * alpha_e ); the FC1 output
       passes through the FP32 activation and is rounded once to BF16 (RNE),
       which is FC2's input; z = bf16(fp32(acc2 * alpha2_e)). Activations and
       intermediates stay BF16 [FlashInfer #5019 . Tensor and numerical
       contract, 'Compute order'].
"""
from dataclasses import dataclass

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16_rne, pack_nibbles
from .layer import finalize_fused, swiglu_clamp
from .moe import Routing, Weights, activation, detect_gating, finalize, route, ACTS
from .quant import (block_quantize, dequantize_blocks, quantize_rows_f32, quantize_weights,
                    weight_global_scale)

F32 = np.float32
RECIPES = ("per_token", "per_tensor", "weight_only")


# ----------------------------------------------------------------------------- per-tensor
def static_row_scale(a):
    """Row scale of a quantizer with a static global scale a (reading R20): fp32(1 / a)."""
    with np.errstate(divide="ignore"):
        return F32(F32(1.0) / F32(a))


def quantize_rows_static(x, a):
    """FP32 rows [R, L] quantized with one static scale a -> (packed [R, L/2], sf [R, L/16]).

    The block steps are those of the per-token quantizer (readings R6, R7)
    with g = fp32(1 / a) for every row; values beyond the range the scale
    allows saturate (E4M3 scales at 448, codes at 6; readings R1, R4).
    """
    x = np.asarray(x, dtype=F32)
    g = np.full((x.shape[0],), static_row_scale(a), dtype=F32)
    codes, sf = block_quantize(x, g)
    return pack_nibbles(codes), sf


def quantize_input_per_tensor(x_bf16, a1):
    """BF16 activations [T, H] (uint16 bits) -> (xq [T, H/2], x_sf [T, H/16]) with the static a1."""
    return quantize_rows_static(bf16_to_f32(x_bf16), a1)


def fold_input_scale(w_bf16, a):
    """Per-expert alpha' = fp32(1 / fp32(w_scale_e * a)) for a stack [E, N, K] (reading R21)."""
    w = bf16_to_f32(np.asarray(w_bf16, np.uint16))
    out = np.empty((w.shape[0],), F32)
    for e in range(w.shape[0]):
        _, w_scale = weight_global_scale(w[e])
        with np.errstate(divide="ignore", over="ignore"):
            out[e] = F32(1.0) / F32(w_scale * F32(a))
    return out


def prepare_weights_per_tensor(w1_bf16, w2_bf16, a1, a2):
    """Per-tensor prepared weights: the per-token codes and scales, folded alphas."""
    w1_bf16 = np.asarray(w1_bf16, np.uint16)
    w2_bf16 = np.asarray(w2_bf16, np.uint16)
    detect_gating(w1_bf16.shape[1], w2_bf16.shape[2], w1_bf16.shape[2], w2_bf16.shape[1])
    q1, s1, _ = quantize_weights(w1_bf16)
    q2, s2, _ = quantize_weights(w2_bf16)
    return Weights(q1, s1, fold_input_scale(w1_bf16, a1), q2, s2, fold_input_scale(w2_bf16, a2))


class LazyWeightsPerTensor:
    """Per-tensor weights quantized per expert on first use (stacks too large to hold).

    `source(e)` returns (w1_bf16 [N1, H], w2_bf16 [H, I]) of expert e; a1, a2 are
    folded into that expert's alphas (reading R21). `cache` (optional) is the
    dict that keeps the quantized experts, shared by instances with the same
    source and scales.
    """

    def __init__(self, source, E, N1, H, I, a1, a2, cache=None):
        self._source, self._cache = source, ({} if cache is None else cache)
        self._shape = (E, N1, H, I)
        self._a1, self._a2 = F32(a1), F32(a2)
        detect_gating(N1, I)

    @property
    def shape(self):
        return self._shape

    def expert(self, e):
        if e not in self._cache:
            w1, w2 = (np.asarray(m, np.uint16)[None] for m in self._source(e))
            q1, s1, _ = quantize_weights(w1)
            q2, s2, _ = quantize_weights(w2)
            self._cache[e] = (q1[0], s1[0], fold_input_scale(w1, self._a1)[0],
                              q2[0], s2[0], fold_input_scale(w2, self._a2)[0])
        return self._cache[e]


# ----------------------------------------------------------------------------- pipeline
@dataclass
class RecipeResult:
    out: np.ndarray            # uint16 BF16 [T, H]
    routing: Routing
    h: np.ndarray              # float32 [R, I] FP32 activation output
    hq: np.ndarray             # NVFP4 recipes: uint8 [R, I/2]; weight_only: empty
    h_sf: np.ndarray           # NVFP4 recipes: uint8 [R, I/16]; weight_only: empty
    h_bf16: np.ndarray         # weight_only: uint16 [R, I] FC2 input; else empty
    z: np.ndarray              # uint16 BF16 [R, H]
    computed_rows: np.ndarray  # bool [R]
    zf: np.ndarray = None      # float32 [R, H] unrounded FC2 rows (input of the fused finalize)


def _fc_exact(A, wq_e, w_sf_e, alpha_e, row_scale=None):
    """fp32( fp32(A @ w_hat^T) * s ) with A float64 holding exact input values;
    s = fp32(row_scale * alpha) per row, or alpha alone."""
    B = dequantize_blocks(wq_e, w_sf_e)
    acc = (A @ B.T).astype(F32)
    if row_scale is None:
        return (acc * F32(alpha_e)).astype(F32)
    s = (np.asarray(row_scale, F32) * F32(alpha_e)).astype(F32)
    return (acc * s[:, None]).astype(F32)


def _act(y, act, inter, limit):
    if act == "swiglu" and limit:
        gate, up = swiglu_clamp(y[:, :inter], y[:, inter:], limit)
        y = np.concatenate([gate, up], axis=1)
    return activation(y, act, inter)


def routed_moe_recipe(recipe, x, topk_ids, topk_w, weights, act, expert_offset=0, a2=None,
                      tokens=None, experts=None, swiglu_limit=0.0, finalize_mode="ordered"):
    """S2..S6 under one recipe, with the layer options.

    per_token  : x = (xq, x_sf, x_scale) from quant.quantize_input_per_token;
                 the same arithmetic as moe.routed_moe.
    per_tensor : x = (xq, x_sf) from quantize_input_per_tensor; `weights` from
                 prepare_weights_per_tensor (folded alphas); a2 = the static FC2
                 input scale.
    weight_only: x = BF16 activations [T, H] (uint16 bits); `weights` from the
                 per-token preparation (alphas = 1/w_scale).
    swiglu_limit : SwiGLU clamp limit (reading R25); 0 = none.
    finalize_mode: "ordered" (fixed slot order, BF16 z) or "fused" (reading R23).
    `tokens` / `experts` restrict the work as in moe.routed_moe.
    """
    if recipe not in RECIPES:
        raise ValueError(recipe)
    if finalize_mode not in ("ordered", "fused"):
        raise ValueError(finalize_mode)
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

    x_scale = None
    if recipe == "per_token":
        xq, x_sf, x_scale = x
    elif recipe == "per_tensor":
        xq, x_sf = x
    else:
        x_f64 = bf16_to_f32(x).astype(np.float64)

    def rows_of(e):
        rows = np.arange(rt.offsets[e], rt.offsets[e + 1])
        return rows[row_on[rows]] if rows.size else rows

    h = np.zeros((R, I), F32)
    for e in range(E):
        rows = rows_of(e)
        if rows.size == 0:
            continue
        w1q, w1sf, al1, _, _, _ = weights.expert(e)
        t = tok_of_row[rows]
        A = x_f64[t] if recipe == "weight_only" else dequantize_blocks(xq[t], x_sf[t])
        rs = x_scale[t] if recipe == "per_token" else None
        h[rows] = _act(_fc_exact(A, w1q, w1sf, al1, rs), act, I, swiglu_limit)

    nvfp4 = recipe != "weight_only"
    hq = np.zeros((R, I // 2) if nvfp4 else (0, 0), np.uint8)
    h_sf = np.zeros((R, I // 16) if nvfp4 else (0, 0), np.uint8)
    h_scale = np.zeros((R,), F32)
    h_bf16 = np.zeros((R, I) if not nvfp4 else (0, 0), np.uint16)
    if row_on.any():
        if recipe == "per_token":
            hq[row_on], h_sf[row_on], h_scale[row_on] = quantize_rows_f32(h[row_on])
        elif recipe == "per_tensor":
            hq[row_on], h_sf[row_on] = quantize_rows_static(h[row_on], a2)
        else:
            h_bf16[row_on] = f32_to_bf16_rne(h[row_on])

    z = np.zeros((R, H), np.uint16)
    zf = np.zeros((R, H), F32)
    for e in range(E):
        rows = rows_of(e)
        if rows.size == 0:
            continue
        _, _, _, w2q, w2sf, al2 = weights.expert(e)
        if nvfp4:
            A = dequantize_blocks(hq[rows], h_sf[rows])
        else:
            A = bf16_to_f32(h_bf16[rows]).astype(np.float64)
        zf[rows] = _fc_exact(A, w2q, w2sf, al2, h_scale[rows] if recipe == "per_token" else None)
        z[rows] = f32_to_bf16_rne(zf[rows])

    if R and experts is None:
        if finalize_mode == "ordered":
            out = finalize(z, rt.row_of_route, topk_w, T, K)
        else:
            out = finalize_fused(zf, rt.row_of_route, topk_w, T, K)
    else:
        out = np.zeros((T, H), np.uint16)
    if tokens is not None:
        out[~want] = 0
    return RecipeResult(out, rt, h, hq, h_sf, h_bf16, z, row_on, zf)


# ----------------------------------------------------------------------------- brute force
def dequant_static(x, a):
    """float rows -> quantized with the static scale a and dequantized, float64 (brute force)."""
    x = np.asarray(x, F32)
    q, sf = quantize_rows_static(x, a)
    g = static_row_scale(a)
    return (dequantize_blocks(q, sf).astype(F32) * g).astype(F32).astype(np.float64)
