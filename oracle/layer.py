"""The steps on either side of the routed path, on the CPU: the router front, the
SwiGLU clamp, and the fused (order-free) finalize.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Readings (continuing the numbering of the other oracle modules):
  R23  Fused finalize (the default, non-deterministic mode the two-stage
       finalize replaces [Megatron-LM #8262 . What is added; Why CuTe DSL]):
       each route's FC2 result in FP32, zf = fp32(acc2 * s), is multiplied by
       its routing weight and added into an FP32 accumulator in any order; the
       total is rounded once to BF16. Its plain definition, used here, is the
       exact sum of fp32(w * zf) rounded to BF16; the GPU's FP32 atomic adds
       in arbitrary order agree to FP32 rounding.
  R24  Router front: plain top-k (no group-limited routing [Megatron-LM #8262 .
       Performance]) over the local experts' FP32 logits, ties to the lower
       expert id. Softmax is strictly increasing, so the top-k of the logits is
       the top-k of the probabilities; choosing on the logits keeps the choice
       exact. Weights are the softmax probabilities of the chosen experts,
       p_e = exp(l_e - max) / sum_all exp(l - max), optionally renormalized to
       sum 1 over the top k.
  R25  SwiGLU clamp with limit L > 0: gate = min(gate, L), up = min(max(up, -L),
       L), then silu(gate) * up [FlashInfer #5019 . Tensor and numerical
       contract, 'Compute order']; L = 0 means no clamp.
"""
import numpy as np

from .formats import f32_to_bf16_rne

F32 = np.float32


def router_topk(logits, k, renormalize=False):
    """FP32 logits [T, E] -> (ids int32 [T, k], weights float32 [T, k]) (reading R24).

    Selection: the k largest logits, larger first, equal logits by lower id.
    Weights: float64 softmax over all E, rounded to FP32, then (optionally)
    divided by their sum in FP32.
    """
    lg = np.asarray(logits, F32)
    T, E = lg.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -lg.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    l64 = lg.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1).astype(F32)
    if renormalize:
        s = np.zeros((T,), F32)
        for j in range(k):
            s = (s + w[:, j]).astype(F32)
        w = (w / s[:, None]).astype(F32)
    return ids, w


def swiglu_clamp(gate, up, limit):
    """Clamped SwiGLU inputs (reading R25): gate <= L, -L <= up <= L; L = 0 leaves them."""
    gate = np.asarray(gate, F32)
    up = np.asarray(up, F32)
    if not limit:
        return gate, up
    L = F32(limit)
    return np.minimum(gate, L).astype(F32), np.minimum(np.maximum(up, -L), L).astype(F32)


def finalize_fused(zf, row_of_route, topk_w, T, K):
    """Order-free finalize (reading R23): out[t] = bf16( sum_j fp32(w[t,j] * zf[row(t,j)]) ).

    zf : float32 [R, H] unrounded FC2 rows. The sum is exact (float64 of the
    FP32 products) and rounded once: the GPU adds the same products in FP32 in
    arbitrary order, so it agrees to FP32 rounding, not bit for bit.
    """
    zf = np.asarray(zf, F32)
    H = zf.shape[1]
    rr = np.asarray(row_of_route).reshape(T, K)
    w = np.asarray(topk_w, F32).reshape(T, K)
    acc = np.zeros((T, H), np.float64)
    for j in range(K):
        r = rr[:, j]
        v = r >= 0
        acc[v] += (w[v, j][:, None] * zf[r[v]]).astype(F32)
    return f32_to_bf16_rne(acc.astype(F32))
