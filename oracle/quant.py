"""NVFP4 quantizers of the routed-MoE path, step by step in FP32.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

All arithmetic that decides a stored byte is done in IEEE binary32 with numpy
float32 operations (each +, *, / is correctly rounded), so the GPU kernels must
reproduce these bits exactly. Denormals are kept.

Block layout: one E4M3 scale per 16 consecutive elements along the reduction
dimension (K = hidden size for FC1 inputs / weights, K = intermediate size for
FC2) [FlashInfer #5019 . Tensor and numerical contract, scale shapes [E,N,K/16]].
"""
import numpy as np

from .formats import (e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode_sat,
                      pack_nibbles, unpack_nibbles, bf16_to_f32)

BLOCK = 16
# Recipe global constant 1/(448*6): 448 is the E4M3 maximum, 6 the E2M1 maximum
# [Megatron-LM #8262 . What is added; How to extend]. Reading R5: it is used as
# its FP32 rounding, 0x1.861862p-12.
RECIPE_CONST = np.float32(1.0 / 2688.0)
F32 = np.float32


def block_quantize(x, g):
    """Quantize rows of FP32 values given one FP32 scale per row.

    x : float32 [R, L], L a multiple of 16;  g : float32 [R] (the row scale).
    Returns (codes uint8 [R, L] unpacked nibbles, sf uint8 [R, L/16]).

    For every 16-block b of a row (readings R6, R7):
      amax_b = max |x_i|
      sf_b   = E4M3_sat( fp32( fp32(amax_b / 6) / g ) )    (0 when g == 0)
      e_b    = fp32( dec(sf_b) * g )
      q_i    = E2M1( fp32(x_i / e_b) )   when e_b > 0, else code 0x0
    """
    x = np.asarray(x, dtype=F32)
    g = np.asarray(g, dtype=F32)
    R, L = x.shape
    assert L % BLOCK == 0 and g.shape == (R,)
    xb = x.reshape(R, L // BLOCK, BLOCK)
    amax_b = np.max(np.abs(xb), axis=2)                       # float32, exact
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = amax_b / F32(6.0)                                  # fp32 division
        v = t / g[:, None]                                     # fp32 division
    v = np.where(g[:, None] > 0, v, F32(0.0)).astype(F32)
    sf = e4m3_encode_sat(v)
    e = e4m3_decode(sf).astype(F32) * g[:, None]               # fp32 product
    e = e.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = xb / e[:, :, None]                                 # fp32 division
    codes = np.where(e[:, :, None] > 0, e2m1_encode(q), np.uint8(0))
    return codes.reshape(R, L).astype(np.uint8), sf.astype(np.uint8)


def per_row_scale(x):
    """Per-row scale g = fp32(amax * fp32(1/2688)) (reading R5); 0 for an all-zero row.

    The per-token scale is the token's absolute maximum times the recipe
    constant [Megatron-LM #8262 . What is added; How to extend table, rows
    'FC1 input' and 'per_token_scale'].
    """
    x = np.asarray(x, dtype=F32)
    amax = np.max(np.abs(x), axis=1).astype(F32)
    return (amax * RECIPE_CONST).astype(F32)


def quantize_rows_f32(x):
    """Per-row NVFP4 quantization of FP32 rows (intermediate requant, reading R15).

    x : float32 [R, L]. Returns (packed uint8 [R, L/2], sf uint8 [R, L/16],
    scale float32 [R]).
    """
    x = np.asarray(x, dtype=F32)
    g = per_row_scale(x)
    codes, sf = block_quantize(x, g)
    return pack_nibbles(codes), sf, g


def quantize_input_per_token(x_bf16):
    """Per-token NVFP4 quantization of BF16 activations (uint16 bit patterns [T, H]).

    Online, one FP32 scale per token, no calibration [Megatron-LM #8262 .
    Background; What is added]. Returns (xq uint8 [T, H/2], x_sf uint8 [T, H/16],
    x_scale float32 [T]).
    """
    return quantize_rows_f32(bf16_to_f32(x_bf16))


def weight_global_scale(w):
    """Per-expert (alpha, w_scale) for one FP32 matrix (reading R10).

    w_scale = fp32(2688 / amax), alpha = fp32(1 / w_scale); alpha is the
    per-expert FP32 factor the GEMM applies after accumulation
    [Megatron-LM #8262 . How to extend table, row 'fc1_alpha / fc2_alpha'].
    amax == 0 gives w_scale = +inf and alpha = 0 (reading R11).
    """
    amax = F32(np.max(np.abs(np.asarray(w, dtype=F32))))
    with np.errstate(divide="ignore"):
        w_scale = F32(2688.0) / amax
        alpha = F32(1.0) / w_scale
    return F32(alpha), F32(w_scale)


def quantize_weight_matrix(w_bf16):
    """One expert's BF16 matrix [N, K] (uint16) -> (packed [N, K/2], sf [N, K/16], alpha).

    One amax over the whole matrix -- for a gated FC1 over the gate and up
    halves together -- gives one alpha per expert and FC (reading R9); the
    blocks then use g = alpha (steps of block_quantize).
    """
    w = bf16_to_f32(w_bf16)
    alpha, _ = weight_global_scale(w)
    g = np.full((w.shape[0],), alpha, dtype=F32)
    codes, sf = block_quantize(w, g)
    return pack_nibbles(codes), sf, alpha


def quantize_weights(w_bf16):
    """Stack [E, N, K] of BF16 -> (packed [E, N, K/2], sf [E, N, K/16], alpha [E])."""
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    E, N, K = w_bf16.shape
    q = np.empty((E, N, K // 2), np.uint8)
    s = np.empty((E, N, K // BLOCK), np.uint8)
    a = np.empty((E,), np.float32)
    for e in range(E):
        q[e], s[e], a[e] = quantize_weight_matrix(w_bf16[e])
    return q, s, a


def dequantize_blocks(packed, sf):
    """Packed codes [R, L/2] + block scales [R, L/16] -> float64 [R, L] = val(q) * dec(sf).

    Each product has at most 6 significant bits and is exact in float64 (and in
    FP16/BF16).
    """
    codes = unpack_nibbles(packed)
    R, L = codes.shape
    vals = e2m1_decode(codes).reshape(R, L // BLOCK, BLOCK)
    return (vals * e4m3_decode(sf)[:, :, None]).reshape(R, L)


def dequantize_rows(packed, sf, g):
    """Full dequantization x_hat = fp32( fp32(val(q) * dec(sf)) * g ) as float32 [R, L]."""
    inner = dequantize_blocks(packed, sf).astype(F32)          # exact
    return (inner * np.asarray(g, F32).reshape(-1, 1)).astype(F32)
