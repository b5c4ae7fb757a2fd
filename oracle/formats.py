"""Number formats of the NVFP4 recipe, written from their definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

NVFP4 as used on the pages: E2M1 element codes, one E4M3 block scale per 16
elements, plus one FP32 scale per token (activations) or per expert (weights)
[Megatron-LM #8262 . Background]; codes are packed two per byte
[FlashInfer #5019 . Tensor and numerical contract].

E2M1: 1 sign, 2 exponent, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
E4M3 ("fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest
finite 448 (byte 0x7E); 0x7F/0xFF are NaN; no infinities; subnormal step 2^-9.
BF16: the upper 16 bits of an IEEE binary32.
"""
import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0


# ----------------------------------------------------------------------------- E2M1
def e2m1_decode(codes):
    """Nibble codes (0..15) -> float64 values. Bit 3 is the sign (0x8 is -0)."""
    c = np.asarray(codes).astype(np.uint8)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_encode(v):
    """float32 values -> nibble codes, round-to-nearest with ties to the even code.

    Reading R1: deterministic round-to-nearest (the training-side recipe named
    in [Megatron-LM #8262 . Background] disables stochastic rounding); a value
    exactly between two neighbours goes to the one whose code is even, which is
    IEEE ties-to-even on the one-bit mantissa. Magnitudes above 6 saturate to 6.
    Reading R2: the sign bit is the IEEE sign of the input, so a negative value
    that rounds to zero (and -0.0) gives 0x8.

    The rule is written as "count the midpoints the magnitude has passed": the
    code of a magnitude a is the number of consecutive-pair midpoints m_c
    (between codes c and c+1) with a > m_c, or a == m_c when c+1 is even.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)                      # every midpoint is exact in float32
    code = np.zeros(a.shape, dtype=np.uint8)
    for c in range(7):
        mid = np.float32(0.5 * (E2M1_MAGNITUDES[c] + E2M1_MAGNITUDES[c + 1]))
        tie_goes_up = ((c + 1) % 2) == 0
        passed = (a >= mid) if tie_goes_up else (a > mid)
        code += passed
    code |= np.signbit(v).view(np.uint8) << np.uint8(3)
    return code


def pack_nibbles(codes):
    """[..., 2n] nibble codes -> [..., n] bytes; element 2i in the low nibble (reading R3)."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[..., n] bytes -> [..., 2n] nibble codes (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------- E4M3
def e4m3_decode(b):
    """E4M3fn bytes -> float64 values (NaN for 0x7F / 0xFF)."""
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 7
    sub = (m / 8.0) * 2.0 ** (1 - 7)
    nrm = (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(s == 1, -val, val)


# The 127 non-negative finite E4M3 values in byte order 0x00..0x7E; byte order
# equals value order for non-negative E4M3, which the encoder relies on.
_E4M3_GRID = e4m3_decode(np.arange(0x7F))


def e4m3_encode_sat(v):
    """Non-negative float32 values (or +inf) -> E4M3fn bytes.

    Round to nearest, ties to the even code (= even mantissa), and values at or
    above 448 -- including +inf -- saturate to 448 (0x7E). Reading R4: the
    pages name E4M3 and its maximum 448 as part of the recipe constant
    [Megatron-LM #8262 . What is added] but not an overflow rule; saturation
    keeps every block scale finite.
    """
    a = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(a)) or np.any(a < 0):
        raise ValueError("e4m3_encode_sat expects non-negative, non-NaN values")
    grid = _E4M3_GRID
    a_cl = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(grid, a_cl, side="left")          # grid[hi] >= a
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_cl - grid[lo]
    d_hi = grid[hi] - a_cl
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    out = np.where(pick_hi, hi, lo)
    out = np.where(a_cl == grid[hi], hi, out)               # exact hits
    return out.astype(np.uint8)


# ----------------------------------------------------------------------------- BF16
def bf16_to_f32(u16):
    """BF16 bit patterns (uint16) -> float32."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def f32_to_bf16_rne(x):
    """float32 -> BF16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = np.where(nan, (u >> 16) | 0x40, rounded)
    return out.astype(np.uint16)
