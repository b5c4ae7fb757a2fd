// Device-side building blocks shared by the pmoe kernels (gfx950 only).
//
// Number formats of the per-token NVFP4 recipe [Megatron-LM #8262 . Background]:
// E2M1 codes (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign), E4M3 ("fn")
// block scales (bias 7, largest finite 448 = 0x7E), one scale per 16 elements
// along the reduction dimension [FlashInfer #5019 . Tensor and numerical contract].
// Everything that decides a stored byte is plain IEEE binary32 arithmetic
// (correctly rounded division, denormals kept, no contraction: the library is
// compiled with -ffp-contract=off), so it reproduces the CPU definition bit for
// bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmoe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2v_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// fp32(1 / (448 * 6)): the recipe's global constant [Megatron-LM #8262 . What is added].
constexpr float kRecipeConst = 0x1.861862p-12f;
constexpr int kBlock = 16;  // elements per E4M3 block scale

// ------------------------------------------------------------------ BF16
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest even; NaN stays a (quiet) NaN: the BF16 bits are
// (u + 0x7FFF + bit 16 of u) >> 16 for non-NaN bits u, and (u >> 16) | 0x40
// for NaN. gfx950's v_cvt_pk_bf16_f32 computes exactly this for every FP32
// input (all 2^32 bit patterns compared on the device against the integer
// form above, denormals kept), in one instruction per two values.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
}

// ------------------------------------------------------------------ E4M3
// Non-negative finite value (or +inf) -> E4M3fn byte: round to nearest even,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_sat(float v) {
  // Both forms are computed and one is selected (no branch):
  // below 2^-6: subnormal grid of step 2^-9 (v*512 is exact), 0..8, where 8
  // is 2^-6 = byte 0x08;
  const uint32_t sub = (uint32_t)__builtin_rintf(__builtin_fminf(v, 0.015625f) * 512.0f);
  // normal: round the 23-bit mantissa to 3 bits (ties to even); a carry moves
  // into the exponent field, which is what rounding up to the next binade
  // means; then rebias 127 -> 7.
  const uint32_t u = __float_as_uint(v);
  const uint32_t nrm = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  return !(v < 448.0f) ? 0x7Eu : (v < 0.015625f ? sub : nrm);
}

// E4M3fn byte (sign ignored; never 0x7F here) -> exact float.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const float sub = (float)(b & 7u) * 0.001953125f;                 // m * 2^-9
  const float nrm = __uint_as_float(((b & 0x7Fu) << 20) + (120u << 23));  // exponent e + 120, mantissa m
  return ((b >> 3) & 0xFu) == 0 ? sub : nrm;
}

// ------------------------------------------------------------------ E2M1
// float -> nibble: round to nearest, ties to the even code, saturate at 6;
// bit 3 copies the IEEE sign (a negative value rounding to 0 gives 0x8).
// The code is the number of midpoints passed: 0.25 1.25 2.5 5 (ties stay)
// and 0.75 1.75 3.5 (ties go up).
__device__ __forceinline__ uint32_t e2m1_encode(float q) {
  float a = __builtin_fabsf(q);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(q) >> 28) & 8u);
}

// ------------------------------------------------------------------ block quantizer
// One 16-element block given the row scale g (per-token scale or expert alpha):
//   sf = E4M3_sat(fp32(fp32(amax_b / 6) / g)),  e = fp32(dec(sf) * g),
//   q_i = E2M1(fp32(x_i / e)) if e > 0 else 0.
// Returns the scale byte; codes go to lo (elements 0..7) and hi (8..15),
// element 2i in the low nibble of byte i.
// The E2M1 code of every q = fp32(x / e) of a block, packed low nibble first.
// Fast form: q is approximated by y = fp32(x * fp32(1 / e)), which is within
// 3 ulp of q, and encoded by the hardware FP32 -> E2M1 conversion (scale 1.0:
// round to nearest, ties to the even code, saturating at 6, sign from the
// IEEE sign; checked against e2m1_encode over every non-NaN FP32 input). Every
// code boundary (0.25, 0.75, ..., 5) has at most 3 significant bits, so y can
// round differently from q only when its low 21 mantissa bits sit within 4 of
// such a value; then the block takes the exact division, as it does when
// 1 / e overflows.
__device__ __forceinline__ uint32_t e2m1_pack4(float a, float b, float c, float d) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c, d, 1.0f, 1);
}
// The low 21 bits of y + 4 moved to the top: y is near a code boundary when
// this is at most kNearCode (the minimum over a block decides for the block).
__device__ __forceinline__ uint32_t code_boundary_gap(float y) {
  return (__float_as_uint(y) << 11) + (4u << 11);
}
constexpr uint32_t kNearCode = 8u << 11;
// The block scale byte from the block amax a:
//   sf = E4M3_sat(fp32(fp32(a / 6) / g)).
// c6g = recip6(g) = fp32(1 / fp32(6 g)), taken once per row or tensor. Then
// z = fp32(a * c6g) is within 5 ulp of the two-division value, and the E4M3
// rounding of a value only changes at points whose low 19 mantissa bits are
// zero (the midpoints of the normal range, the half steps of the subnormal
// grid), so unless z lies within 16 ulp of such a point (bit patterns
// checked, zero, inf and NaN included) it encodes to the same byte; otherwise
// the two divisions are taken. c6g = 0 (g outside [2^-100, 2^100], where
// 6 g or its reciprocal could lose precision) always takes the divisions.
__device__ __forceinline__ float recip6(float g) {
  return (g >= 0x1p-100f && g <= 0x1p100f) ? 1.0f / (6.0f * g) : 0.0f;
}
__device__ __forceinline__ uint32_t block_scale_byte(float a, float g, float c6g) {
  const float z = a * c6g;
  if (((__float_as_uint(z) << 13) + (16u << 13)) <= (32u << 13)) return e4m3_encode_sat(a / 6.0f / g);
  return e4m3_encode_sat(z);
}

__device__ __forceinline__ uint32_t quant_block16(const float (&x)[16], float g, float c6g,
                                                  uint32_t& lo, uint32_t& hi) {
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(x[i]));
  uint32_t sf = 0;
  float e = 0.0f;
  if (g > 0.0f) {
    sf = block_scale_byte(amax_b, g, c6g);
    e = e4m3_decode(sf) * g;
  }
  lo = 0;
  hi = 0;
  if (e > 0.0f) {
    const float r = 1.0f / e;
    float y[16];
    uint32_t gap = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      y[i] = x[i] * r;
      gap = min(gap, code_boundary_gap(y[i]));
    }
    if (gap <= kNearCode || !(r <= 3.4e38f)) {  // or 1 / e overflowed
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = x[i] / e;
    }
    lo = e2m1_pack4(y[0], y[1], y[2], y[3]) |
         (e2m1_pack4(y[4], y[5], y[6], y[7]) << 16);
    hi = e2m1_pack4(y[8], y[9], y[10], y[11]) |
         (e2m1_pack4(y[12], y[13], y[14], y[15]) << 16);
  }
  return sf;
}

// ------------------------------------------------------------------ exact decode to FP16
// Every E2M1 x E4M3 product has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in FP16 (normal range), and FP16 x FP16
// products are exact in the FP32 MFMA accumulator. This is the decode-then-
// accumulate order of the pages [FlashInfer #5019 . Tensor and numerical
// contract, 'Compute order'], with FP16 as the exact carrier.
//
// The gfx950 FP4 -> FP16 convert applies only the exponent of its FP32 scale
// operand, so it runs with scale 1.0 and the E4M3 block scale is applied by a
// packed FP16 multiply (exact, see above).

// Four E4M3 bytes (byte j = scale of block j) -> FP16, as two packed pairs.
__device__ __forceinline__ void decode_scales4(uint32_t s, half2_t& s01, half2_t& s23) {
  s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
  s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true);
}

// Eight E2M1 codes (low nibble first) times an FP32 block scale, as BF16. The
// codes convert exactly to FP32, the product with an E4M3 scale has at most 6
// significant bits and is exact in FP32, and its low 16 bits are zero, so
// keeping the high half is the exact BF16 value (gfx950 has no packed BF16
// multiply).
__device__ __forceinline__ uint32_t bf16_pair_exact(float2v_t f, float sc) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, f[0] * sc);
  const uint32_t hi = __builtin_bit_cast(uint32_t, f[1] * sc);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // {hi[31:16], lo[31:16]}
}
__device__ __forceinline__ bf16x8_t decode8_bf16(uint32_t w, float sc) {
  const uint32_t p[4] = {
      bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), sc),
      bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), sc),
      bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), sc),
      bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), sc)};
  bf16x8_t r;
  __builtin_memcpy(&r, p, 16);
  return r;
}

// One dword of 8 E2M1 codes (element i in nibble i) times the block scale
// `sc` -> 8 FP16 values in element order.
__device__ __forceinline__ half8_t decode8(uint32_t w, _Float16 sc) {
  const half2_t s2 = {sc, sc};
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ------------------------------------------------------------------ barriers
// Workgroup barrier for hand-offs through LDS only: the fences order this
// wave's LDS accesses around the barrier (it waits for its own LDS operations,
// not for global loads still in flight), so prefetches issued before the
// barrier keep flying. __syncthreads() would also drain every global load.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace pmoe
