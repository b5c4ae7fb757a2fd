// One row of the per-row NVFP4 quantizer: the per-token activation quantizer
// (BF16 rows) and the requantizer of the FP32 expert intermediate (FP32 rows)
// [Megatron-LM #8262 . Background; What is added; How to extend].
//
// The row's absolute maximum (exact and order-free), g = fp32(amax *
// fp32(1/2688)), then per 16-element block the exact steps of quant_block16:
// E4M3 block scale, E2M1 codes. With a static scale a (per-tensor recipe)
// every row uses g = fp32(1 / a) instead and no scale is written.
//
// Two bodies, the same bytes: quantize_row_group (256 threads per row, one
// pass from registers: more waves per row hide the load latency), used where
// the quantizer has the GPU to itself or shares it with the routing; and
// quantize_row_wave (one wave per row, two passes), used by a looping grid that
// starts few waves -- starting waves is what bounds a quantizer launched
// while another stream's grouped GEMM holds the CUs.
#pragma once

#include "device.h"
#include "kernels.h"

namespace pmoe {

template <bool kBf16>
__device__ __forceinline__ void load_block16(const void* row, int b, float (&x)[16]) {
  if constexpr (kBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + b * 16);
    uint4 u0 = p[0], u1 = p[1];
    uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + b * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v = p[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  }
}

// Output rows may be wider than the input: Lq >= L (both multiples of 16)
// elements per output row, so q rows are Lq/2 bytes and sf rows Lq/16; the
// blocks in [L, Lq) get zero codes and a zero scale, which is what the grouped
// GEMMs need where a reduction is padded up to whole 64-element chunks.

// Row `row` of x ([rows][L], BF16 or FP32) -> q [rows][Lq/2], sf [rows][Lq/16],
// scale [rows] (per-row recipe), by one whole wave (lane = 0..63; every lane
// of the wave calls it for the same row). Two passes over the row: lane l's
// blocks are l, l+64, ...; pass 1 reads them for the row amax (a wave
// reduction: no LDS, no barrier), pass 2 reads them again (from cache) and
// quantizes four blocks at a time.
template <bool kBf16, bool kStatic>
__device__ __forceinline__ void quantize_row_wave(const void* __restrict__ x, long row, int L,
                                                  int Lq, int lane, const float* __restrict__ static_a,
                                                  uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ sf,
                                                  float* __restrict__ scale) {
  const int nblk = L / kBlock;
  const void* xr = kBf16 ? (const void*)(static_cast<const uint16_t*>(x) + row * L)
                         : (const void*)(static_cast<const float*>(x) + row * L);
  constexpr int kGroup = 4;  // blocks in registers at once per lane
  float g;
  if constexpr (kStatic) {
    g = 1.0f / *static_a;  // IEEE division (correctly rounded)
  } else {
    float amax = 0.0f;
    for (int b0 = lane; b0 < nblk; b0 += 64 * kGroup) {
      float v[kGroup][16];
#pragma unroll
      for (int i = 0; i < kGroup; ++i)
        if (b0 + 64 * i < nblk) load_block16<kBf16>(xr, b0 + 64 * i, v[i]);
#pragma unroll
      for (int i = 0; i < kGroup; ++i)
        if (b0 + 64 * i < nblk) {
#pragma unroll
          for (int k = 0; k < 16; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i][k]));
        }
    }
    g = wave_max(amax) * kRecipeConst;
  }
  const float c6g = recip6(g);
  const int nblk_q = Lq / kBlock;
  uint2* qr = reinterpret_cast<uint2*>(q + row * (Lq / 2));
  uint8_t* sr = sf + row * nblk_q;
  for (int b0 = lane; b0 < nblk; b0 += 64 * kGroup) {
    float v[kGroup][16];
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      if (b0 + 64 * i < nblk) load_block16<kBf16>(xr, b0 + 64 * i, v[i]);
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int b = b0 + 64 * i;
      if (b < nblk) {
        uint32_t lo, hi;
        const uint32_t s = quant_block16(v[i], g, c6g, lo, hi);
        qr[b] = make_uint2(lo, hi);
        sr[b] = (uint8_t)s;
      }
    }
  }
  for (int b = nblk + lane; b < nblk_q; b += 64) {  // padding blocks
    qr[b] = make_uint2(0u, 0u);
    sr[b] = 0;
  }
  if constexpr (!kStatic) {
    if (lane == 0) scale[row] = g;
  }
}


// The same row with a group of 256 threads (lt = 0..255): thread lt owns
// blocks lt, lt+256, ... (at most 4, rows up to 16384), kept in registers for
// a single pass; the group's amax goes through `red` (4 floats of LDS owned by
// the group) and one workgroup barrier, so every thread of the workgroup makes
// the call, and a group with no row passes active = false.
template <bool kBf16, bool kStatic>
__device__ __forceinline__ void quantize_row_group(const void* __restrict__ x, long row,
                                                   bool active, int L, int Lq, int lt,
                                                   const float* __restrict__ static_a,
                                                   uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ sf,
                                                   float* __restrict__ scale, float* red) {
  constexpr int kPer = kMaxRow / 16 / 256;
  const int nblk = L / kBlock;
  const void* xr = kBf16 ? (const void*)(static_cast<const uint16_t*>(x) + row * L)
                         : (const void*)(static_cast<const float*>(x) + row * L);
  float v[kPer][16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = lt + 256 * i;
    if (active && b < nblk) {
      load_block16<kBf16>(xr, b, v[i]);
      if constexpr (!kStatic) {
#pragma unroll
        for (int k = 0; k < 16; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i][k]));
      }
    }
  }
  float g;
  if constexpr (kStatic) {
    g = 1.0f / *static_a;
  } else {
    amax = wave_max(amax);
    if ((lt & 63) == 0) red[lt >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    g = amax * kRecipeConst;
  }
  if (!active) return;
  const float c6g = recip6(g);
  const int nblk_q = Lq / kBlock;
  uint2* qr = reinterpret_cast<uint2*>(q + row * (Lq / 2));
  uint8_t* sr = sf + row * nblk_q;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = lt + 256 * i;
    if (b < nblk) {
      uint32_t lo, hi;
      const uint32_t s = quant_block16(v[i], g, c6g, lo, hi);
      qr[b] = make_uint2(lo, hi);
      sr[b] = (uint8_t)s;
    } else if (b < nblk_q) {  // padding block
      qr[b] = make_uint2(0u, 0u);
      sr[b] = 0;
    }
  }
  if constexpr (!kStatic) {
    if (lt == 0) scale[row] = g;
  }
}

}  // namespace pmoe
