// One row of the per-row NVFP4 quantizer, done by a group of 256 threads:
// the per-token activation quantizer (BF16 rows) and the requantizer of the
// FP32 expert intermediate (FP32 rows) [Megatron-LM #8262 . Background; What
// is added; How to extend]. Shared by the standalone quantizer kernels and the
// launch that routes and quantizes the input together.
//
// Thread lt of the group owns 16-element blocks lt, lt+256, ... (at most
// kMaxBlocksPerThread), keeps them in registers, the group reduces the row's
// absolute maximum (max is exact and order-free), then each thread quantizes
// its blocks: g = fp32(amax * fp32(1/2688)), E4M3 block scales, E2M1 codes,
// with the exact steps of quant_block16. With a static scale a (per-tensor
// recipe) every row uses g = fp32(1 / a) instead and no scale is written.
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

// Row `row` of x ([rows][L], BF16 or FP32) -> q [rows][L/2], sf [rows][L/16],
// scale [rows] (per-row recipe). lt: the thread's index in its group of 256.
// red: 4 floats of LDS owned by this group. Without a static scale the call
// holds one workgroup barrier: every thread of the workgroup must make it the
// same number of times, so a group with no row passes active = false (it
// takes the barrier and touches no memory).
template <bool kBf16, bool kStatic>
__device__ __forceinline__ void quantize_row(const void* __restrict__ x, long row, bool active,
                                             int L, int lt, const float* __restrict__ static_a,
                                             uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                                             float* __restrict__ scale, float* red) {
  const int nblk = L / kBlock;
  const void* xr = kBf16 ? (const void*)(static_cast<const uint16_t*>(x) + row * L)
                         : (const void*)(static_cast<const float*>(x) + row * L);
  float v[kMaxBlocksPerThread][16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxBlocksPerThread; ++i) {
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
    g = 1.0f / *static_a;  // IEEE division (correctly rounded)
  } else {
    amax = wave_max(amax);
    if ((lt & 63) == 0) red[lt >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    g = amax * kRecipeConst;
  }
  if (!active) return;
  uint2* qr = reinterpret_cast<uint2*>(q + row * (L / 2));
  uint8_t* sr = sf + row * nblk;
#pragma unroll
  for (int i = 0; i < kMaxBlocksPerThread; ++i) {
    const int b = lt + 256 * i;
    if (b < nblk) {
      uint32_t lo, hi;
      const uint32_t s = quant_block16(v[i], g, lo, hi);
      qr[b] = make_uint2(lo, hi);
      sr[b] = (uint8_t)s;
    }
  }
  if constexpr (!kStatic) {
    if (lt == 0) scale[row] = g;
  }
}

}  // namespace pmoe
