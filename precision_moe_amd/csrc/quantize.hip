// Per-row NVFP4 quantizers: the per-token activation quantizer (BF16 rows) and
// the requantizer of the FP32 expert intermediate (FP32 rows)
// [Megatron-LM #8262 . Background; What is added; How to extend].
//
// One wave per row. Pass 1 reads the row once for its absolute maximum
// (wave-reduced; max is exact and order-free), pass 2 re-reads it (now in
// cache) and quantizes 16-element blocks, lane b handling blocks b, b+64, ...
// so every load and store of a wave is one contiguous span. HBM bound: a BF16
// row of H elements moves 2H bytes in and 9H/16 bytes out.
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

// rows: number of rows, or (if rows_dev != nullptr) read from *rows_dev at run
// time (the intermediate has a device-side count of valid routes).
template <bool kBf16>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ x, int rows,
                                                            const int* __restrict__ rows_dev,
                                                            int L, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nrows = rows_dev ? *rows_dev : rows;
  if (row >= nrows) return;
  const int nblk = L / kBlock;
  const void* xr = kBf16 ? (const void*)(static_cast<const uint16_t*>(x) + row * L)
                         : (const void*)(static_cast<const float*>(x) + row * L);
  float amax = 0.0f;
  for (int b = lane; b < nblk; b += 64) {
    float v[16];
    load_block16<kBf16>(xr, b, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  }
  amax = wave_max(amax);
  const float g = amax * kRecipeConst;
  uint2* qr = reinterpret_cast<uint2*>(q + row * (L / 2));
  uint8_t* sr = sf + row * nblk;
  for (int b = lane; b < nblk; b += 64) {
    float v[16];
    load_block16<kBf16>(xr, b, v);
    uint32_t lo, hi;
    uint32_t s = quant_block16(v, g, lo, hi);
    qr[b] = make_uint2(lo, hi);
    sr[b] = (uint8_t)s;
  }
  if (lane == 0) scale[row] = g;
}

hipError_t launch_quantize_bf16(const void* x, int T, int H, uint8_t* xq, uint8_t* x_sf,
                                float* x_scale, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  quantize_rows_kernel<true><<<grid, 256, 0, s>>>(x, T, nullptr, H, xq, x_sf, x_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_f32(const float* h, int R, const int* rows_dev, int L, uint8_t* hq,
                               uint8_t* h_sf, float* h_scale, hipStream_t s) {
  dim3 grid((R + 3) / 4);
  quantize_rows_kernel<false><<<grid, 256, 0, s>>>(h, R, rows_dev, L, hq, h_sf, h_scale);
  return hipGetLastError();
}

}  // namespace pmoe
