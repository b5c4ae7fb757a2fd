// Per-row NVFP4 quantizers: the per-token activation quantizer (BF16 rows) and
// the requantizer of the FP32 expert intermediate (FP32 rows)
// [Megatron-LM #8262 . Background; What is added; How to extend].
//
// With a static scale a (per-tensor recipe [Megatron-LM #8262 . How to
// extend]) every row uses g = fp32(1 / a) instead of its own amax, read from
// device memory so that nothing waits on the host; no scale is written.
//
// One 256-thread workgroup per row, single pass: thread t owns 16-element
// blocks t, t+256, ... (at most kMaxBlocksPerThread), keeps them in registers,
// reduces the row's absolute maximum across the workgroup (max is exact and
// order-free), then quantizes its blocks. Loads and stores of a wave are
// contiguous spans. HBM bound: a BF16 row of H elements moves 2H bytes in and
// 9H/16 out; an FP32 row 4L in and 9L/16 out.
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

// Rows [begin, end): begin = *row_begin_dev (0 if null), end = *row_end_dev
// (rows if null), read at run time (the intermediate has a device-side count
// of valid routes). Workgroup b handles row begin + b.
// static_a: null for per-row scales, else the static scale a (kStatic).
template <bool kBf16, bool kStatic>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ x, int rows,
                                                            const int* __restrict__ row_begin_dev,
                                                            const int* __restrict__ row_end_dev,
                                                            int L, const float* __restrict__ static_a,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            float* __restrict__ scale) {
  __shared__ float red[4];
  const long row = blockIdx.x + (row_begin_dev ? *row_begin_dev : 0);
  const int nrows = row_end_dev ? *row_end_dev : rows;
  if (row >= nrows) return;
  const int tid = threadIdx.x;
  const int nblk = L / kBlock;
  const void* xr = kBf16 ? (const void*)(static_cast<const uint16_t*>(x) + row * L)
                         : (const void*)(static_cast<const float*>(x) + row * L);
  float v[kMaxBlocksPerThread][16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxBlocksPerThread; ++i) {
    const int b = tid + 256 * i;
    if (b < nblk) {
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
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    g = amax * kRecipeConst;
  }
  uint2* qr = reinterpret_cast<uint2*>(q + row * (L / 2));
  uint8_t* sr = sf + row * nblk;
#pragma unroll
  for (int i = 0; i < kMaxBlocksPerThread; ++i) {
    const int b = tid + 256 * i;
    if (b < nblk) {
      uint32_t lo, hi;
      const uint32_t s = quant_block16(v[i], g, lo, hi);
      qr[b] = make_uint2(lo, hi);
      sr[b] = (uint8_t)s;
    }
  }
  if constexpr (!kStatic) {
    if (tid == 0) scale[row] = g;
  }
}

hipError_t launch_quantize_bf16(const void* x, int T, int H, const float* static_a, uint8_t* xq,
                                uint8_t* x_sf, float* x_scale, hipStream_t s) {
  if (static_a)
    quantize_rows_kernel<true, true><<<T, 256, 0, s>>>(x, T, nullptr, nullptr, H, static_a, xq, x_sf,
                                                       nullptr);
  else
    quantize_rows_kernel<true, false><<<T, 256, 0, s>>>(x, T, nullptr, nullptr, H, nullptr, xq, x_sf,
                                                        x_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_f32(const float* h, int R, const int* row_begin_dev,
                               const int* row_end_dev, int L, const float* static_a, uint8_t* hq,
                               uint8_t* h_sf, float* h_scale, hipStream_t s) {
  if (static_a)
    quantize_rows_kernel<false, true><<<R, 256, 0, s>>>(h, R, row_begin_dev, row_end_dev, L, static_a,
                                                        hq, h_sf, nullptr);
  else
    quantize_rows_kernel<false, false><<<R, 256, 0, s>>>(h, R, row_begin_dev, row_end_dev, L, nullptr,
                                                         hq, h_sf, h_scale);
  return hipGetLastError();
}

}  // namespace pmoe
