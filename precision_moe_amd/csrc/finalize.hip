// Deterministic two-stage finalize: each token's top-k routes are reduced in a
// fixed order (slot order j = 0..K-1), after FC2 has written one BF16 row per
// route [Megatron-LM #8262 . Background, 'deterministic two-stage finalize';
// What is added]. Routing weights are FP32 and applied here, after FC2; every
// product and sum is rounded to FP32 separately (the library is built without
// FP contraction) and the sum is rounded to BF16 once [FlashInfer #5019 .
// Tensor and numerical contract, 'Compute order'].
//
// grid (ceil(H / 2048), T): each thread owns 8 consecutive columns of one
// token, so a workgroup reads K contiguous 4 KB spans of z and writes one. The
// route rows and weights of the token are uniform across the workgroup.
#include "device.h"
#include "kernels.h"

namespace pmoe {

__global__ __launch_bounds__(256) void finalize_kernel(const uint16_t* __restrict__ z,
                                                       const int* __restrict__ row_of_route,
                                                       const float* __restrict__ w, int K, int H,
                                                       uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int col = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (col >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int j = 0; j < K; ++j) {
    const int r = row_of_route[(long)t * K + j];
    if (r < 0) continue;
    const float wt = w[(long)t * K + j];
    const uint4 u = *reinterpret_cast<const uint4*>(z + (long)r * H + col);
    const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = acc[2 * i] + wt * bf16_to_f32(v[i] & 0xFFFFu);
      acc[2 * i + 1] = acc[2 * i + 1] + wt * bf16_to_f32(v[i] >> 16);
    }
  }
  uint4 o;
  o.x = f32x2_to_bf16x2(acc[0], acc[1]);
  o.y = f32x2_to_bf16x2(acc[2], acc[3]);
  o.z = f32x2_to_bf16x2(acc[4], acc[5]);
  o.w = f32x2_to_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + (long)t * H + col) = o;
}

hipError_t launch_finalize(const uint16_t* z, const int* row_of_route, const float* w, int T,
                           int K, int H, uint16_t* out, hipStream_t s) {
  dim3 grid((H + 2047) / 2048, T);
  finalize_kernel<<<grid, 256, 0, s>>>(z, row_of_route, w, K, H, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused finalize
// The order-free finalize accumulates fp32(w * z) of every route with FP32
// atomic adds inside FC2 (the non-deterministic mode the two-stage finalize
// replaces); these two kernels clear the accumulator before FC2 and round it
// to BF16 after. A plain fill kernel rather than a memset keeps the sequence
// safe to capture in a graph. n is a multiple of 8 (H is a multiple of 16).
__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ p, long n4) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n4; i += (long)gridDim.x * 256)
    p[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4* __restrict__ in, long n8,
                                                          uint4* __restrict__ out) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    const float4 a = in[2 * i], b = in[2 * i + 1];
    uint4 o;
    o.x = f32x2_to_bf16x2(a.x, a.y);
    o.y = f32x2_to_bf16x2(a.z, a.w);
    o.z = f32x2_to_bf16x2(b.x, b.y);
    o.w = f32x2_to_bf16x2(b.z, b.w);
    out[i] = o;
  }
}

static int stream_grid(long items) {
  const long g = (items + 255) / 256;
  return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

hipError_t launch_fill_zero(float* p, long n, hipStream_t s) {
  fill_zero_kernel<<<stream_grid(n / 4), 256, 0, s>>>(reinterpret_cast<float4*>(p), n / 4);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, long n, uint16_t* out, hipStream_t s) {
  f32_to_bf16_kernel<<<stream_grid(n / 8), 256, 0, s>>>(reinterpret_cast<const float4*>(in), n / 8,
                                                        reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace pmoe
