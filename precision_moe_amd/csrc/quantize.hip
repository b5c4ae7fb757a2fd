// Per-row NVFP4 quantizers: the per-token activation quantizer (BF16 rows) and
// the requantizer of the FP32 expert intermediate (FP32 rows)
// [Megatron-LM #8262 . Background; What is added; How to extend].
//
// With a static scale a (per-tensor recipe [Megatron-LM #8262 . How to
// extend]) every row uses g = fp32(1 / a) instead of its own amax, read from
// device memory so that nothing waits on the host; no scale is written.
//
// One wave per row (the row body is quantize_row) and a bounded grid whose
// waves loop over the rows. Loads and stores of a wave are contiguous spans.
// Algorithmic bytes: a BF16 row of H elements moves 2H in and 9H/16 out; an
// FP32 row 4L in and 9L/16 out.
#include "rowquant.h"

namespace pmoe {

// Rows [begin, end): begin = *row_begin_dev (0 if null), end = *row_end_dev
// (rows if null), read at run time (the intermediate has a device-side count
// of valid routes). Wave w of workgroup b takes rows begin + 4b + w, then
// every 4 * gridDim.x rows after it.
// static_a: null for per-row scales, else the static scale a (kStatic).
template <bool kBf16, bool kStatic>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ x, int rows,
                                                            const int* __restrict__ row_begin_dev,
                                                            const int* __restrict__ row_end_dev,
                                                            int L, const float* __restrict__ static_a,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            float* __restrict__ scale) {
  const long begin = row_begin_dev ? *row_begin_dev : 0;
  const long end = row_end_dev ? *row_end_dev : rows;
  const long step = (long)gridDim.x * 4;
  for (long row = begin + (long)blockIdx.x * 4 + (threadIdx.x >> 6); row < end; row += step)
    quantize_row<kBf16, kStatic>(x, row, L, threadIdx.x & 63, static_a, q, sf, scale);
}

// Workgroups of four waves, one row per wave and pass, at most kQuantGroups
// of them (rows beyond take further passes).
constexpr int kQuantGroups = 512;
static int quant_grid(int rows) {
  const int g = (rows + 3) / 4;
  return g < 1 ? 1 : (g < kQuantGroups ? g : kQuantGroups);
}

hipError_t launch_quantize_bf16(const void* x, int T, int H, const float* static_a, uint8_t* xq,
                                uint8_t* x_sf, float* x_scale, hipStream_t s) {
  if (static_a)
    quantize_rows_kernel<true, true><<<quant_grid(T), 256, 0, s>>>(x, T, nullptr, nullptr, H,
                                                                   static_a, xq, x_sf, nullptr);
  else
    quantize_rows_kernel<true, false><<<quant_grid(T), 256, 0, s>>>(x, T, nullptr, nullptr, H,
                                                                    nullptr, xq, x_sf, x_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_f32(const float* h, int R, const int* row_begin_dev,
                               const int* row_end_dev, int L, const float* static_a, uint8_t* hq,
                               uint8_t* h_sf, float* h_scale, hipStream_t s) {
  if (static_a)
    quantize_rows_kernel<false, true><<<quant_grid(R), 256, 0, s>>>(h, R, row_begin_dev, row_end_dev,
                                                                    L, static_a, hq, h_sf, nullptr);
  else
    quantize_rows_kernel<false, false><<<quant_grid(R), 256, 0, s>>>(h, R, row_begin_dev, row_end_dev,
                                                                     L, nullptr, hq, h_sf, h_scale);
  return hipGetLastError();
}

}  // namespace pmoe
