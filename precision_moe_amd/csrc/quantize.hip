// Per-row NVFP4 quantizers: the per-token activation quantizer (BF16 rows) and
// the requantizer of the FP32 expert intermediate (FP32 rows)
// [Megatron-LM #8262 . Background; What is added; How to extend].
//
// With a static scale a (per-tensor recipe [Megatron-LM #8262 . How to
// extend]) every row uses g = fp32(1 / a) instead of its own amax, read from
// device memory so that nothing waits on the host; no scale is written.
//
// Two kernels with the same bytes. quantize_rows_kernel gives each row a
// workgroup of 256 threads (quantize_row_group: one pass from registers),
// the faster layout when the quantizer has the GPU to itself.
// quantize_rows_loop_kernel gives each row one wave (quantize_row_wave) and
// loops a bounded grid over the rows: it starts a few thousand waves instead
// of four per row, which is what it costs while the other stream's grouped
// GEMM holds the CUs (the requant of one expert half inside the two-stream
// path).
// Loads and stores of a wave are contiguous spans. Algorithmic bytes: a BF16
// row of H elements moves 2H in and 9H/16 out; an FP32 row 4L in and 9L/16
// out.
#include "rowquant.h"

namespace pmoe {

// Rows [begin, end): begin = *row_begin_dev (0 if null), end = *row_end_dev
// (rows if null), read at run time (the intermediate has a device-side count
// of valid routes). static_a: null for per-row scales, else the static scale
// a (kStatic).
//
// Workgroup b handles row begin + b (the grid covers every row that can exist).
template <bool kBf16, bool kStatic>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ x, int rows,
                                                            const int* __restrict__ row_begin_dev,
                                                            const int* __restrict__ row_end_dev,
                                                            int L, int Lq,
                                                            const float* __restrict__ static_a,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            float* __restrict__ scale) {
  __shared__ float red[4];
  const long row = blockIdx.x + (row_begin_dev ? *row_begin_dev : 0);
  const int nrows = row_end_dev ? *row_end_dev : rows;
  if (row >= nrows) return;  // uniform across the workgroup
  quantize_row_group<kBf16, kStatic>(x, row, true, L, Lq, threadIdx.x, static_a, q, sf, scale, red);
}

// Wave w of workgroup b takes rows begin + 4b + w, then every 4 * gridDim.x
// rows after it.
template <bool kBf16, bool kStatic>
__global__ __launch_bounds__(256) void quantize_rows_loop_kernel(
    const void* __restrict__ x, int rows, const int* __restrict__ row_begin_dev,
    const int* __restrict__ row_end_dev, int L, int Lq, const float* __restrict__ static_a,
    uint8_t* __restrict__ q, uint8_t* __restrict__ sf, float* __restrict__ scale) {
  const long begin = row_begin_dev ? *row_begin_dev : 0;
  const long end = row_end_dev ? *row_end_dev : rows;
  const long step = (long)gridDim.x * 4;
  for (long row = begin + (long)blockIdx.x * 4 + (threadIdx.x >> 6); row < end; row += step)
    quantize_row_wave<kBf16, kStatic>(x, row, L, Lq, threadIdx.x & 63, static_a, q, sf, scale);
}

// At most kLoopGroups workgroups of four waves for the looping kernel.
constexpr int kLoopGroups = 512;
static int loop_grid(int rows) {
  const int g = (rows + 3) / 4;
  return g < 1 ? 1 : (g < kLoopGroups ? g : kLoopGroups);
}

hipError_t launch_quantize_bf16(const void* x, int T, int H, int Hq, const float* static_a,
                                uint8_t* xq, uint8_t* x_sf, float* x_scale, hipStream_t s) {
  if (static_a)
    quantize_rows_kernel<true, true><<<T, 256, 0, s>>>(x, T, nullptr, nullptr, H, Hq, static_a, xq,
                                                       x_sf, nullptr);
  else
    quantize_rows_kernel<true, false><<<T, 256, 0, s>>>(x, T, nullptr, nullptr, H, Hq, nullptr, xq,
                                                        x_sf, x_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_f32(const float* h, int R, const int* row_begin_dev,
                               const int* row_end_dev, int L, int Lq, const float* static_a,
                               uint8_t* hq, uint8_t* h_sf, float* h_scale, bool beside_gemm,
                               hipStream_t s) {
  if (beside_gemm) {
    if (static_a)
      quantize_rows_loop_kernel<false, true><<<loop_grid(R), 256, 0, s>>>(
          h, R, row_begin_dev, row_end_dev, L, Lq, static_a, hq, h_sf, nullptr);
    else
      quantize_rows_loop_kernel<false, false><<<loop_grid(R), 256, 0, s>>>(
          h, R, row_begin_dev, row_end_dev, L, Lq, nullptr, hq, h_sf, h_scale);
  } else if (static_a) {
    quantize_rows_kernel<false, true><<<R, 256, 0, s>>>(h, R, row_begin_dev, row_end_dev, L, Lq,
                                                        static_a, hq, h_sf, nullptr);
  } else {
    quantize_rows_kernel<false, false><<<R, 256, 0, s>>>(h, R, row_begin_dev, row_end_dev, L, Lq,
                                                         nullptr, hq, h_sf, h_scale);
  }
  return hipGetLastError();
}

// Copy rows of `row_bytes` bytes into rows of `dst_row_bytes` >= row_bytes, zero-filling
// the rest: a canonical operand whose reduction length is not a multiple of 64, laid
// out for the grouped GEMMs (whole 64-element chunks). kW bytes per thread and step;
// both row sizes are multiples of kW.
template <typename W>
__global__ __launch_bounds__(256) void pad_rows_kernel(const W* __restrict__ src, long rows,
                                                       int row_w, int dst_row_w,
                                                       W* __restrict__ dst) {
  const long n = rows * dst_row_w;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long r = i / dst_row_w;
    const int c = (int)(i - r * dst_row_w);
    W v;
    if (c < row_w)
      v = src[r * row_w + c];
    else
      __builtin_memset(&v, 0, sizeof(W));
    dst[i] = v;
  }
}

hipError_t launch_pad_rows(const void* src, long rows, long row_bytes, long dst_row_bytes, void* dst,
                           hipStream_t s) {
  const long n = rows * dst_row_bytes;
  long blocks = (n / 16 + 255) / 256;
  const int grid = (int)(blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks));
  if (row_bytes % 16 == 0 && dst_row_bytes % 16 == 0)
    pad_rows_kernel<uint4><<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), rows, (int)(row_bytes / 16),
                                                (int)(dst_row_bytes / 16), static_cast<uint4*>(dst));
  else if (row_bytes % 8 == 0 && dst_row_bytes % 8 == 0)
    pad_rows_kernel<uint2><<<grid, 256, 0, s>>>(static_cast<const uint2*>(src), rows, (int)(row_bytes / 8),
                                                (int)(dst_row_bytes / 8), static_cast<uint2*>(dst));
  else
    pad_rows_kernel<uint8_t><<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(src), rows, (int)row_bytes,
                                                  (int)dst_row_bytes, static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace pmoe
