// Weight preparation: BF16 expert stacks -> NVFP4 in the prepared layout
// [Megatron-LM #8262 . What is added, 'prepare_routed_nvfp4_weights'].
//
// Two kernels per FC matrix:
//   1. amax partials: each workgroup reduces max|w| over a 64K-element span of
//      one expert (exact and order-free, so the result is deterministic);
//   2. quantize: each workgroup owns one 32-row column block of one expert
//      (column blocks past N, which pad the last 8-block column tile, are
//      written as zeros),
//      folds its expert's partials into amax, derives
//        w_scale = fp32(2688 / amax), alpha = fp32(1 / w_scale)
//      and quantizes every 16-block of its rows with g = alpha, writing codes
//      and E4M3 scales straight into the prepared layout (see include/pmoe.h).
//      For the per-tensor recipe the stored alpha folds in the static input
//      scale a: alpha' = fp32(1 / fp32(w_scale * a)); codes and block scales do
//      not change [Megatron-LM #8262 . How to extend].
// Writing into caller buffers in place keeps their addresses fixed across a
// refresh (in-place refit).
#include "device.h"
#include "kernels.h"

namespace pmoe {

constexpr int kAmaxSpan = 256 * 256;  // elements reduced per workgroup in pass 1

int weight_amax_parts(long elems) { return (int)((elems + kAmaxSpan - 1) / kAmaxSpan); }

__global__ __launch_bounds__(256) void weight_amax_kernel(const uint16_t* __restrict__ w,
                                                          long per_expert, int parts,
                                                          float* __restrict__ partials) {
  const int e = blockIdx.y, part = blockIdx.x;
  const long begin = (long)part * kAmaxSpan;
  const long end = begin + kAmaxSpan < per_expert ? begin + kAmaxSpan : per_expert;
  const uint16_t* base = w + (long)e * per_expert;
  float m = 0.0f;
  for (long i = begin + threadIdx.x * 8; i < end; i += 256 * 8) {
    uint4 u = *reinterpret_cast<const uint4*>(base + i);  // per_expert is a multiple of 8
    uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_to_f32(v[k] & 0xFFFFu)));
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_to_f32(v[k] >> 16)));
    }
  }
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    partials[(long)e * parts + part] =
        __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

// grid (NBp, E) with NBp = NB rounded up to a multiple of 8. gated_I > 0
// selects the gate/up interleave of a gated FC1. KC chunks of 64 cover Kd
// (a multiple of 16) rounded up; blocks past Kd, rows past N (past I in each
// half of a gated FC1) and whole padding column blocks are written as zeros.
__global__ __launch_bounds__(256) void weight_quant_kernel(
    const uint16_t* __restrict__ w, int N, int Kd, int gated_I, int NB, int NBp, int KC,
    const float* __restrict__ partials, int parts, const float* __restrict__ fold_a,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ alpha_out) {
  const int p = blockIdx.x, e = blockIdx.y;
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += 256) m = __builtin_fmaxf(m, partials[(long)e * parts + i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float w_scale = 2688.0f / amax;  // +inf for an all-zero expert
  const float alpha = 1.0f / w_scale;    // then 0
  if (p == 0 && threadIdx.x == 0) alpha_out[e] = fold_a ? 1.0f / (w_scale * *fold_a) : alpha;

  // Chunk c of column block p is one 1 KB code slab (+ 128 B of scales) at
  // slab ((e*NT + p/8)*KC + c)*8 + p%8. Two chunks per round: thread t
  // quantizes, of row t/8 of the column block, block (t%8)%4 of chunk
  // c0 + (t%8)/4; the codes and scales go into LDS in slab order, then the
  // two slabs are copied out with 16-byte stores (the prepared layout spreads
  // a block's codes over lanes, so storing them directly would write each
  // line several times over).
  __shared__ uint32_t lcodes[2][256];
  __shared__ uint32_t lscales[2][32];
  const long tile_base = ((long)e * (NBp / kColTileBlocks) + p / kColTileBlocks) * KC;
  const int pos = p % kColTileBlocks;
  const int tid = threadIdx.x;
  const int col = tid >> 3;  // row of the column block (0..31)
  const int bl = tid & 7;    // block of the round: chunk bl/4, block bl%4 of that chunk
  int n;                     // canonical row (only read when row_ok)
  bool row_ok;
  if (gated_I > 0) {
    const int r = kColBlock * (p >> 1) + col;  // row within the gate or the up half
    n = ((p & 1) ? gated_I : 0) + r;
    row_ok = p < NB && r < gated_I;
  } else {
    n = kColBlock * p + col;
    row_ok = p < NB && n < N;
  }
  const int cs = bl >> 2, j = bl & 3;
  // block j of a chunk is half jj of k-step s; its row sits in 16-column
  // block h of the position. Lane 32*jj + col%16 holds elements 0..7, lane
  // + 16 elements 8..15, each as word 2h + s of its 16 bytes; the scale is
  // byte 2h + s of dword col%16 + 16*jj.
  const int s = j >> 1, jj = j & 1, h = col >> 4, n16 = col & 15;
  const int lane_lo = 32 * jj + n16;
  for (int c0 = 0; c0 < KC; c0 += 2) {
    const int c = c0 + cs;
    uint32_t lo = 0, hi = 0, sf = 0;
    if (row_ok && c < KC && (4 * c + j) * kBlock < Kd) {
      const uint4* src =
          reinterpret_cast<const uint4*>(w + ((long)e * N + n) * Kd + (4 * c + j) * kBlock);
      uint4 u0 = src[0], u1 = src[1];
      uint32_t v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      float x[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_to_f32(v[i] >> 16);
      }
      sf = quant_block16(x, alpha, lo, hi);
    }
    lcodes[cs][lane_lo * 4 + 2 * h + s] = lo;
    lcodes[cs][(lane_lo + 16) * 4 + 2 * h + s] = hi;
    reinterpret_cast<uint8_t*>(lscales[cs])[(n16 + 16 * jj) * 4 + 2 * h + s] = (uint8_t)sf;
    __syncthreads();
    if (tid < 128) {  // codes: two slabs of 64 lanes x 16 bytes
      const int k = tid >> 6, l = tid & 63;
      if (c0 + k < KC) {
        const long slab = (tile_base + c0 + k) * kColTileBlocks + pos;
        reinterpret_cast<uint4*>(codes + slab * 1024)[l] = reinterpret_cast<const uint4*>(lcodes[k])[l];
      }
    } else if (tid < 144) {  // scales: two slabs of 8 x 16 bytes
      const int k = (tid - 128) >> 3, q = (tid - 128) & 7;
      if (c0 + k < KC) {
        const long slab = (tile_base + c0 + k) * kColTileBlocks + pos;
        reinterpret_cast<uint4*>(scales + slab * 128)[q] = reinterpret_cast<const uint4*>(lscales[k])[q];
      }
    }
    __syncthreads();
  }
}

hipError_t launch_prepare_fc(const uint16_t* w, int E, int N, int Kd, int gated_I, float* partials,
                             const float* fold_a, uint8_t* codes, uint8_t* scales, float* alpha,
                             hipStream_t s) {
  const long per_expert = (long)N * Kd;
  const int parts = weight_amax_parts(per_expert);
  weight_amax_kernel<<<dim3(parts, E), 256, 0, s>>>(w, per_expert, parts, partials);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int NB = col_blocks(N, gated_I), KC = padded_k(Kd) / kChunk;
  const int NBp = padded_col_blocks(NB);
  weight_quant_kernel<<<dim3(NBp, E), 256, 0, s>>>(w, N, Kd, gated_I, NB, NBp, KC, partials, parts,
                                                   fold_a, codes, scales, alpha);
  return hipGetLastError();
}

}  // namespace pmoe
