// Weight preparation: BF16 expert stacks -> NVFP4 in the prepared layout
// [Megatron-LM #8262 . What is added, 'prepare_routed_nvfp4_weights'].
//
// Three kernels per FC matrix:
//   1. amax partials: each workgroup reduces max|w| over a 64K-element span of
//      one expert (exact and order-free, so the result is deterministic);
//   2. fold: one workgroup per expert folds its partials into amax and
//      writes the expert's alpha;
//   3. quantize: each workgroup owns eight 64-element chunks of one 32-row
//      column block of one expert, read row by row in contiguous pieces
//      (column blocks past N, which pad the last 8-block column tile, are
//      written as zeros); it derives
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

// grid E: folds each expert's partial maxima into its amax, stored in place
// of its first partial, and writes the expert's alpha.
__global__ __launch_bounds__(256) void weight_amax_fold_kernel(float* __restrict__ partials, int parts,
                                                               const float* __restrict__ fold_a,
                                                               float* __restrict__ alpha_out) {
  const int e = blockIdx.x;
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += 256) m = __builtin_fmaxf(m, partials[(long)e * parts + i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    const float w_scale = 2688.0f / amax;  // +inf for an all-zero expert
    partials[(long)e * parts] = amax;
    alpha_out[e] = fold_a ? 1.0f / (w_scale * *fold_a) : 1.0f / w_scale;
  }
}

// grid (NBp * KR, E): NBp = NB rounded up to a multiple of 8, KR = KC / 8
// rounded up. Workgroup (p, kr) quantizes chunks 8*kr .. 8*kr + 7 of column
// block p. gated_I > 0 selects the gate/up interleave of a gated FC1. KC
// chunks of 64 cover Kd (a multiple of 16) rounded up; blocks past Kd, rows
// past N (past I in each half of a gated FC1) and whole padding column
// blocks are written as zeros.
constexpr int kRoundChunks = 8;  // chunks of a column block per workgroup

__global__ __launch_bounds__(256) void weight_quant_kernel(
    const uint16_t* __restrict__ w, int N, int Kd, int gated_I, int NB, int NBp, int KC,
    const float* __restrict__ amax_of, int parts, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int KR = (KC + kRoundChunks - 1) / kRoundChunks;
  const int p = blockIdx.x / KR, c0 = (blockIdx.x - p * KR) * kRoundChunks, e = blockIdx.y;
  const float amax = amax_of[(long)e * parts];
  const float w_scale = 2688.0f / amax;  // +inf for an all-zero expert
  const float alpha = 1.0f / w_scale;    // then 0
  const float c6g = recip6(alpha);

  // Chunk c of column block p is one 1 KB code slab (+ 128 B of scales) at
  // slab ((e*NT + p/8)*KC + c)*8 + p%8. The eight threads of row t/8 of the
  // column block take its 32 16-element blocks in turn: thread t quantizes
  // blocks t%8, t%8 + 8, t%8 + 16 and t%8 + 24 (block j = t%4 of chunks
  // c0 + t%8/4, c0 + 2 + t%8/4, ...), so each pair of 16-byte loads of a
  // wave covers eight rows x 256 contiguous bytes. The codes and scales go
  // into LDS in slab order, then the eight slabs are copied out with 16-byte
  // stores (the prepared layout spreads a block's codes over lanes, so
  // storing them directly would write each line several times over).
  __shared__ uint32_t lcodes[kRoundChunks][256];  // [chunk][lane * 4 + word]
  __shared__ uint8_t lscales[kRoundChunks][128];  // [chunk][scale dword * 4 + byte]
  const long tile_base = ((long)e * (NBp / kColTileBlocks) + p / kColTileBlocks) * KC;
  const int pos = p % kColTileBlocks;
  const int tid = threadIdx.x;
  const int col = tid >> 3;  // row of the column block (0..31)
  const int q = tid & 7;     // first block of this thread
  int n;                     // canonical row
  bool row_ok;
  if (gated_I > 0) {
    const int r = kColBlock * (p >> 1) + col;  // row within the gate or the up half
    n = ((p & 1) ? gated_I : 0) + r;
    row_ok = p < NB && r < gated_I;
  } else {
    n = kColBlock * p + col;
    row_ok = p < NB && n < N;
  }
  // The expert's rows as one buffer: reads of blocks past Kd or of rows that
  // do not exist get an offset past its end and return zeros, which quantize
  // to zero codes and a zero scale.
  const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + (long)e * N * Kd), (short)0, (int)((long)N * Kd * 2), 0x00020000);
  const uint32_t row_off = row_ok ? (uint32_t)n * (uint32_t)Kd * 2u : 0x80000000u;
  uint4 u[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = c0 * kChunk + kBlock * (8 * i + q);
    const uint32_t off = k < Kd ? row_off + (uint32_t)k * 2u : 0x80000000u;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src, off + 16 * hf, 0, 0);
      u[i][hf] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // all eight loads in flight before the first use
  // Block j of a chunk is half jj = j%2 of k-step s = j/2; its row sits in
  // 16-column block h of the position. Lane 32*jj + col%16 holds elements
  // 0..7, lane + 16 elements 8..15, each as word 2h + s of its 16 bytes; the
  // scale is byte 2h + s of dword col%16 + 16*jj.
  const int h = col >> 4, n16 = col & 15, j = q & 3, jj = j & 1, s = j >> 1;
  const int word = (32 * jj + n16) * 4 + 2 * h + s;
  const int sbyte = (n16 + 16 * jj) * 4 + 2 * h + s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cl = 2 * i + (q >> 2);  // chunk of the workgroup
    const uint32_t v[8] = {u[i][0].x, u[i][0].y, u[i][0].z, u[i][0].w,
                           u[i][1].x, u[i][1].y, u[i][1].z, u[i][1].w};
    float x[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[2 * k] = bf16_to_f32(v[k] & 0xFFFFu);
      x[2 * k + 1] = bf16_to_f32(v[k] >> 16);
    }
    uint32_t lo, hi;
    const uint32_t sf = quant_block16(x, alpha, c6g, lo, hi);
    lcodes[cl][word] = lo;
    lcodes[cl][word + 64] = hi;  // lane + 16
    lscales[cl][sbyte] = (uint8_t)sf;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {  // codes: eight slabs of 64 lanes x 16 bytes
    const int t = tid + 256 * r, k = t >> 6, l = t & 63;
    if (c0 + k < KC) {
      const long slab = (tile_base + c0 + k) * kColTileBlocks + pos;
      reinterpret_cast<uint4*>(codes + slab * 1024)[l] = reinterpret_cast<const uint4*>(lcodes[k])[l];
    }
  }
  if (tid < 64) {  // scales: eight slabs of 8 x 16 bytes
    const int k = tid >> 3, t = tid & 7;
    if (c0 + k < KC) {
      const long slab = (tile_base + c0 + k) * kColTileBlocks + pos;
      reinterpret_cast<uint4*>(scales + slab * 128)[t] = reinterpret_cast<const uint4*>(lscales[k])[t];
    }
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
  weight_amax_fold_kernel<<<E, 256, 0, s>>>(partials, parts, fold_a, alpha);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int NB = col_blocks(N, gated_I), KC = padded_k(Kd) / kChunk;
  const int NBp = padded_col_blocks(NB), KR = (KC + kRoundChunks - 1) / kRoundChunks;
  weight_quant_kernel<<<dim3(NBp * KR, E), 256, 0, s>>>(w, N, Kd, gated_I, NB, NBp, KC, partials, parts,
                                                        codes, scales);
  return hipGetLastError();
}

}  // namespace pmoe
