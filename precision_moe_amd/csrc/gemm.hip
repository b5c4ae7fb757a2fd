// Expert-sorted grouped GEMMs of the routed-MoE path (FC1 with the fused
// activation, FC2 with the fused per-row / per-expert scaling and BF16 output)
// [Megatron-LM #8262 . Background; FlashInfer #5019 . Tensor and numerical
// contract, 'Compute order'].
//
// Work unit: one M-tile (32 expert-sorted rows of one expert, from the device
// tile list) x one column tile (8 prepared column blocks = 256 weight rows).
// A workgroup is 4 waves; wave w owns column blocks 2w and 2w+1 of the tile.
//
// Per 64-element reduction chunk:
//   * A (activations, NVFP4 rows gathered by route for FC1, contiguous for FC2):
//     256 threads each load one dword of codes + its scale byte, decode 8 values
//     exactly to FP16 and store them into a double-buffered LDS tile
//     [32 rows][64 k] (row stride 144 B: conflict-free 16-byte reads/writes).
//   * B (weights, prepared layout): each wave loads one 16-byte span per lane
//     and column block -- a contiguous 1 KB per wave-load -- plus one dword of
//     four E4M3 scales, prefetched two chunks ahead in registers, and decodes
//     them in registers directly into MFMA operand order.
//   * 4 x v_mfma_f32_32x32x16_f16 per column block, FP32 accumulation; the
//     MFMA's k-step of 16 is exactly one NVFP4 block.
// Epilogue: y = acc * fp32(g_row * alpha_e) (the scales are applied after
// accumulation, never folded into the decoded values), then
//   FC1 squared ReLU: h = max(y, 0)^2;  FC1 SwiGLU: h = silu(gate) * up (the
//   gate and up blocks of one output sit in the same wave);  FC2: bf16(y).
//
// Batch invariance: every output element is one chain of MFMAs over k in
// fixed order, whatever T, the tile, or the other rows are; no split-K.
// Block->tile order: consecutive logical ids share an XCD (blockIdx % 8 picks
// the XCD), and the M-tiles of one expert are adjacent, so the weight stream of
// a hot expert is fetched once into that XCD's L2.
#include "device.h"
#include "kernels.h"

namespace pmoe {

constexpr int kWaves = 4;
constexpr int kBlocksPerWave = 2;
constexpr int kColTile = kWaves * kBlocksPerWave;  // column blocks per workgroup
constexpr int kLdsRow = 144;                       // bytes per LDS A row (128 + 16 pad)

__host__ __device__ int fc_col_tiles(int NB) { return (NB + kColTile - 1) / kColTile; }

__device__ __forceinline__ _Float16 e4m3_to_half(uint32_t b) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false)[0];
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void fc_kernel(FcParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kTileM * kLdsRow];
  __shared__ int a_row[kTileM];
  __shared__ float s_row[kTileM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int NT = fc_col_tiles(P.NB);
  const int nt = logical / P.max_tiles;
  const int tile = logical - nt * P.max_tiles;
  if (nt >= NT || tile >= P.counters[1]) return;
  const int e = P.tiles[2 * tile];
  const int row0 = P.expert_offsets[e] + P.tiles[2 * tile + 1];
  const int mrows = min(kTileM, P.expert_offsets[e + 1] - row0);
  const int NB = P.NB, KC = P.KC;

  if (tid < kTileM) {
    const int r = row0 + min(tid, mrows - 1);  // rows past the tile end repeat a valid row
    const int ar = P.route_of_row ? P.route_of_row[r] / P.topk : r;
    a_row[tid] = ar;
    s_row[tid] = P.a_scale[ar] * P.w_alpha[e];
  }
  __syncthreads();

  // A loader: thread -> (row am, 8-element piece ad) of each chunk.
  const int am = tid >> 3, ad = tid & 7;
  const uint8_t* a_code = P.a_codes + (long)a_row[am] * (KC * 32) + ad * 4;
  const uint8_t* a_scl = P.a_sf + (long)a_row[am] * (KC * 4) + (ad >> 1);
  uint8_t* a_dst0 = &a_lds[0][am * kLdsRow + ad * 16];
  uint8_t* a_dst1 = &a_lds[1][am * kLdsRow + ad * 16];
  // A fragment reads: lane -> row lane%32, k-offset 16*j + 8*(lane/32).
  const int frag_off = (lane & 31) * kLdsRow + (lane >> 5) * 16;

  // B streams of this wave's two column blocks (clamped in range when unused).
  const int p0 = nt * kColTile + wave * kBlocksPerWave;
  const bool use0 = p0 < NB, use1 = p0 + 1 < NB;
  const int q0 = min(p0, NB - 1), q1 = min(p0 + 1, NB - 1);
  const uint4* bq0 = reinterpret_cast<const uint4*>(P.w_codes + ((long)e * NB + q0) * KC * 1024) + lane;
  const uint4* bq1 = reinterpret_cast<const uint4*>(P.w_codes + ((long)e * NB + q1) * KC * 1024) + lane;
  const uint32_t* bs0 = reinterpret_cast<const uint32_t*>(P.w_scales + ((long)e * NB + q0) * KC * 128) + (lane & 31);
  const uint32_t* bs1 = reinterpret_cast<const uint32_t*>(P.w_scales + ((long)e * NB + q1) * KC * 128) + (lane & 31);

  floatx16 acc0 = {}, acc1 = {};

  // prologue: A chunk 0 into LDS, B chunks 0 and 1 into registers
  uint4 b0q[2], b1q[2];
  uint32_t b0s[2], b1s[2];
  b0q[0] = bq0[0];
  b1q[0] = bq1[0];
  b0s[0] = bs0[0];
  b1s[0] = bs1[0];
  if (KC > 1) {
    b0q[1] = bq0[64];
    b1q[1] = bq1[64];
    b0s[1] = bs0[32];
    b1s[1] = bs1[32];
  }
  {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(a_code);
    *reinterpret_cast<half8_t*>(a_dst0) = decode8(w, e4m3_to_half(a_scl[0]));
  }
  __syncthreads();

  // One chunk: consume the B registers of this slot, refill them two chunks
  // ahead, decode the next A chunk into the other LDS buffer.
  auto step = [&](const int c, uint4& q0r, uint4& q1r, uint32_t& s0r, uint32_t& s1r) {
    const bool more = c + 1 < KC;
    uint32_t aw = 0, as = 0;
    if (more) {
      aw = *reinterpret_cast<const uint32_t*>(a_code + (c + 1) * 32);
      as = a_scl[(c + 1) * 4];
    }
    const uint8_t* abuf = (c & 1) ? &a_lds[1][0] : &a_lds[0][0];
    half8_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const half8_t*>(abuf + frag_off + 32 * j);
    if (use0) {
      half2_t s01, s23;
      decode_scales4(s0r, s01, s23);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], decode8(q0r.x, s01[0]), acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[1], decode8(q0r.y, s01[1]), acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[2], decode8(q0r.z, s23[0]), acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[3], decode8(q0r.w, s23[1]), acc0, 0, 0, 0);
    }
    if (use1) {
      half2_t s01, s23;
      decode_scales4(s1r, s01, s23);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], decode8(q1r.x, s01[0]), acc1, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[1], decode8(q1r.y, s01[1]), acc1, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[2], decode8(q1r.z, s23[0]), acc1, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[3], decode8(q1r.w, s23[1]), acc1, 0, 0, 0);
    }
    if (c + 2 < KC) {
      q0r = bq0[(c + 2) * 64];
      q1r = bq1[(c + 2) * 64];
      s0r = bs0[(c + 2) * 32];
      s1r = bs1[(c + 2) * 32];
    }
    if (more) {
      uint8_t* dst = ((c + 1) & 1) ? a_dst1 : a_dst0;
      *reinterpret_cast<half8_t*>(dst) = decode8(aw, e4m3_to_half(as));
    }
    __syncthreads();
  };

  for (int c = 0; c < KC; c += 2) {
    step(c, b0q[0], b1q[0], b0s[0], b1s[0]);
    if (c + 1 < KC) step(c + 1, b0q[1], b1q[1], b0s[1], b1s[1]);
  }

  // ------------------------------------------------------------------ epilogue
  const int n = lane & 31;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (m >= mrows) continue;
    const float s = s_row[m];
    const long orow = (long)(row0 + m) * P.out_stride;
    if constexpr (MODE == kFc1Relu2) {
      float* out = static_cast<float*>(P.out) + orow;
      if (use0) {
        const float y = __builtin_fmaxf(acc0[r] * s, 0.0f);
        out[kColBlock * p0 + n] = y * y;
      }
      if (use1) {
        const float y = __builtin_fmaxf(acc1[r] * s, 0.0f);
        out[kColBlock * (p0 + 1) + n] = y * y;
      }
    } else if constexpr (MODE == kFc1Swiglu) {
      // p0 is even: block p0 holds gate rows, p0 + 1 the matching up rows.
      if (use0) {
        const float g = acc0[r] * s;
        const float u = acc1[r] * s;
        const float silu = g / (1.0f + expf(-g));
        float* out = static_cast<float*>(P.out) + orow;
        out[kColBlock * (p0 >> 1) + n] = silu * u;
      }
    } else {
      uint16_t* out = static_cast<uint16_t*>(P.out) + orow;
      if (use0) out[kColBlock * p0 + n] = (uint16_t)f32_to_bf16(acc0[r] * s);
      if (use1) out[kColBlock * (p0 + 1) + n] = (uint16_t)f32_to_bf16(acc1[r] * s);
    }
  }
}

hipError_t launch_fc(FcMode mode, const FcParams& p, hipStream_t s) {
  const long blocks = (long)p.max_tiles * fc_col_tiles(p.NB);
  const long grid = (blocks + 7) / 8 * 8;
  switch (mode) {
    case kFc1Relu2: fc_kernel<kFc1Relu2><<<grid, 256, 0, s>>>(p); break;
    case kFc1Swiglu: fc_kernel<kFc1Swiglu><<<grid, 256, 0, s>>>(p); break;
    case kFc2: fc_kernel<kFc2><<<grid, 256, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace pmoe
