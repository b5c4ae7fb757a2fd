// Expert-sorted grouped GEMMs of the routed-MoE path (FC1 with the fused
// activation, FC2 with the fused per-row / per-expert scaling and BF16 output)
// [Megatron-LM #8262 . Background; FlashInfer #5019 . Tensor and numerical
// contract, 'Compute order'].
//
// Work unit: one M-tile (up to 64 expert-sorted rows of one expert, from the
// device tile list) x one column tile (8 prepared column blocks = 256 weight
// rows). A workgroup is 4 waves; wave w owns column blocks 2w and 2w+1 and all
// rows of the tile, as 2 x 2 accumulators of v_mfma_f32_32x32x16_f16. A tile
// with at most 32 rows skips the upper row block entirely.
//
// Reduction loop, in stages of 128 elements (two 64-element chunks):
//   * A (activations: NVFP4 rows gathered by route for FC1, contiguous for
//     FC2): each thread loads 16 bytes of codes + 2 scale bytes of one row,
//     decodes 32 values exactly to FP16 and writes them into a double-
//     buffered LDS stage [64 rows][128 k] (row stride 272 B).
//   * B (weights, prepared layout): per chunk and column block each lane loads
//     one 16-byte span (a contiguous 1 KB per wave-load) and one dword of four
//     E4M3 scales. Loads run four chunks ahead in registers; decoding happens
//     in registers straight into MFMA operand order, and every decoded B
//     fragment feeds both row blocks.
//   * The MFMA k-step of 16 is exactly one NVFP4 block; FP32 accumulation.
// Epilogue: y = acc * fp32(g_row * alpha_e) (scales applied after
// accumulation, never folded into decoded values), then
//   FC1 squared ReLU: h = max(y, 0)^2;  FC1 SwiGLU: h = silu(gate) * up (gate
//   and up column blocks of one output sit in the same wave);  FC2: bf16(y).
//
// Batch invariance: every output element is one chain of MFMAs over k in fixed
// order whatever T, the tile or the other rows are; no split-K.
// Block -> tile order: consecutive logical ids share an XCD (blockIdx % 8 picks
// the XCD) and the M-tiles of one expert are adjacent, so a hot expert's weight
// stream is fetched once into that XCD's L2 for all of its M-tiles.
#include "device.h"
#include "kernels.h"

namespace pmoe {

constexpr int kWaves = 4;
constexpr int kBlocksPerWave = 2;
constexpr int kColTile = kWaves * kBlocksPerWave;  // column blocks per workgroup
constexpr int kStageK = 128;                       // reduction elements per LDS stage
constexpr int kLdsRow = kStageK * 2 + 16;          // bytes per LDS A row (+16 pad)
constexpr int kRing = 4;                           // B register ring slots per wave
constexpr int kPrefetch = kRing - 1;               // B chunks in flight ahead of the one in use

__host__ __device__ int fc_col_tiles(int NB) { return (NB + kColTile - 1) / kColTile; }

__device__ __forceinline__ _Float16 e4m3_to_half(uint32_t b) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false)[0];
}

// 4 x 8 codes of one row (16 bytes) with the scales of the 2 blocks they span
// -> 32 FP16 values written to LDS as four 16-byte stores.
__device__ __forceinline__ void decode_a_store(const uint4& q, uint32_t s2, uint8_t* dst) {
  const _Float16 s0 = e4m3_to_half(s2 & 0xFFu), s1 = e4m3_to_half(s2 >> 8);
  *reinterpret_cast<half8_t*>(dst + 0) = decode8(q.x, s0);
  *reinterpret_cast<half8_t*>(dst + 16) = decode8(q.y, s0);
  *reinterpret_cast<half8_t*>(dst + 32) = decode8(q.z, s1);
  *reinterpret_cast<half8_t*>(dst + 48) = decode8(q.w, s1);
}

// Main loop + epilogue for one tile. TWO: the tile has more than 32 rows, so
// both row blocks are computed. Every global load inside the loop is
// unconditional (addresses past the end are clamped to the last chunk and the
// data is never used), which keeps the in-order load counters exact so the
// four-chunk B ring really stays in flight.
template <int MODE, bool TWO>
__device__ __forceinline__ void fc_tile(const FcParams& P, uint8_t (*a_lds)[kTileM * kLdsRow],
                                        const int* a_row, const float* s_row, int e, int row0,
                                        int mrows, int nt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NB = P.NB, KC = P.KC;

  // A loader: thread -> (row am, 32-element quarter aq) of each 128-element stage.
  const int am = tid >> 2, aq = tid & 3;
  const long a_row_bytes = (long)KC * 32;
  const uint8_t* a_code = P.a_codes + (long)a_row[am] * a_row_bytes;
  const uint8_t* a_scl = P.a_sf + (long)a_row[am] * (KC * 4);
  uint8_t* a_dst0 = &a_lds[0][am * kLdsRow + aq * 64];
  uint8_t* a_dst1 = &a_lds[1][am * kLdsRow + aq * 64];
  // Stage s of this thread covers chunk 2s + aq/2; past the last chunk (the
  // empty half of an odd final stage) it re-reads the last chunk instead.
  auto a_load = [&](int s, uint4& q, uint32_t& sc) {
    const int c = min(2 * s + (aq >> 1), KC - 1);
    const int part = aq & 1;
    q = *reinterpret_cast<const uint4*>(a_code + c * 32 + part * 16);
    sc = *reinterpret_cast<const uint16_t*>(a_scl + c * 4 + part * 2);
  };

  const int frag_off = (lane & 31) * kLdsRow + (lane >> 5) * 16;

  const int p0 = nt * kColTile + wave * kBlocksPerWave;
  const int q0 = min(p0, NB - 1), q1 = min(p0 + 1, NB - 1);
  const uint4* bq0 = reinterpret_cast<const uint4*>(P.w_codes + ((long)e * NB + q0) * KC * 1024) + lane;
  const uint4* bq1 = reinterpret_cast<const uint4*>(P.w_codes + ((long)e * NB + q1) * KC * 1024) + lane;
  const uint32_t* bs0 = reinterpret_cast<const uint32_t*>(P.w_scales + ((long)e * NB + q0) * KC * 128) + (lane & 31);
  const uint32_t* bs1 = reinterpret_cast<const uint32_t*>(P.w_scales + ((long)e * NB + q1) * KC * 128) + (lane & 31);

  floatx16 acc00 = {}, acc01 = {}, acc10 = {}, acc11 = {};  // [row block][col block]

  // B register ring: chunk c lives in slot c % kRing. Chunk c refills slot
  // (c + kPrefetch) % kRing -- the slot chunk c - 1 has just finished
  // decoding -- with chunk c + kPrefetch, so each slot keeps its registers
  // around the loop and kPrefetch chunks stay in flight.
  uint4 rq0[kRing], rq1[kRing];
  uint32_t rs0[kRing], rs1[kRing];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    const int c = min(i, KC - 1);
    rq0[i] = bq0[c * 64];
    rq1[i] = bq1[c * 64];
    rs0[i] = bs0[c * 32];
    rs1[i] = bs1[c * 32];
  }
  {
    uint4 q;
    uint32_t sc;
    a_load(0, q, sc);
    decode_a_store(q, sc, a_dst0);
  }
  __syncthreads();

  auto chunk = [&](const int c, const uint8_t* abuf, const int half, const int i) {
    // Refill the slot freed by chunk c - 1 before decoding slot i; the
    // scheduling barrier keeps these loads ahead of the decode.
    const int r = (i + kPrefetch) % kRing;
    const int cn = min(c + kPrefetch, KC - 1);
    rq0[r] = bq0[cn * 64];
    rq1[r] = bq1[cn * 64];
    rs0[r] = bs0[cn * 32];
    rs1[r] = bs1[cn * 32];
    __builtin_amdgcn_sched_barrier(0);
    const uint4 q0 = rq0[i], q1 = rq1[i];
    const uint32_t sc0 = rs0[i], sc1 = rs1[i];
    const uint8_t* ab = abuf + frag_off + half * 128;
    half8_t a0[4], a1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a0[j] = *reinterpret_cast<const half8_t*>(ab + 32 * j);
    if constexpr (TWO) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a1[j] = *reinterpret_cast<const half8_t*>(ab + 32 * kLdsRow + 32 * j);
    }
    {
      half2_t s01, s23;
      decode_scales4(sc0, s01, s23);
      const half8_t b0 = decode8(q0.x, s01[0]), b1 = decode8(q0.y, s01[1]);
      const half8_t b2 = decode8(q0.z, s23[0]), b3 = decode8(q0.w, s23[1]);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[0], b0, acc00, 0, 0, 0);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[1], b1, acc00, 0, 0, 0);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[2], b2, acc00, 0, 0, 0);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[3], b3, acc00, 0, 0, 0);
      if constexpr (TWO) {
        acc10 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[0], b0, acc10, 0, 0, 0);
        acc10 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[1], b1, acc10, 0, 0, 0);
        acc10 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[2], b2, acc10, 0, 0, 0);
        acc10 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[3], b3, acc10, 0, 0, 0);
      }
    }
    {
      half2_t s01, s23;
      decode_scales4(sc1, s01, s23);
      const half8_t b0 = decode8(q1.x, s01[0]), b1 = decode8(q1.y, s01[1]);
      const half8_t b2 = decode8(q1.z, s23[0]), b3 = decode8(q1.w, s23[1]);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[0], b0, acc01, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[1], b1, acc01, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[2], b2, acc01, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[3], b3, acc01, 0, 0, 0);
      if constexpr (TWO) {
        acc11 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[0], b0, acc11, 0, 0, 0);
        acc11 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[1], b1, acc11, 0, 0, 0);
        acc11 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[2], b2, acc11, 0, 0, 0);
        acc11 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[3], b3, acc11, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Full stage st (two chunks) in LDS buffer st & 1 == t, ring slots 2t, 2t+1;
  // loads the next stage's A and decodes it into the other buffer.
  auto stage = [&](const int st, const int t) {
    uint4 qn;
    uint32_t scn;
    a_load(st + 1, qn, scn);  // clamped past the end; the last stage's copy is unused
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* abuf = t ? &a_lds[1][0] : &a_lds[0][0];
    chunk(2 * st, abuf, 0, 2 * t);
    chunk(2 * st + 1, abuf, 1, 2 * t + 1);
    decode_a_store(qn, scn, t ? a_dst0 : a_dst1);
    __syncthreads();
  };

  const int nfull = KC >> 1;  // stages holding two chunks
  int st = 0;
  for (; st + 2 <= nfull; st += 2) {
    stage(st, 0);
    stage(st + 1, 1);
  }
  if (st < nfull) {  // one more full stage (st even: buffer 0, slots 0 and 1)
    stage(st, 0);
    ++st;
  }
  if (KC & 1) {  // final half stage: chunk KC-1 = 2*st, buffer st & 1, slot (2*st) % 4
    const uint8_t* abuf = (st & 1) ? &a_lds[1][0] : &a_lds[0][0];
    if (st & 1)
      chunk(2 * st, abuf, 0, 2);
    else
      chunk(2 * st, abuf, 0, 0);
  }

  // ------------------------------------------------------------------ epilogue
  const bool use0 = p0 < NB, use1 = p0 + 1 < NB;
  const int n = lane & 31;
#pragma unroll
  for (int rb = 0; rb < (TWO ? 2 : 1); ++rb) {
    const floatx16& c0 = rb ? acc10 : acc00;
    const floatx16& c1 = rb ? acc11 : acc01;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * rb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= mrows) continue;
      const float s = s_row[m];
      const long orow = (long)(row0 + m) * P.out_stride;
      if constexpr (MODE == kFc1Relu2) {
        float* out = static_cast<float*>(P.out) + orow;
        if (use0) {
          const float y = __builtin_fmaxf(c0[r] * s, 0.0f);
          out[kColBlock * p0 + n] = y * y;
        }
        if (use1) {
          const float y = __builtin_fmaxf(c1[r] * s, 0.0f);
          out[kColBlock * (p0 + 1) + n] = y * y;
        }
      } else if constexpr (MODE == kFc1Swiglu) {
        // p0 is even: block p0 holds gate rows, p0 + 1 the matching up rows.
        if (use0) {
          const float g = c0[r] * s;
          const float u = c1[r] * s;
          const float silu = g / (1.0f + expf(-g));
          static_cast<float*>(P.out)[orow + kColBlock * (p0 >> 1) + n] = silu * u;
        }
      } else {
        uint16_t* out = static_cast<uint16_t*>(P.out) + orow;
        if (use0) out[kColBlock * p0 + n] = (uint16_t)f32_to_bf16(c0[r] * s);
        if (use1) out[kColBlock * (p0 + 1) + n] = (uint16_t)f32_to_bf16(c1[r] * s);
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void fc_kernel(FcParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kTileM * kLdsRow];
  __shared__ int a_row[kTileM];
  __shared__ float s_row[kTileM];

  const int tid = threadIdx.x;
  const int per = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int NT = fc_col_tiles(P.NB);
  const int nt = logical / P.max_tiles;
  const int tile = logical - nt * P.max_tiles;
  if (nt >= NT || tile >= P.counters[1]) return;
  const int e = P.tiles[2 * tile];
  const int row0 = P.expert_offsets[e] + P.tiles[2 * tile + 1];
  const int mrows = min(kTileM, P.expert_offsets[e + 1] - row0);

  if (tid < kTileM) {
    const int r = row0 + min(tid, mrows - 1);  // rows past the tile end repeat a valid row
    const int ar = P.route_of_row ? P.route_of_row[r] / P.topk : r;
    a_row[tid] = ar;
    s_row[tid] = P.a_scale[ar] * P.w_alpha[e];
  }
  __syncthreads();
  if (mrows > 32)
    fc_tile<MODE, true>(P, a_lds, a_row, s_row, e, row0, mrows, nt);
  else
    fc_tile<MODE, false>(P, a_lds, a_row, s_row, e, row0, mrows, nt);
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
