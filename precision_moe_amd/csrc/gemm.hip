// Expert-sorted grouped GEMMs of the routed-MoE path (FC1 with the fused
// activation, FC2 with the fused per-row / per-expert scaling and BF16 output)
// [Megatron-LM #8262 . Background; FlashInfer #5019 . Tensor and numerical
// contract, 'Compute order'].
//
// Work unit: one M-tile (up to 64 expert-sorted rows of one expert, from the
// device tile list) x one column tile (8 prepared positions of 32 weight rows
// = 256 columns). A workgroup is 4 waves; wave w owns positions 2w and 2w+1
// (four 16-column blocks) and every 16-row block of the tile that holds rows,
// as NRB x 4 accumulators of v_mfma_f32_16x16x32_f16 (NRB = 1..4: a ragged
// tile neither stages nor multiplies the row blocks past its last row).
//
// Reduction loop, in stages of 128 elements (two 64-element chunks):
//   * A (activations, NVFP4 rows gathered by route for FC1, contiguous rows
//     for FC2): each thread buffer-loads 16 bytes of codes (32 elements) and
//     their two block scales of one row, decodes them exactly to FP16 and writes
//     them into a multi-buffered LDS stage [64 rows][128 k]. Within a row the
//     16-byte slots are XOR-swizzled by the row index, so both the stage
//     writes and the MFMA fragment reads hit distinct bank groups (conflict
//     free). BF16 rows (W4A16) are copied into the stage as they are.
//   * B (weights, prepared layout): a column tile's chunk is one contiguous
//     9 KB slab, so a workgroup streams a single sequential region; per chunk
//     and position each lane loads one 16-byte span (1 KB per wave-load) and
//     one dword of four E4M3 scales, by buffer loads with scalar chunk
//     offsets, through a register ring of 2 (W4A16: 4) chunks that is refilled as
//     soon as a position has been decoded; decoding
//     happens in registers straight into MFMA operand order (each block scale
//     multiplied into its 16 decoded values, exact in FP16), and every decoded
//     B fragment feeds all row blocks.
//   * One MFMA k-step of 32 spans two NVFP4 blocks of both operands, whose
//     scales are already in the decoded values; FP32 accumulation.
// Epilogue: y = acc * fp32(g_row * alpha_e) (scales applied after
// accumulation, never folded into decoded values), then
//   FC1 squared ReLU: h = max(y, 0)^2;  FC1 SwiGLU: h = silu(gate) * up, with
//   silu(g) = g * rcp(1 + exp(-g)) on the hardware exp and reciprocal (gate
//   and up column blocks of one output sit in the same wave), optionally with
//   the clamp gate <= L, -L <= up <= L;  FC2: bf16(y);  FC2 with the fused
//   finalize: FP32 atomic add of w * y into the token's row (order-free).
// Outputs other than the atomic adds go through the freed A-stage LDS so that
// each wave writes whole 16-byte pieces of its (contiguous) output columns.
//
// Batch invariance: every output element is one chain of MFMAs over k in fixed
// order whatever T, the tile or the other rows are; no split-K.
// Work order: the real work items (M-tile x column tile) are numbered
// expert-major, then column tile, then M-tile, and each XCD (blockIdx % 8
// picks it) takes one contiguous eighth of them. So the M-tiles that need the
// same weight slab are dispatched together on one XCD and share it through
// its L2 (a hot expert's weights are fetched once, not once per M-tile), and
// an expert's activation rows stay in that L2 across its column tiles.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace pmoe {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlocksPerWave = 2;
constexpr int kColTile = kColTileBlocks;            // column blocks per workgroup (4 waves x 2)
constexpr int kStageK = 128;                       // reduction elements per LDS stage
constexpr int kLdsRow = kStageK * 2;               // bytes per LDS A row (16 slots of 16 B)
constexpr int kLdsStage = kTileM * kLdsRow;        // bytes per LDS stage buffer
constexpr int kBufFlags = 0x00020000;              // raw buffer, 32-bit data format
constexpr int kCpolNT = 2;                         // cache-policy operand: non-temporal
constexpr int kGroup = 2;                          // stages per loop iteration
constexpr int kStages = 2;                         // LDS A stage buffers (double buffer)
// B register ring (chunks per wave) and resident workgroups per CU. The NVFP4
// recipes use a ring of 2 (166-168 VGPRs), which lets 3 workgroups share a CU:
// with the early refill (each load has almost two chunks of work to arrive
// in) that beats a ring of 4 at 2 workgroups per CU, by 6 % for FC1 as one
// launch at the 1024-token EP4 shape. W4A16 (AK = 1: BF16 activations, more
// registers for its decode) keeps a ring of 4 at 2 workgroups per CU
// (200-204 VGPRs).
template <int AK>
struct FcConfig {
  static constexpr int kRing = AK == 0 ? 2 : 4;
  static constexpr int kWgPerCu = AK == 0 ? 3 : 2;
};

__host__ __device__ int fc_col_tiles(int NB) { return padded_col_blocks(NB) / kColTileBlocks; }

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(half8_t a, half8_t b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(bf16x8_t a, bf16x8_t b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The four decoded B fragments of one prepared position (32 weight rows = two
// 16-column blocks h) for one 64-element chunk (two 32-element k-steps s):
// b[2h + s]. FP16 for NVFP4 activations (AK = 0), BF16 for BF16 activations
// (AK = 1). Lane l holds column l%16 of each block and the 8 elements
// 32s + 8(l/16) .. +7; its scale dword holds the E4M3 scale of word (h, s) in
// byte 2h + s.
template <int AK>
struct BFrag {
  using V = std::conditional_t<AK == 1, bf16x8_t, half8_t>;
  V b[4];
  __device__ __forceinline__ BFrag(const uint4& q, uint32_t sc) {
    half2_t s01, s23;
    decode_scales4(sc, s01, s23);
    if constexpr (AK == 1) {
      b[0] = decode8_bf16(q.x, (float)s01[0]);
      b[1] = decode8_bf16(q.y, (float)s01[1]);
      b[2] = decode8_bf16(q.z, (float)s23[0]);
      b[3] = decode8_bf16(q.w, (float)s23[1]);
    } else {
      b[0] = decode8(q.x, s01[0]);
      b[1] = decode8(q.y, s01[1]);
      b[2] = decode8(q.z, s23[0]);
      b[3] = decode8(q.w, s23[1]);
    }
  }
};

// Epilogue of one tile: acc[rb][cb][i] of this wave -> the output. wbuf: this
// wave's kWaveStage bytes of LDS that no other wave uses any more (the caller
// has passed the barrier that ends the main loop's reads).
template <int MODE, int NRB, int AK, int kWaveStage>
__device__ __forceinline__ void fc_epilogue(const FcParams& P, const floatx4 (&acc)[NRB][4],
                                            const float* s_row, int row0, int mrows, int p0, int lane,
                                            uint8_t* wbuf) {
  // acc[rb][cb][i] is row 16*rb + 4*(lane/16) + i, column 16*cb + lane%16 of
  // the wave's 64 columns: position p0 + cb/2, half h = cb%2. Only output
  // columns below P.n_out are written (padding positions and the zero rows
  // that pad a partial column block are dropped; P.n_out is a multiple of 16).
  const int n16 = lane & 15;
  if constexpr (MODE == kFc2Fused) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * rb + 4 * (lane >> 4) + i;
        if (m >= mrows) continue;
        const float s = s_row[m];
        // fused finalize: fp32(w * z) added into the token's FP32 row, in any order
        const int f = P.out_route[row0 + m];
        const float wgt = P.out_w[f];
        float* acc_row = static_cast<float*>(P.out) + (long)(f / P.topk) * P.out_stride;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col0 = kColBlock * p0 + 16 * h + n16, col1 = col0 + kColBlock;
          if (col0 < P.n_out) unsafeAtomicAdd(acc_row + col0, wgt * (acc[rb][h][i] * s));
          if (col1 < P.n_out) unsafeAtomicAdd(acc_row + col1, wgt * (acc[rb][2 + h][i] * s));
        }
      }
    }
  } else {
    // Staged stores: each wave writes its part of the output tile into its own
    // kWaveStage bytes of free LDS, pass by pass, then copies it out in 16-byte
    // row-contiguous pieces. The wave's output columns are contiguous: 64
    // (squared ReLU, FC2) or 32 (SwiGLU: gate and up fold into one). FC1
    // writes FP32 h for the NVFP4 recipes (requantized next) and BF16 h for
    // W4A16 (FC2's input as it is); FC2 writes BF16 z.
    constexpr bool kSwiglu = MODE == kFc1Swiglu;
    constexpr int kS = (MODE == kFc2 || AK == 1) ? 2 : 4;           // bytes per element
    constexpr int kCw = kSwiglu ? 32 : 64;                          // columns per wave
    constexpr int kRowB = kCw * kS;                                 // LDS bytes per row
    constexpr int kPassRows = (kWaveStage / kRowB) < kTileM ? kWaveStage / kRowB : kTileM;
    const int col_base = kSwiglu ? kColBlock * (p0 >> 1) : kColBlock * p0;
    // bytes of an LDS row that exist in the output (whole 16-byte pieces)
    const int row_bytes = min(max(P.n_out - col_base, 0), kCw) * kS;
    auto put = [&](int m, int lc, float v) {
      if constexpr (kS == 2)
        *reinterpret_cast<uint16_t*>(wbuf + m * kRowB + lc * 2) = (uint16_t)f32_to_bf16(v);
      else
        *reinterpret_cast<float*>(wbuf + m * kRowB + lc * 4) = v;
    };
#pragma unroll
    for (int r_lo = 0; r_lo < 16 * NRB; r_lo += kPassRows) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if (16 * rb + 16 <= r_lo || 16 * rb >= r_lo + kPassRows) continue;  // resolved at compile time
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * rb + 4 * (lane >> 4) + i;
          if (m >= mrows) continue;
          const float s = s_row[m];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float c0 = acc[rb][h][i], c1 = acc[rb][2 + h][i];  // positions p0, p0 + 1
            const int lc = 16 * h + n16;
            if constexpr (MODE == kFc1Relu2) {
              const float y0 = __builtin_fmaxf(c0 * s, 0.0f);
              const float y1 = __builtin_fmaxf(c1 * s, 0.0f);
              put(m - r_lo, lc, y0 * y0);
              put(m - r_lo, lc + kColBlock, y1 * y1);
            } else if constexpr (kSwiglu) {
              // p0 is even: position p0 holds gate rows, p0 + 1 the matching up rows.
              float g = c0 * s;
              float u = c1 * s;
              if (P.swiglu_limit > 0.0f) {  // clamp: gate from above, up on both sides
                g = __builtin_fminf(g, P.swiglu_limit);
                u = __builtin_fminf(__builtin_fmaxf(u, -P.swiglu_limit), P.swiglu_limit);
              }
              // hardware exp and reciprocal (a few ulp; h is compared to
              // tolerance, and the requant works on whatever h this writes)
              const float silu = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
              put(m - r_lo, lc, silu * u);
            } else {
              put(m - r_lo, lc, c0 * s);
              put(m - r_lo, lc + kColBlock, c1 * s);
            }
          }
        }
      }
      __syncthreads();
      const int nrow = min(kPassRows, mrows - r_lo);
      uint8_t* out = static_cast<uint8_t*>(P.out) + ((long)(row0 + r_lo) * P.out_stride + (long)col_base) * kS;
#pragma unroll
      for (int k = 0; k < kPassRows * kRowB / (64 * 16); ++k) {
        const int off = (k * 64 + lane) * 16;
        const int r = off / kRowB, cb = off % kRowB;
        if (r < nrow && cb < row_bytes) {
          // FC1's h is written once and read once, by the next kernel:
          // non-temporal stores keep it from displacing the weight slabs
          // that the M-tiles of an expert share in L2
          u32x4* dst = reinterpret_cast<u32x4*>(out + (long)r * P.out_stride * kS + cb);
          const u32x4 val = *reinterpret_cast<const u32x4*>(wbuf + off);
          if constexpr (MODE == kFc1Swiglu || MODE == kFc1Relu2)
            __builtin_nontemporal_store(val, dst);
          else
            *dst = val;
        }
      }
      if (r_lo + kPassRows < 16 * NRB) __syncthreads();  // the next pass overwrites the buffer
    }
  }
}

// Main loop + epilogue for one tile. NRB: the tile's rows rounded up to 16-row
// blocks (1..4); blocks past it are neither staged nor multiplied. kNT = 1:
// the weight loads carry the non-temporal hint (slabs read by this tile only).
// Every global load inside the loop is unconditional, which keeps the in-order
// load counters exact so the B ring really stays in flight: prefetches past
// the last chunk (or stage) re-read the last one -- the chunk index is clamped
// on the scalar side, because the buffer range check does not cover the
// scalar offset -- and their data is never used.
template <int MODE, int NRB, int AK, int kRing, int kNT>
__device__ __forceinline__ void fc_tile(const FcParams& P, uint8_t (*a_lds)[kLdsStage],
                                        const int* a_row, const float* s_row, int e, int row0,
                                        int mrows, int nt) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps descriptors in SGPRs
  const int NB = P.NB, KC = P.KC;

  // A stage fill: thread t -> row r = t/4 of the stage, elements 32*(t%4) ..
  // +32 (k-slots kk = 4*(t%4) + i of 8 elements), stored at slots kk ^ (r % 16).
  // Rows of skipped 16-row blocks are not filled. Out-of-range buffer reads
  // (past the last stage at the last row) return zeros and are never used.
  // AK = 0: NVFP4 rows (K/2 bytes of codes + K/16 scales per row), decoded
  // exactly to FP16 on the way into LDS. AK = 1: BF16 rows (2K bytes), copied
  // into LDS as they are (W4A16).
  constexpr int kAQ = AK == 1 ? 4 : 1;             // 16-byte loads per thread and stage
  const int a_row_bytes = AK == 1 ? KC * 128 : KC * 32;
  const int ar = tid >> 2, aq = tid & 3;
  const bool a_fill = ar < 16 * NRB;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)P.a_codes, (short)0, (int)(P.a_rows * a_row_bytes), kBufFlags);
  const __amdgpu_buffer_rsrc_t a_srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)P.a_sf, (short)0, AK == 1 ? 0 : (int)(P.a_rows * KC * 4), kBufFlags);
  const uint32_t a_voff = (uint32_t)a_row[ar] * (uint32_t)a_row_bytes + aq * 16 * kAQ;
  const uint32_t a_svoff = (uint32_t)a_row[ar] * (uint32_t)(KC * 4) + aq * 2;
  int a_loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_loff[i] = ar * kLdsRow + (((4 * aq + i) ^ (ar & 15)) << 4);
  struct ARaw {
    u32x4 q[kAQ];
    uint32_t s;
  };
  // The stage offset goes into the per-lane offset, which the buffer range
  // check covers: the half stage that ends an odd chunk count reads past the
  // end of the row (data never used), and past the last row of the buffer
  // such reads return zeros instead of touching memory beyond it.
  auto a_copy_load = [&](int st, ARaw& v) {
    if (a_fill) {
      if constexpr (AK == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v.q[i] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff + st * 256 + 16 * i, 0, 0);
      } else {
        v.q[0] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff + st * 64, 0, 0);
        v.s = __builtin_amdgcn_raw_buffer_load_b16(a_srsrc, a_svoff + st * 8, 0, 0);
      }
    }
  };
  auto a_copy_store = [&](uint8_t* buf, const ARaw& v) {
    if (a_fill) {
      if constexpr (AK == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(buf + a_loff[i]) = v.q[i];
      } else {
        const half2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.s, 1.0f, false);
        *reinterpret_cast<half8_t*>(buf + a_loff[0]) = decode8(v.q[0].x, sc[0]);
        *reinterpret_cast<half8_t*>(buf + a_loff[1]) = decode8(v.q[0].y, sc[0]);
        *reinterpret_cast<half8_t*>(buf + a_loff[2]) = decode8(v.q[0].z, sc[1]);
        *reinterpret_cast<half8_t*>(buf + a_loff[3]) = decode8(v.q[0].w, sc[1]);
      }
    }
  };
  // MFMA fragment reads: row block rb, lane -> row 16*rb + lane%16, k-slot
  // kk = 8*half + 4*s + lane/16 of the stage (k-step s of the chunk), at slot
  // kk ^ row%16 (eight lanes of a 128-byte access hit eight distinct slots).
  int frag[2][2];
  {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2) frag[hf][st2] = r * kLdsRow + (((8 * hf + 4 * st2 + g) ^ r) << 4);
  }

  // B stream of this column tile: chunk c of its 8 positions (32 weight rows
  // each) is one contiguous 9 KB slab (8 KB codes + 1 KB scales); wave w reads
  // positions 2w and 2w+1 of it. Reads past the last chunk are out of the
  // buffer range and return zeros. Positions past NB (padding of the last
  // tile) hold zeros.
  const int NT = padded_col_blocks(NB) / kColTileBlocks;
  const int p0 = nt * kColTile + wave * kBlocksPerWave;
  const long tile = (long)e * NT + nt;
  const __amdgpu_buffer_rsrc_t bq = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(P.w_codes + tile * KC * (kColTileBlocks * 1024)), (short)0, KC * kColTileBlocks * 1024,
      kBufFlags);
  const __amdgpu_buffer_rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(P.w_scales + tile * KC * (kColTileBlocks * 128)), (short)0, KC * kColTileBlocks * 128,
      kBufFlags);
  const int pos0 = wave * kBlocksPerWave;
  const int bq_voff0 = pos0 * 1024 + lane * 16, bq_voff1 = bq_voff0 + 1024;
  const int sdw = (lane & 15) + 16 * (lane >> 5);  // this lane's scale dword of a position
  const int bs_voff0 = pos0 * 128 + sdw * 4, bs_voff1 = bs_voff0 + 128;
  auto load_q = [&](int voff, int c) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(bq, voff, c * (kColTileBlocks * 1024),
                                                          kNT ? kCpolNT : 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  auto load_s = [&](int voff, int c) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(bs, voff, c * (kColTileBlocks * 128),
                                                          kNT ? kCpolNT : 0);
  };

  // acc[rb][cb]: 16-row block rb, 16-column block cb of the wave's 64 columns
  // (cb = 2 * (position - p0) + h).
  floatx4 acc[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // B register ring: chunk c lives in slot c % kRing. Early refill: as soon
  // as chunk c has decoded one position's codes and scales, it reloads that
  // half of its slot with chunk c + kRing, so each load has almost kRing
  // chunks of work to arrive in with no registers beyond the ring (a ring of
  // 2 then hides about as much latency as a ring of 3 refilled per chunk:
  // the NVFP4 half launches are 3 % faster). Otherwise (the atomic-finalize
  // FC2, whose epilogue leaves no register for it) chunk c refills slot
  // (c + kRing - 1) % kRing, which chunk c - 1 has finished, before it decodes.
  static_assert(kRing == 2 || kRing == 4, "the stage loop assumes a ring of 2 or 4 chunks");
  constexpr bool kEarly = MODE != kFc2Fused;
  constexpr int kAhead = kEarly ? kRing : kRing - 1;  // chunks loaded before the loop
  uint4 rq0[kRing], rq1[kRing];
  uint32_t rs0[kRing], rs1[kRing];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    const int ci = min(i, KC - 1);
    rq0[i] = load_q(bq_voff0, ci);
    rq1[i] = load_q(bq_voff1, ci);
    rs0[i] = load_s(bs_voff0, ci);
    rs1[i] = load_s(bs_voff1, ci);
  }
  {
    ARaw v;
    a_copy_load(0, v);
    a_copy_store(&a_lds[0][0], v);
  }
  lds_barrier();

  auto chunk = [&](const int c, const uint8_t* abuf, const int half, const int i) {
    if constexpr (!kEarly) {
      // Refill the slot freed by chunk c - 1 before decoding slot i; the
      // scheduling barrier keeps these loads ahead of the decode.
      const int r = (i + kRing - 1) % kRing;
      const int cn = min(c + kRing - 1, KC - 1);
      rq0[r] = load_q(bq_voff0, cn);
      rq1[r] = load_q(bq_voff1, cn);
      rs0[r] = load_s(bs_voff0, cn);
      rs1[r] = load_s(bs_voff1, cn);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int cn = min(c + kRing, KC - 1);  // early refill: the chunk slot i holds next
    using AV = typename BFrag<AK>::V;
    AV a[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        a[rb][s2] = *reinterpret_cast<const AV*>(abuf + 16 * rb * kLdsRow + frag[half][s2]);
    // Each position's fragments are decoded in one block of VALU work and then
    // fed to its MFMAs in one block (scheduling barriers between them): the
    // waves sharing a SIMD then alternate whole decode and MFMA phases, which
    // co-execute better than the compiler's finer interleave (FC1 at the
    // 4096-token shape 2 % faster, the 1024-token step unchanged).
    {
      const BFrag<AK> f(rq0[i], rs0[i]);  // column blocks 0, 1 of the wave
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kEarly) {
        rq0[i] = load_q(bq_voff0, cn);
        rs0[i] = load_s(bs_voff0, cn);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          acc[rb][0] = mfma16(a[rb][s2], f.b[s2], acc[rb][0]);
          acc[rb][1] = mfma16(a[rb][s2], f.b[2 + s2], acc[rb][1]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const BFrag<AK> f(rq1[i], rs1[i]);  // column blocks 2, 3
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kEarly) {
        rq1[i] = load_q(bq_voff1, cn);
        rs1[i] = load_s(bs_voff1, cn);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          acc[rb][2] = mfma16(a[rb][s2], f.b[s2], acc[rb][2]);
          acc[rb][3] = mfma16(a[rb][s2], f.b[2 + s2], acc[rb][3]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Full stage st (two chunks) in LDS buffer t, ring slots slot and slot + 1;
  // loads the next stage's A and stores it into the next buffer.
  const int last_stage = (KC - 1) >> 1;  // stage of the last chunk
  auto stage = [&](const int st, const int t, const int slot) {
    ARaw v;
    a_copy_load(min(st + 1, last_stage), v);  // on the last stage a copy that is unused
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* abuf = &a_lds[t][0];
    chunk(2 * st, abuf, 0, slot);
    chunk(2 * st + 1, abuf, 1, slot + 1);
    a_copy_store(&a_lds[(t + 1) % kStages][0], v);
    lds_barrier();
  };

  // The loop body covers two stages (four chunks): stage j of a pair uses LDS
  // buffer j and ring slots (2j) % kRing and the next one, so every index is
  // a compile-time constant after unrolling (st is even, so chunk c sits in
  // slot c % kRing as the ring requires).
  const int nfull = KC >> 1;  // stages holding two chunks
  int st = 0;
  for (; st + kGroup <= nfull; st += kGroup) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) stage(st + j, j, (2 * j) % kRing);
  }
  const int rem = nfull - st;  // remaining full stages, fewer than kGroup
#pragma unroll
  for (int j = 0; j < kGroup - 1; ++j)
    if (j < rem) stage(st + j, j, (2 * j) % kRing);
  if (KC & 1) {  // final half stage: chunk KC-1 = 2*nfull, group position rem
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      if (j == rem) chunk(2 * nfull, &a_lds[j][0], 0, (2 * j) % kRing);
  }

  // ------------------------------------------------------------------ epilogue
  // The barrier ends every wave's reads of the A stages, which the staged
  // stores below reuse.
  __syncthreads();
  fc_epilogue<MODE, NRB, AK, 8192>(P, acc, s_row, row0, mrows, p0, lane, &a_lds[0][0] + wave * 8192);
}

template <int MODE, int NRB, int AK, int kRing>
__device__ __forceinline__ void tile_nt(bool single, const FcParams& P, uint8_t (*a_lds)[kLdsStage],
                                        const int* a_row, const float* s_row, int e, int row0,
                                        int mrows, int nt) {
  if (single)
    fc_tile<MODE, NRB, AK, kRing, 1>(P, a_lds, a_row, s_row, e, row0, mrows, nt);
  else
    fc_tile<MODE, NRB, AK, kRing, 0>(P, a_lds, a_row, s_row, e, row0, mrows, nt);
}

// The work item of this workgroup -> its expert, rows and column tile; fills
// the tile's A row indices and row scales in LDS. False: no item (the grid is
// rounded up), the workgroup returns.
struct FcItem {
  int e, row0, mrows, nt, count;
};
__device__ __forceinline__ bool fc_item(const FcParams& P, int* a_row, float* s_row, FcItem& it) {
  const int tid = threadIdx.x;
  // Work item -> (tile, column tile): items are numbered expert-major, then
  // column tile, then M-tile; XCD x = blockIdx % 8 takes items
  // [x*per, (x+1)*per) in order.
  const int NT = fc_col_tiles(P.NB);
  // the part's tiles: all, or those of the first / second half of the experts
  const int t_lo = P.part == 2 ? P.counters[2] : 0;
  const int t_hi = P.part == 1 ? P.counters[2] : P.counters[1];
  const int total = (t_hi - t_lo) * NT;
  const int per = (total + 7) >> 3;
  const int j = blockIdx.x >> 3;
  if (j >= per) return false;
  const int item = t_lo * NT + (blockIdx.x & 7) * per + j;
  if (item >= t_hi * NT) return false;
  // Every tile entry of an expert holds {expert, its first row, its first
  // tile, its row count}: one load gives the item's rows.
  const int4 ta = reinterpret_cast<const int4*>(P.tiles)[item / NT];
  const int e = ta.x, first = ta.z, rows_e = ta.w;
  const int count = (rows_e + kTileM - 1) / kTileM;
  const int local = item - first * NT;
  const int nt = local / count;
  const int m_tile = local - nt * count;
  const int row0 = ta.y + m_tile * kTileM;
  const int mrows = min(kTileM, rows_e - m_tile * kTileM);

  if (tid < kTileM) {
    const int r = row0 + min(tid, mrows - 1);  // rows past the tile end repeat a valid row
    const int ar = P.route_of_row ? P.route_of_row[r] / P.topk : r;
    a_row[tid] = ar;
    // per-token / per-row scale times alpha, or the (folded) alpha alone
    s_row[tid] = P.a_scale ? P.a_scale[ar] * P.w_alpha[e] : P.w_alpha[e];
  }
  __syncthreads();
  it = FcItem{e, row0, mrows, nt, count};
  return true;
}

template <int MODE, int AK, int kRing>
__device__ __forceinline__ void fc_block(const FcParams& P, uint8_t (*a_lds)[kLdsStage],
                                         int* a_row, float* s_row) {
  FcItem it;
  if (!fc_item(P, a_row, s_row, it)) return;
  const int e = it.e, row0 = it.row0, mrows = it.mrows, nt = it.nt, count = it.count;
  switch ((mrows + 15) >> 4) {  // 16-row blocks that hold rows of this tile
    // An expert with one M-tile reads its weight slabs once: its B loads are
    // non-temporal (kNT), so they do not displace the slabs that the M-tiles
    // of a multi-tile expert share in L2.
    case 1: tile_nt<MODE, 1, AK, kRing>(count == 1, P, a_lds, a_row, s_row, e, row0, mrows, nt); break;
    case 2: tile_nt<MODE, 2, AK, kRing>(count == 1, P, a_lds, a_row, s_row, e, row0, mrows, nt); break;
    case 3: tile_nt<MODE, 3, AK, kRing>(count == 1, P, a_lds, a_row, s_row, e, row0, mrows, nt); break;
    default: tile_nt<MODE, 4, AK, kRing>(count == 1, P, a_lds, a_row, s_row, e, row0, mrows, nt); break;
  }
}

// One launch over the tiles of every local expert.
template <int MODE, int AK>
__global__ __launch_bounds__(kThreads, (FcConfig<AK>::kWgPerCu)) void fc_kernel(FcParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kStages][kLdsStage];
  __shared__ int a_row[kTileM];
  __shared__ float s_row[kTileM];
  fc_block<MODE, AK, FcConfig<AK>::kRing>(P, a_lds, a_row, s_row);
}

// The same code over one half of the experts (P.part = 1 or 2); a kernel of
// its own name so that a trace tells the half launches from the whole ones.
template <int MODE, int AK>
__global__ __launch_bounds__(kThreads, (FcConfig<AK>::kWgPerCu)) void fc_half_kernel(FcParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kStages][kLdsStage];
  __shared__ int a_row[kTileM];
  __shared__ float s_row[kTileM];
  fc_block<MODE, AK, FcConfig<AK>::kRing>(P, a_lds, a_row, s_row);
}

template <int MODE, int AK>
void launch_fc_mode(const FcParams& p, long grid, hipStream_t s) {
  if (p.part)
    fc_half_kernel<MODE, AK><<<grid, kThreads, 0, s>>>(p);
  else
    fc_kernel<MODE, AK><<<grid, kThreads, 0, s>>>(p);
}

template <int AK>
void launch_fc_ak(FcMode mode, const FcParams& p, long grid, hipStream_t s) {
  switch (mode) {
    case kFc1Relu2: launch_fc_mode<kFc1Relu2, AK>(p, grid, s); break;
    case kFc1Swiglu: launch_fc_mode<kFc1Swiglu, AK>(p, grid, s); break;
    case kFc2: launch_fc_mode<kFc2, AK>(p, grid, s); break;
    case kFc2Fused: launch_fc_mode<kFc2Fused, AK>(p, grid, s); break;
  }
}

hipError_t launch_fc(FcMode mode, const FcParams& p, hipStream_t s) {
  const long blocks = (long)p.max_tiles * fc_col_tiles(p.NB);
  const long grid = (blocks + 7) / 8 * 8;
  if (p.a_bf16)
    launch_fc_ak<1>(mode, p, grid, s);
  else
    launch_fc_ak<0>(mode, p, grid, s);
  return hipGetLastError();
}

}  // namespace pmoe
