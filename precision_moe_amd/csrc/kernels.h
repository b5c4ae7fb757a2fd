// Internal launchers of the pmoe kernels (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmoe {

constexpr int kTileM = 64;     // rows per M-tile of the grouped GEMMs (two MFMA row blocks)
constexpr int kColBlock = 32;  // weight rows per prepared column block
constexpr int kChunk = 64;     // reduction elements per prepared chunk
constexpr int kColTileBlocks = 8;  // column blocks per column tile (one GEMM workgroup)
__host__ __device__ inline int padded_col_blocks(int NB) {
  return (NB + kColTileBlocks - 1) / kColTileBlocks * kColTileBlocks;
}
constexpr int kRouteBlock = 256;
constexpr int kMaxExperts = 1024;
constexpr int kMaxRow = 16384;  // longest row (H, I) the path accepts
constexpr int kDimStep = 16;    // H and I are multiples of this (one E4M3 block)
// A reduction length padded to whole GEMM chunks: the operands of the grouped
// GEMMs carry zero codes and zero scales in [Kd, padded_k(Kd)).
__host__ __device__ inline int padded_k(int Kd) { return (Kd + kChunk - 1) / kChunk * kChunk; }
// Prepared column blocks of an FC matrix with N output rows; a gated FC1
// (N = 2I) has ceil(I/32) gate blocks and as many up blocks, interleaved.
__host__ __device__ inline int col_blocks(int N, int gated_I) {
  return gated_I > 0 ? 2 * ((gated_I + kColBlock - 1) / kColBlock) : (N + kColBlock - 1) / kColBlock;
}

// ---------------------------------------------------------------- quantizers
// static_a: null for per-row scales (written to *_scale), else the device
// address of a static scale a (rows use g = 1/a; no scale is written).
// Input rows have H (L) elements; output rows Hq (Lq) >= H, the blocks past H
// written as zeros.
hipError_t launch_quantize_bf16(const void* x, int T, int H, int Hq, const float* static_a,
                                uint8_t* xq, uint8_t* x_sf, float* x_scale, hipStream_t s);
// Rows [*row_begin_dev, *row_end_dev) of R (either pointer may be null: 0 / R).
// beside_gemm: the launch runs while another stream's grouped GEMM holds the
// CUs (one wave per row over a bounded grid); else one workgroup per row.
hipError_t launch_quantize_f32(const float* h, int R, const int* row_begin_dev,
                               const int* row_end_dev, int L, int Lq, const float* static_a,
                               uint8_t* hq, uint8_t* h_sf, float* h_scale, bool beside_gemm,
                               hipStream_t s);
// rows x row_bytes -> rows x dst_row_bytes, the tail of every row zero-filled.
hipError_t launch_pad_rows(const void* src, long rows, long row_bytes, long dst_row_bytes, void* dst,
                           hipStream_t s);

// ---------------------------------------------------------------- weights
int weight_amax_parts(long elems);
// fold_a: null, or the device address of a static input scale folded into alpha.
hipError_t launch_prepare_fc(const uint16_t* w, int E, int N, int Kd, int gated_I, float* partials,
                             const float* fold_a, uint8_t* codes, uint8_t* scales, float* alpha,
                             hipStream_t s);

// ---------------------------------------------------------------- routing
struct RouteBuffers {
  int* rank_local;      // [TK]
  int* block_counts;    // [route blocks][E]
  int* expert_offsets;  // [E+1]
  int* tiles;           // [max_tiles][4]: every M-tile of expert e holds {e, e's first row,
                        // e's first tile, e's row count}; tiles are grouped by expert
  int* counters;        // [4] = {R, tiles, first tile and first row of the second part}
  int* row_of_route;    // [TK]
  int* route_of_row;    // [TK]
};
int route_blocks(int TK);
hipError_t launch_route(const void* ids, bool ids64, int TK, int E, int expert_offset,
                        const RouteBuffers& b, hipStream_t s);
// The routing and the per-token (or static-scale) quantization of BF16 input
// rows [T][H] in one launch, for TK routes that one workgroup can route
// (route_quantize_fits); same results as launch_route + launch_quantize_bf16.
bool route_quantize_fits(int TK);
hipError_t launch_route_quantize(const void* ids, bool ids64, int TK, int E, int expert_offset,
                                 const RouteBuffers& b, const void* x, int T, int H, int Hq,
                                 const float* static_a, uint8_t* xq, uint8_t* x_sf, float* x_scale,
                                 hipStream_t s);

// ---------------------------------------------------------------- grouped GEMMs
enum FcMode { kFc1Relu2 = 0, kFc1Swiglu = 1, kFc2 = 2, kFc2Fused = 3 };

struct FcParams {
  const uint8_t* a_codes;    // A rows of Kd/2 bytes (packed E2M1), or of 2*Kd bytes (BF16)
  const uint8_t* a_sf;       // A rows of Kd/16 bytes (E4M3 block scales); unused for BF16 A
  long a_rows;               // rows in the A buffer (< 4 GiB)
  int a_bf16;                // 1: A is BF16 (W4A16: BF16 MFMA, FC1 writes BF16 h)
  const float* a_scale;      // per A row, or null (per-tensor / W4A16: alpha alone)
  const int* route_of_row;   // FC1: expert-sorted row -> route (A row = route / topk); FC2: null
  int topk;
  const uint8_t* w_codes;    // prepared layout
  const uint8_t* w_scales;
  const float* w_alpha;
  int NB;                    // column blocks of 32 in this FC (before padding to whole tiles)
  int KC;                    // chunks of 64 along the (padded) reduction
  int n_out;                 // output columns written (FC1 SwiGLU: of the activation output)
  const int* tiles;          // [tiles][4], see RouteBuffers
  const int* counters;       // [1] = number of M-tiles, [2] = first M-tile of the second part
  int part;                  // 0: all tiles; 1 / 2: the tiles before / from counters[2]
  int max_tiles;
  void* out;                 // FC1: h [rows][out_stride] (float, BF16 when a_bf16); FC2: BF16 z;
                             // FC2 fused: float accumulator [T][out_stride]
  int out_stride;
  float swiglu_limit;        // FC1 SwiGLU clamp limit, 0 = none
  const int* out_route;      // FC2 fused: route of each expert-sorted row
  const float* out_w;        // FC2 fused: routing weights [T*K]
};
__host__ __device__ int fc_col_tiles(int NB);
hipError_t launch_fc(FcMode mode, const FcParams& p, hipStream_t s);

// ---------------------------------------------------------------- finalize
hipError_t launch_finalize(const uint16_t* z, const int* row_of_route, const float* w, int T,
                           int K, int H, uint16_t* out, hipStream_t s);
// Fused finalize: zero the FP32 accumulator [n] before FC2, round it to BF16 after.
hipError_t launch_fill_zero(float* p, long n, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, long n, uint16_t* out, hipStream_t s);

// ---------------------------------------------------------------- router
hipError_t launch_router_topk(const float* logits, int T, int E, int K, int renorm, int* ids,
                              float* w, hipStream_t s);

}  // namespace pmoe
