// Routing: histogram + prefix-sum permutation of the valid routes into
// expert-contiguous rows, feeding the grouped GEMMs (the expert-sorted layout
// the pages' block-scaled grouped GEMMs consume [Megatron-LM #8262 .
// Background]). Deterministic by construction: integer counts only, and the
// order is fixed -- rows of an expert follow ascending route index f = t*K + j
// (a stable sort).
//
//   route_count   : per 256-route block, each valid route's rank among the
//                   block's earlier routes to the same expert (wave ballots on
//                   the expert id bits + per-wave counts in LDS), and the block's
//                   per-expert counts.
//   route_scan    : one workgroup: per expert, exclusive prefix over blocks
//                   (in place), totals, exclusive scan over experts, the
//                   M-tile list (tiles of 64 rows, grouped by expert in
//                   expert order; every tile of an expert holds {expert, its
//                   first row, its first tile, its row count}), and the
//                   expert boundary nearest 44 % of the tiles (counters[2],
//                   counters[3]: first tile and row of the second part), for
//                   running the two parts on two streams.
//   route_scatter : row = expert start + block prefix + in-block rank;
//                   writes row_of_route and route_of_row.
// A route is valid iff expert_offset <= id < expert_offset + E; other ids
// (the -1 fill of unused slots, other ranks' experts) are skipped.
#include "rowquant.h"

namespace pmoe {

int route_blocks(int TK) { return (TK + kRouteBlock - 1) / kRouteBlock; }

template <typename IdT>
__device__ __forceinline__ int local_expert(const IdT* ids, int f, int E, int offset) {
  const long long loc = (long long)ids[f] - (long long)offset;
  return (loc >= 0 && loc < E) ? (int)loc : -1;
}

template <typename IdT>
__global__ __launch_bounds__(256) void route_count_kernel(const IdT* __restrict__ ids, int TK, int E,
                                                          int offset, int nbits,
                                                          int* __restrict__ rank_local,
                                                          int* __restrict__ block_counts) {
  __shared__ int wcnt[4][kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += 256) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int f = blockIdx.x * kRouteBlock + tid;
  const int e = f < TK ? local_expert(ids, f, E, offset) : -1;
  // Lanes of this wave routed to the same expert: AND of per-bit ballots.
  uint64_t match = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t set = __ballot(bit);
    match &= bit ? set : ~set;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_w = __popcll(match & below);
  if (e >= 0 && rank_w == 0) wcnt[wave][e] = __popcll(match);
  __syncthreads();
  if (f < TK) {
    int r = -1;
    if (e >= 0) {
      r = rank_w;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
    }
    rank_local[f] = r;
  }
  for (int x = tid; x < E; x += 256)
    block_counts[(long)blockIdx.x * E + x] = wcnt[0][x] + wcnt[1][x] + wcnt[2][x] + wcnt[3][x];
}

#ifndef PMOE_SPLIT_PCT
#define PMOE_SPLIT_PCT 44
#endif
// Where the expert-sorted tiles are cut into the two parts that run on two
// streams: at the expert boundary nearest to PMOE_SPLIT_PCT % of the tiles
// (counters[2] = first tile, counters[3] = first row of the second part).
// The first part, on the caller's stream, starts right after the routing and
// its workgroups are dispatched ahead of the second part's, which waits for a
// cross-stream event; giving it less than half the tiles lets the two chains
// end closer together (44 % measured best of 35-56 %).
// The expert whose tiles straddle the target writes it; with no tiles at all,
// the first thread writes 0.
__device__ __forceinline__ void write_split(bool is_expert, int tstart, int ntiles, int start,
                                            int rows, int total_tiles, bool first_thread,
                                            int* counters) {
  const int target = (int)((long long)total_tiles * PMOE_SPLIT_PCT / 100);
  if (is_expert && ntiles > 0 && tstart <= target && target < tstart + ntiles) {
    const bool before = target - tstart <= tstart + ntiles - target;
    counters[2] = before ? tstart : tstart + ntiles;
    counters[3] = before ? start : start + rows;
  }
  if (total_tiles == 0 && first_thread) {
    counters[2] = 0;
    counters[3] = 0;
  }
}

// Inclusive prefix sum over the 1024 threads of a workgroup; the total is left
// in sh[1023]. Each wave scans its 64 values with shuffles, then adds the
// totals of the waves before it (two barriers instead of twenty).
__device__ __forceinline__ int block_inclusive_scan_1024(int v, int* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int t = sh[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();  // every wave has read sh[0..15]
  if (tid == 1023) sh[1023] = total;
  __syncthreads();
  return x + before;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(int* __restrict__ block_counts, int NB,
                                                          int E, int* __restrict__ expert_offsets,
                                                          int* __restrict__ tiles,
                                                          int* __restrict__ counters) {
  __shared__ int sh[1024];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    // exclusive prefix over blocks, in place; eight independent loads per
    // round so the latency is paid once per eight blocks, not once per block
    for (int b0 = 0; b0 < NB; b0 += 8) {
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = b0 + i < NB ? block_counts[(long)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (b0 + i < NB) block_counts[(long)(b0 + i) * E + e] = total;
        total += c[i];
      }
    }
  }
  const int incl = block_inclusive_scan_1024(total, sh);
  const int start = incl - total;
  const int R = sh[1023];
  __syncthreads();
  const int ntiles = (total + kTileM - 1) / kTileM;
  const int tincl = block_inclusive_scan_1024(ntiles, sh);
  const int tstart = tincl - ntiles;
  if (e < E) {
    expert_offsets[e] = start;
    for (int i = 0; i < ntiles; ++i) {
      int4* t = reinterpret_cast<int4*>(tiles) + tstart + i;
      *t = make_int4(e, start, tstart, total);
    }
  }
  if (e == 0) {
    expert_offsets[E] = R;
    counters[0] = R;
    counters[1] = sh[1023];
  }
  write_split(e < E, tstart, ntiles, start, total, sh[1023], e == 0, counters);
}

template <typename IdT>
__global__ __launch_bounds__(256) void route_scatter_kernel(
    const IdT* __restrict__ ids, int TK, int E, int offset, const int* __restrict__ rank_local,
    const int* __restrict__ block_prefix, const int* __restrict__ expert_offsets,
    int* __restrict__ row_of_route, int* __restrict__ route_of_row) {
  const int f = blockIdx.x * kRouteBlock + threadIdx.x;
  if (f >= TK) return;
  const int r = rank_local[f];
  if (r < 0) {
    row_of_route[f] = -1;
    return;
  }
  const int e = local_expert(ids, f, E, offset);
  const int row = expert_offsets[e] + block_prefix[(long)blockIdx.x * E + e] + r;
  row_of_route[f] = row;
  route_of_row[row] = f;
}

// The whole routing in one workgroup of 1024 threads, for up to
// kRouteSmall routes (one launch instead of three). Wave w owns the
// contiguous routes [w*seg*64, (w+1)*seg*64) (seg = ceil(TK / 1024) chunks of
// 64) and loads all of its ids up front. Within a chunk, lanes with the same
// expert find each other by ballots on the expert id bits, which gives each
// route its rank among them and one leader per (chunk, expert) that adds the
// group's size to the wave's own count of that expert in LDS; each route
// first reads that count (its expert's routes in the wave's earlier chunks).
// Only the wave itself touches its counts and a wave's LDS operations run in
// program order, so the chunks need no barrier. After one barrier, each
// expert's counts become exclusive prefixes over the waves and its total
// feeds the scans. A route's row is then its expert's start + the expert's
// routes in earlier waves + in the wave's earlier chunks + its rank: the same
// stable order (ascending route index within an expert) as the three-kernel
// path.
constexpr int kRouteSmall = 8192;
constexpr int kRouteSmallPer = kRouteSmall / 1024;

// LDS of the one-workgroup routing.
struct RouteSmallLds {
  int base[kMaxExperts];      // each expert's first row
  int wcnt[16][kMaxExperts];  // routes per (wave, expert), then the exclusive prefix over waves
  int sh[1024];
};

// The routing body; the caller is a workgroup of 1024 threads.
template <typename IdT>
__device__ __forceinline__ void route_small_body(const IdT* __restrict__ ids, int TK, int E,
                                                 int offset, int nbits,
                                                 int* __restrict__ expert_offsets,
                                                 int* __restrict__ tiles, int* __restrict__ counters,
                                                 int* __restrict__ row_of_route,
                                                 int* __restrict__ route_of_row, RouteSmallLds& lds) {
  int* base = lds.base;
  int(*wcnt)[kMaxExperts] = lds.wcnt;
  int* sh = lds.sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int seg = (TK + 1023) >> 10;  // chunks of 64 per wave, at most kRouteSmallPer
  const int f0 = wave * seg * 64 + lane;
  int ev[kRouteSmallPer], rank[kRouteSmallPer], before[kRouteSmallPer];
#pragma unroll
  for (int c = 0; c < kRouteSmallPer; ++c) {
    const int f = f0 + 64 * c;
    ev[c] = (c < seg && f < TK) ? local_expert(ids, f, E, offset) : -1;
  }
  for (int i = tid; i < 16 * kMaxExperts; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* mine = wcnt[wave];
#pragma unroll
  for (int c = 0; c < kRouteSmallPer; ++c) {
    rank[c] = 0;
    before[c] = 0;
    if (c >= seg) continue;  // uniform across the workgroup
    const int e = ev[c];
    uint64_t match = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(bit);
      match &= bit ? set : ~set;
    }
    rank[c] = __popcll(match & below);
    if (e >= 0) {
      before[c] = mine[e];  // read before this chunk's leaders add to it
      if (rank[c] == 0) atomicAdd(&mine[e], __popcll(match));
    }
  }
  __syncthreads();
  int total = 0;
  if (tid < E) {
    int cw[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) cw[w] = wcnt[w][tid];
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      wcnt[w][tid] = total;
      total += cw[w];
    }
  }
  const int incl = block_inclusive_scan_1024(total, sh);
  const int start = incl - total;
  const int R = sh[1023];
  __syncthreads();
  const int ntiles = (total + kTileM - 1) / kTileM;
  const int tincl = block_inclusive_scan_1024(ntiles, sh);
  const int tstart = tincl - ntiles;
  const int T_tiles = sh[1023];
  if (tid < E) {
    expert_offsets[tid] = start;
    base[tid] = start;
    for (int i = 0; i < ntiles; ++i)
      reinterpret_cast<int4*>(tiles)[tstart + i] = make_int4(tid, start, tstart, total);
  }
  if (tid == 0) {
    expert_offsets[E] = R;
    counters[0] = R;
    counters[1] = T_tiles;
  }
  write_split(tid < E, tstart, ntiles, start, total, T_tiles, tid == 0, counters);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kRouteSmallPer; ++c) {
    if (c >= seg) break;  // uniform
    const int f = f0 + 64 * c;
    const int e = ev[c];
    if (e >= 0) {
      const int row = base[e] + mine[e] + before[c] + rank[c];
      row_of_route[f] = row;
      route_of_row[row] = f;
    } else if (f < TK) {
      row_of_route[f] = -1;
    }
  }
}

template <typename IdT>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const IdT* __restrict__ ids, int TK, int E, int offset, int nbits,
    int* __restrict__ expert_offsets, int* __restrict__ tiles, int* __restrict__ counters,
    int* __restrict__ row_of_route, int* __restrict__ route_of_row) {
  __shared__ RouteSmallLds lds;
  route_small_body<IdT>(ids, TK, E, offset, nbits, expert_offsets, tiles, counters, row_of_route,
                        route_of_row, lds);
}

// The routing and the per-token quantization of the BF16 input in one launch:
// workgroup 0 routes (as route_small_kernel), workgroup b >= 1 quantizes rows
// 4(b-1) .. 4(b-1)+3, one group of 256 threads per row (quantize_row_group:
// the same bytes as quantize_rows_kernel). The two jobs share no data, so
// they run side by side and the grouped GEMM that needs both can follow on
// the same stream.
template <typename IdT, bool kStatic>
__global__ __launch_bounds__(1024) void route_quantize_kernel(
    const IdT* __restrict__ ids, int TK, int E, int offset, int nbits,
    int* __restrict__ expert_offsets, int* __restrict__ tiles, int* __restrict__ counters,
    int* __restrict__ row_of_route, int* __restrict__ route_of_row, const void* __restrict__ x,
    int T, int H, int Hq, const float* __restrict__ static_a, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ x_sf, float* __restrict__ x_scale) {
  __shared__ RouteSmallLds lds;
  if (blockIdx.x == 0) {
    route_small_body<IdT>(ids, TK, E, offset, nbits, expert_offsets, tiles, counters, row_of_route,
                          route_of_row, lds);
    return;
  }
  const int grp = threadIdx.x >> 8;
  const long row = (long)(blockIdx.x - 1) * 4 + grp;
  quantize_row_group<true, kStatic>(x, row, row < T, H, Hq, threadIdx.x & 255, static_a, xq, x_sf,
                                    x_scale, reinterpret_cast<float*>(lds.sh) + 4 * grp);
}

static int expert_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

bool route_quantize_fits(int TK) { return TK <= kRouteSmall; }

template <typename IdT>
static void launch_route_quantize_t(const IdT* ids, int TK, int E, int expert_offset,
                                    const RouteBuffers& b, const void* x, int T, int H, int Hq,
                                    const float* static_a, uint8_t* xq, uint8_t* x_sf,
                                    float* x_scale, hipStream_t s) {
  const int grid = 1 + (T + 3) / 4;
  if (static_a)
    route_quantize_kernel<IdT, true><<<grid, 1024, 0, s>>>(
        ids, TK, E, expert_offset, expert_bits(E), b.expert_offsets, b.tiles, b.counters,
        b.row_of_route, b.route_of_row, x, T, H, Hq, static_a, xq, x_sf, nullptr);
  else
    route_quantize_kernel<IdT, false><<<grid, 1024, 0, s>>>(
        ids, TK, E, expert_offset, expert_bits(E), b.expert_offsets, b.tiles, b.counters,
        b.row_of_route, b.route_of_row, x, T, H, Hq, nullptr, xq, x_sf, x_scale);
}

hipError_t launch_route_quantize(const void* ids, bool ids64, int TK, int E, int expert_offset,
                                 const RouteBuffers& b, const void* x, int T, int H, int Hq,
                                 const float* static_a, uint8_t* xq, uint8_t* x_sf, float* x_scale,
                                 hipStream_t s) {
  if (!route_quantize_fits(TK)) return hipErrorInvalidValue;
  if (ids64)
    launch_route_quantize_t(static_cast<const long long*>(ids), TK, E, expert_offset, b, x, T, H,
                            Hq, static_a, xq, x_sf, x_scale, s);
  else
    launch_route_quantize_t(static_cast<const int*>(ids), TK, E, expert_offset, b, x, T, H, Hq,
                            static_a, xq, x_sf, x_scale, s);
  return hipGetLastError();
}

hipError_t launch_route(const void* ids, bool ids64, int TK, int E, int expert_offset,
                        const RouteBuffers& b, hipStream_t s) {
  const int NB = route_blocks(TK);
  const int nbits = expert_bits(E);
  if (TK <= kRouteSmall) {
    if (ids64)
      route_small_kernel<long long><<<1, 1024, 0, s>>>(
          static_cast<const long long*>(ids), TK, E, expert_offset, nbits, b.expert_offsets, b.tiles,
          b.counters, b.row_of_route, b.route_of_row);
    else
      route_small_kernel<int><<<1, 1024, 0, s>>>(
          static_cast<const int*>(ids), TK, E, expert_offset, nbits, b.expert_offsets, b.tiles,
          b.counters, b.row_of_route, b.route_of_row);
    return hipGetLastError();
  }
  if (ids64)
    route_count_kernel<long long><<<NB, 256, 0, s>>>(static_cast<const long long*>(ids), TK, E,
                                                     expert_offset, nbits, b.rank_local,
                                                     b.block_counts);
  else
    route_count_kernel<int><<<NB, 256, 0, s>>>(static_cast<const int*>(ids), TK, E, expert_offset,
                                               nbits, b.rank_local, b.block_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  route_scan_kernel<<<1, 1024, 0, s>>>(b.block_counts, NB, E, b.expert_offsets, b.tiles,
                                       b.counters);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ids64)
    route_scatter_kernel<long long><<<NB, 256, 0, s>>>(
        static_cast<const long long*>(ids), TK, E, expert_offset, b.rank_local, b.block_counts,
        b.expert_offsets, b.row_of_route, b.route_of_row);
  else
    route_scatter_kernel<int><<<NB, 256, 0, s>>>(static_cast<const int*>(ids), TK, E, expert_offset,
                                                 b.rank_local, b.block_counts, b.expert_offsets,
                                                 b.row_of_route, b.route_of_row);
  return hipGetLastError();
}

}  // namespace pmoe
