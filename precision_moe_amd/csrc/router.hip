// Router front: top-k expert selection and softmax weights from FP32 router
// logits (plain top-k, no group-limited routing [Megatron-LM #8262 .
// Performance]).
//
// One wavefront per token (four per 256-thread workgroup). Lane l holds the
// logits of experts l, l + 64, ... (at most 16). The choice is made on the
// logits themselves -- softmax is strictly increasing, so this is the top-k of
// the probabilities -- and is exact: k rounds of a wave-wide argmax, larger
// logit first, equal logits to the lower expert id. Weights are
// exp(l - max) / sum_all exp(l - max) in FP32, each lane summing its own
// logits in a fixed order and the wave combining the 64 partial sums in a fixed
// butterfly, so the result is deterministic; optionally divided by their sum
// over the k slots (slot order).
#include "device.h"
#include "kernels.h"

namespace pmoe {

constexpr int kRouterPerLane = kMaxExperts / 64;

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int K, int renorm,
                                                          int* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves leave together
  const float* row = logits + (long)t * E;
  float v[kRouterPerLane];
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < kRouterPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
    m = __builtin_fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < kRouterPerLane; ++i)
    if (lane + 64 * i < E) part += expf(v[i] - m);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
  const float den = part;

  uint32_t taken = 0;  // bit i: expert lane + 64 i already chosen
  float wsum = 0.0f;
  float wj_keep = 0.0f;  // the weight of slot `lane` (lanes < K keep one slot each)
  int id_keep = 0;
  for (int j = 0; j < K; ++j) {
    // this lane's best remaining expert: larger logit, then lower id
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kRouterPerLane; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    const float p = expf(bv - m) / den;
    wsum += p;  // slot order, the same value in every lane
    if (lane == j) {
      wj_keep = p;
      id_keep = be;
    }
  }
  if (lane < K) {
    ids[(long)t * K + lane] = id_keep;
    w[(long)t * K + lane] = renorm ? wj_keep / wsum : wj_keep;
  }
}

hipError_t launch_router_topk(const float* logits, int T, int E, int K, int renorm, int* ids,
                              float* w, hipStream_t s) {
  router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, K, renorm, ids, w);
  return hipGetLastError();
}

}  // namespace pmoe
