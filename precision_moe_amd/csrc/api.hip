// C ABI of the pmoe library: host-side validation and launch sequencing.
// No kernel lives here. Every entry point validates all of its arguments on
// the host before the first launch, enqueues on the caller's stream (the
// routed-MoE calls also on one library-owned second stream per device, forked
// from and joined back into the caller's), and never allocates device memory
// for data or synchronizes with the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/pmoe.h"
#include "kernels.h"

#define PMOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace pmoe;

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return PMOE_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ device check
int check_device() {
  static std::mutex mu;
  static int cached[64];  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PMOE_ERR_DEVICE, "no HIP device is current");
  if (dev < 0 || dev >= 64) return fail(PMOE_ERR_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(PMOE_ERR_DEVICE, "hipGetDeviceProperties failed");
    cached[dev] = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : 2;
    if (cached[dev] == 2) {
      g_last_error = std::string("pmoe needs a gfx950 GPU (MI355X / MI350X); current device is ") +
                     prop.gcnArchName;
      return PMOE_ERR_DEVICE;
    }
  }
  if (cached[dev] != 1) return fail(PMOE_ERR_DEVICE, "pmoe needs a gfx950 GPU (MI355X / MI350X)");
  return PMOE_OK;
}

// ------------------------------------------------------------------ pointer check
int check_ptr(const void* p, size_t align, const char* name) {
  if (p == nullptr) return fail(PMOE_ERR_POINTER, std::string(name) + " is null");
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(PMOE_ERR_POINTER, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return fail(PMOE_ERR_POINTER, std::string(name) + " is not a HIP device pointer");
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(PMOE_ERR_POINTER, std::string(name) + " is not device memory");
  return PMOE_OK;
}

#define PMOE_TRY(expr)          \
  do {                          \
    int _rc = (expr);           \
    if (_rc != PMOE_OK) return _rc; \
  } while (0)

#define PMOE_HIP(expr)                                                                    \
  do {                                                                                    \
    hipError_t _e = (expr);                                                               \
    if (_e != hipSuccess) return fail(PMOE_ERR_HIP, std::string("HIP error: ") + hipGetErrorString(_e)); \
  } while (0)

// ------------------------------------------------------------------ shapes
// H and I: multiples of 16 (one E4M3 block) up to 16384. The grouped GEMMs
// reduce over whole chunks of 64; a length that is not a multiple of 64 is
// padded inside the library with zero codes and zero block scales, which add
// exactly zero to every sum.
bool dim_ok(int v) { return v > 0 && v % kDimStep == 0 && v <= kMaxRow; }
#define PMOE_DIM_RULE " must be a multiple of 16 in [16, 16384]"

int check_weight_shape(int E, int N1, int H, int I) {
  if (E < 1 || E > kMaxExperts) return fail(PMOE_ERR_SHAPE, "E must be in [1, 1024]");
  if (!dim_ok(H)) return fail(PMOE_ERR_SHAPE, "H" PMOE_DIM_RULE);
  if (!dim_ok(I)) return fail(PMOE_ERR_SHAPE, "I" PMOE_DIM_RULE);
  if (N1 != I && N1 != 2 * I)
    return fail(PMOE_ERR_SHAPE, "FC1 width N1 must be I (squared ReLU) or 2*I (SwiGLU)");
  return PMOE_OK;
}

struct WeightBytes {
  size_t w1q, w1s, w2q, w2s;
};
WeightBytes weight_bytes(int E, int N1, int H, int I) {
  WeightBytes b;
  // row counts padded to whole column tiles (8 blocks of 32 rows), reduction
  // lengths to whole chunks of 64
  const size_t n1p = (size_t)padded_col_blocks(col_blocks(N1, N1 == 2 * I ? I : 0)) * kColBlock;
  const size_t hp = (size_t)padded_col_blocks(col_blocks(H, 0)) * kColBlock;
  const size_t Hp = padded_k(H), Ip = padded_k(I);
  b.w1q = (size_t)E * n1p * Hp / 2;
  b.w1s = (size_t)E * n1p * Hp / 16;
  b.w2q = (size_t)E * hp * Ip / 2;
  b.w2s = (size_t)E * hp * Ip / 16;
  return b;
}

size_t prepare_ws(int E, int N1, int H, int I) {
  return align_up((size_t)E * weight_amax_parts((long)N1 * H) * 4) +
         align_up((size_t)E * weight_amax_parts((long)H * I) * 4);
}

// routed_moe workspace layout
struct MoeLayout {
  size_t off[PMOE_WS_NUM_FIELDS];
  size_t rank_local, block_counts, tiles, acc32, xq, x_sf, x_scale, xpad;
  size_t total;
  int max_tiles;
};

MoeLayout moe_layout(int T, int K, int E, int H, int I) {
  MoeLayout L;
  const size_t TK = (size_t)T * K;
  const size_t Hp = padded_k(H), Ip = padded_k(I);
  L.max_tiles = (int)((TK + kTileM - 1) / kTileM) + E;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.off[PMOE_WS_ROW_OF_ROUTE] = take(TK * 4);
  L.off[PMOE_WS_ROUTE_OF_ROW] = take(TK * 4);
  L.off[PMOE_WS_EXPERT_OFFSETS] = take((size_t)(E + 1) * 4);
  L.off[PMOE_WS_COUNTERS] = take(16);
  // FP32 h [TK, I], or BF16 h [TK, Ip] under W4A16 (FC2's A operand)
  L.off[PMOE_WS_H] = take(std::max(TK * I * 4, TK * Ip * 2));
  L.off[PMOE_WS_HQ] = take(TK * Ip / 2);
  L.off[PMOE_WS_H_SF] = take(TK * Ip / 16);
  L.off[PMOE_WS_H_SCALE] = take(TK * 4);
  L.off[PMOE_WS_Z] = take(TK * H * 2);
  L.rank_local = take(TK * 4);
  L.block_counts = take((size_t)route_blocks((int)TK) * E * 4);
  L.tiles = take((size_t)L.max_tiles * 4 * 4);
  L.acc32 = take((size_t)T * H * 4);
  L.xq = take((size_t)T * Hp / 2);
  L.x_sf = take((size_t)T * Hp / 16);
  L.x_scale = take((size_t)T * 4);
  // BF16 activations re-laid with padded rows (W4A16 when H is not a multiple of 64)
  L.xpad = take(Hp == (size_t)H ? 0 : (size_t)T * Hp * 2);
  L.total = o;
  return L;
}

int check_moe_shape(int T, int K, int E, int H, int I, int act) {
  if (T < 0) return fail(PMOE_ERR_SHAPE, "T must be >= 0");
  if (E < 1 || E > kMaxExperts) return fail(PMOE_ERR_SHAPE, "E must be in [1, 1024]");
  if (K < 1 || K > 32 || K > E) return fail(PMOE_ERR_SHAPE, "K must be in [1, min(32, E)]");
  if (!dim_ok(H)) return fail(PMOE_ERR_SHAPE, "H" PMOE_DIM_RULE);
  if (!dim_ok(I)) return fail(PMOE_ERR_SHAPE, "I" PMOE_DIM_RULE);
  if ((long long)T * K >= (1LL << 31) / 2) return fail(PMOE_ERR_SHAPE, "T*K too large");
  if ((long long)T * padded_k(H) >= (1LL << 31) || (long long)T * K * padded_k(I) >= (1LL << 31))
    return fail(PMOE_ERR_SHAPE, "T*H and T*K*I (H, I rounded up to 64) must stay below 2^31 elements");
  if (act != PMOE_ACT_RELU2 && act != PMOE_ACT_SWIGLU) return fail(PMOE_ERR_ACT, "unknown activation kind");
  return PMOE_OK;
}

}  // namespace

// ================================================================== exports

PMOE_EXPORT int pmoe_version(void) { return 200; }

PMOE_EXPORT const char* pmoe_last_error(void) { return g_last_error.c_str(); }

PMOE_EXPORT int pmoe_weight_bytes(int E, int N1, int H, int I, size_t sizes[4]) {
  if (!sizes) return fail(PMOE_ERR_ARG, "sizes is null");
  PMOE_TRY(check_weight_shape(E, N1, H, I));
  WeightBytes b = weight_bytes(E, N1, H, I);
  sizes[0] = b.w1q;
  sizes[1] = b.w1s;
  sizes[2] = b.w2q;
  sizes[3] = b.w2s;
  return ok();
}

PMOE_EXPORT size_t pmoe_prepare_workspace_bytes(int E, int N1, int H, int I) {
  if (check_weight_shape(E, N1, H, I) != PMOE_OK) return 0;
  ok();
  return prepare_ws(E, N1, H, I);
}

namespace {

int prepare_weights(const void* w1, const void* w2, int E, int N1, int H, int I, const float* a1,
                    const float* a2, void* w1_codes, void* w1_scales, float* w1_alpha,
                    void* w2_codes, void* w2_scales, float* w2_alpha, void* ws, size_t ws_bytes,
                    void* stream) {
  PMOE_TRY(check_weight_shape(E, N1, H, I));
  PMOE_TRY(check_device());
  PMOE_TRY(check_ptr(w1, 16, "w1"));
  PMOE_TRY(check_ptr(w2, 16, "w2"));
  PMOE_TRY(check_ptr(w1_codes, 16, "w1_codes"));
  PMOE_TRY(check_ptr(w1_scales, 16, "w1_scales"));
  PMOE_TRY(check_ptr(w1_alpha, 4, "w1_alpha"));
  PMOE_TRY(check_ptr(w2_codes, 16, "w2_codes"));
  PMOE_TRY(check_ptr(w2_scales, 16, "w2_scales"));
  PMOE_TRY(check_ptr(w2_alpha, 4, "w2_alpha"));
  PMOE_TRY(check_ptr(ws, 16, "ws"));
  if (a1 || a2) {
    PMOE_TRY(check_ptr(a1, 4, "a1_scale"));
    PMOE_TRY(check_ptr(a2, 4, "a2_scale"));
  }
  const size_t need = prepare_ws(E, N1, H, I);
  if (ws_bytes < need)
    return fail(PMOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part1 = static_cast<float*>(ws);
  float* part2 = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                          align_up((size_t)E * weight_amax_parts((long)N1 * H) * 4));
  const int gated_I = (N1 == 2 * I) ? I : 0;
  PMOE_HIP(launch_prepare_fc(static_cast<const uint16_t*>(w1), E, N1, H, gated_I, part1, a1,
                             static_cast<uint8_t*>(w1_codes), static_cast<uint8_t*>(w1_scales),
                             w1_alpha, s));
  PMOE_HIP(launch_prepare_fc(static_cast<const uint16_t*>(w2), E, H, I, 0, part2, a2,
                             static_cast<uint8_t*>(w2_codes), static_cast<uint8_t*>(w2_scales),
                             w2_alpha, s));
  return ok();
}

}  // namespace

PMOE_EXPORT int pmoe_prepare_weights(const void* w1, const void* w2, int E, int N1, int H, int I,
                                     void* w1_codes, void* w1_scales, float* w1_alpha,
                                     void* w2_codes, void* w2_scales, float* w2_alpha, void* ws,
                                     size_t ws_bytes, void* stream) {
  return prepare_weights(w1, w2, E, N1, H, I, nullptr, nullptr, w1_codes, w1_scales, w1_alpha,
                         w2_codes, w2_scales, w2_alpha, ws, ws_bytes, stream);
}

PMOE_EXPORT int pmoe_prepare_weights_per_tensor(const void* w1, const void* w2, int E, int N1,
                                                int H, int I, const float* a1_scale,
                                                const float* a2_scale, void* w1_codes,
                                                void* w1_scales, float* w1_alpha, void* w2_codes,
                                                void* w2_scales, float* w2_alpha, void* ws,
                                                size_t ws_bytes, void* stream) {
  if (!a1_scale || !a2_scale) return fail(PMOE_ERR_POINTER, "a1_scale and a2_scale are required");
  return prepare_weights(w1, w2, E, N1, H, I, a1_scale, a2_scale, w1_codes, w1_scales, w1_alpha,
                         w2_codes, w2_scales, w2_alpha, ws, ws_bytes, stream);
}

PMOE_EXPORT int pmoe_quantize_input_per_token(const void* x, int T, int H, void* xq, void* x_sf,
                                              float* x_scale, void* stream) {
  if (T < 0) return fail(PMOE_ERR_SHAPE, "T must be >= 0");
  if (!dim_ok(H)) return fail(PMOE_ERR_SHAPE, "H" PMOE_DIM_RULE);
  if (T == 0) return ok();
  PMOE_TRY(check_device());
  PMOE_TRY(check_ptr(x, 16, "x"));
  PMOE_TRY(check_ptr(xq, 16, "xq"));
  PMOE_TRY(check_ptr(x_sf, 4, "x_sf"));
  PMOE_TRY(check_ptr(x_scale, 4, "x_scale"));
  PMOE_HIP(launch_quantize_bf16(x, T, H, H, nullptr, static_cast<uint8_t*>(xq),
                                static_cast<uint8_t*>(x_sf), x_scale,
                                static_cast<hipStream_t>(stream)));
  return ok();
}

PMOE_EXPORT int pmoe_quantize_input_per_tensor(const void* x, int T, int H, const float* a1_scale,
                                               void* xq, void* x_sf, void* stream) {
  if (T < 0) return fail(PMOE_ERR_SHAPE, "T must be >= 0");
  if (!dim_ok(H)) return fail(PMOE_ERR_SHAPE, "H" PMOE_DIM_RULE);
  if (T == 0) return ok();
  PMOE_TRY(check_device());
  PMOE_TRY(check_ptr(x, 16, "x"));
  PMOE_TRY(check_ptr(a1_scale, 4, "a1_scale"));
  PMOE_TRY(check_ptr(xq, 16, "xq"));
  PMOE_TRY(check_ptr(x_sf, 4, "x_sf"));
  PMOE_HIP(launch_quantize_bf16(x, T, H, H, a1_scale, static_cast<uint8_t*>(xq),
                                static_cast<uint8_t*>(x_sf), nullptr,
                                static_cast<hipStream_t>(stream)));
  return ok();
}

PMOE_EXPORT int pmoe_quantize_rows_f32(const float* h, int R, int L, void* hq, void* h_sf,
                                       float* h_scale, void* stream) {
  if (R < 0) return fail(PMOE_ERR_SHAPE, "R must be >= 0");
  if (!dim_ok(L)) return fail(PMOE_ERR_SHAPE, "L" PMOE_DIM_RULE);
  if (R == 0) return ok();
  PMOE_TRY(check_device());
  PMOE_TRY(check_ptr(h, 16, "h"));
  PMOE_TRY(check_ptr(hq, 16, "hq"));
  PMOE_TRY(check_ptr(h_sf, 4, "h_sf"));
  PMOE_TRY(check_ptr(h_scale, 4, "h_scale"));
  PMOE_HIP(launch_quantize_f32(h, R, nullptr, nullptr, L, L, nullptr, static_cast<uint8_t*>(hq),
                               static_cast<uint8_t*>(h_sf), h_scale, false,
                               static_cast<hipStream_t>(stream)));
  return ok();
}

PMOE_EXPORT size_t pmoe_moe_workspace_bytes(int T, int K, int E, int H, int I, int act) {
  if (check_moe_shape(T, K, E, H, I, act) != PMOE_OK) return 0;
  ok();
  return moe_layout(T, K, E, H, I).total;
}

PMOE_EXPORT int pmoe_moe_workspace_layout(int T, int K, int E, int H, int I, int act,
                                          size_t offsets[PMOE_WS_NUM_FIELDS]) {
  if (!offsets) return fail(PMOE_ERR_ARG, "offsets is null");
  PMOE_TRY(check_moe_shape(T, K, E, H, I, act));
  MoeLayout L = moe_layout(T, K, E, H, I);
  for (int i = 0; i < PMOE_WS_NUM_FIELDS; ++i) offsets[i] = L.off[i];
  return ok();
}

namespace {

enum Recipe { kPerToken = PMOE_RECIPE_PER_TOKEN, kPerTensor = PMOE_RECIPE_PER_TENSOR,
              kW4A16 = PMOE_RECIPE_W4A16 };

// A second stream and three events per device, created on first use and kept
// until the process ends: the two parts of the experts run their FC1 ->
// requant -> FC2 chains concurrently, so each chain's launch tail is filled
// with the other's work, and the one-call forward quantizes its input there
// while the routing runs when the routing needs more than one workgroup
// (otherwise both share one launch on the caller's stream). Default stream
// priority. The mutex keeps each
// call's record / wait pairs together when several host threads enqueue on
// the same device.
struct Aux {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, routed = nullptr;
};
std::mutex g_aux_mu;
Aux g_aux[64];

// True when the second stream may join this call: it is idle with respect to
// graph capture, or it is already part of the capture the caller's stream is
// in (a second call inside the same capture). A second stream held by another
// caller's capture would pull this call's kernels into that graph, so the
// call then runs on the caller's stream alone. Call with g_aux_mu held.
bool aux_usable(const Aux& a, hipStream_t s) {
  hipStreamCaptureStatus st2 = hipStreamCaptureStatusNone, st = hipStreamCaptureStatusNone;
  unsigned long long id2 = 0, id = 0;
  if (hipStreamGetCaptureInfo(a.s2, &st2, &id2) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (st2 == hipStreamCaptureStatusNone) return true;
  if (hipStreamGetCaptureInfo(s, &st, &id) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return st == hipStreamCaptureStatusActive && st2 == hipStreamCaptureStatusActive && id == id2;
}

// The current device's Aux, created on first use. Call with g_aux_mu held.
// Either all four objects exist afterwards or none is kept (a failed
// creation is reported and retried on the next call).
int aux_for_current_device(Aux** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(PMOE_ERR_DEVICE, "no usable current device");
  Aux& a = g_aux[dev];
  if (!a.s2) {
    Aux n;
    hipError_t e = hipStreamCreateWithFlags(&n.s2, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.routed, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (n.routed) (void)hipEventDestroy(n.routed);
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s2) (void)hipStreamDestroy(n.s2);
      return fail(PMOE_ERR_HIP, std::string("creating the second stream: ") + hipGetErrorString(e));
    }
    a = n;
  }
  *out = &a;
  return PMOE_OK;
}

// ------------------------------------------------------------------ static scratch
// The workspace of pmoe_routed_moe_static, for callers that cannot allocate
// device memory: one file-scope device array, which every device the library
// runs on holds (its own copy, at its own address) until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress, looked up once per device
// on the entry point's first call there (with that device current) and kept.
constexpr size_t kScratchBytes = PMOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[64];  // device address of `scratch` per device, null until looked up

int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(PMOE_ERR_DEVICE, "no usable current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(PMOE_ERR_HIP, std::string("looking up the static scratch: ") + hipGetErrorString(e));
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return PMOE_OK;
}

// Steps first..last of the routed path under one recipe.
//   per-token : x = xq, x_sf, x_scale (per-token NVFP4); requant per row.
//   per-tensor: x = xq, x_sf (static scale folded into the alphas); x_scale
//               null; the intermediate is quantized with the static a2.
//   W4A16     : x = BF16 activations; FC1 writes BF16 h, FC2 reads it.
// fused: the order-free finalize inside FC2 (FP32 atomics) instead of the
// fixed-order one; swiglu_limit > 0 clamps the SwiGLU inputs.
int moe_path(Recipe rc, int first, int last, const void* x, const void* x_sf, const float* x_scale,
             const float* a2, const void* topk_ids, int ids_type, const float* topk_w, int T, int K,
             int E, int H, int I, int N1, int expert_offset, const void* w1_codes,
             const void* w1_scales, const float* w1_alpha, const void* w2_codes,
             const void* w2_scales, const float* w2_alpha, int act, void* ws, size_t ws_bytes,
             void* out, void* stream, bool fused = false, float swiglu_limit = 0.0f,
             int streams = 0, bool bf16_input = false, const float* a1 = nullptr,
             void* const* step_events = nullptr, bool static_ws = false) {
  if (first < PMOE_STEP_ROUTE || last > PMOE_STEP_FINALIZE || first > last)
    return fail(PMOE_ERR_ARG, "need 0 <= first <= last <= 4");
  if (!(swiglu_limit >= 0.0f)) return fail(PMOE_ERR_ARG, "swiglu_limit must be >= 0");
  PMOE_TRY(check_moe_shape(T, K, E, H, I, act));
  if (N1 != I && N1 != 2 * I) return fail(PMOE_ERR_SHAPE, "FC1 width N1 must be I or 2*I");
  if ((N1 == 2 * I) != (act == PMOE_ACT_SWIGLU))
    return fail(PMOE_ERR_ACT, act == PMOE_ACT_SWIGLU ? "SwiGLU needs a gated FC1 (N1 == 2*I)"
                                                      : "squared ReLU needs a non-gated FC1 (N1 == I)");
  if (ids_type != PMOE_IDS_INT32 && ids_type != PMOE_IDS_INT64)
    return fail(PMOE_ERR_ARG, "ids_type must be PMOE_IDS_INT32 or PMOE_IDS_INT64");
  const int Hp = padded_k(H), Ip = padded_k(I);
  if (rc == kW4A16 && (2LL * T * Hp >= (1LL << 31) || 2LL * T * K * Ip >= (1LL << 31)))
    return fail(PMOE_ERR_SHAPE, "W4A16: 2*T*H and 2*T*K*I (H, I rounded up to 64) must stay below 2^31");
  if (T == 0) return ok();
  PMOE_TRY(check_device());
  if (bf16_input && (first != PMOE_STEP_ROUTE || last != PMOE_STEP_FINALIZE))
    return fail(PMOE_ERR_ARG, "BF16 input runs the whole path");
  if (rc == kW4A16 || bf16_input) {
    PMOE_TRY(check_ptr(x, 16, "x"));
  } else {
    PMOE_TRY(check_ptr(x, 16, "xq"));
    PMOE_TRY(check_ptr(x_sf, 4, "x_sf"));
  }
  if (rc == kPerToken && !bf16_input) PMOE_TRY(check_ptr(x_scale, 4, "x_scale"));
  if (rc == kPerTensor && bf16_input) PMOE_TRY(check_ptr(a1, 4, "a1_scale"));
  if (rc == kPerTensor) PMOE_TRY(check_ptr(a2, 4, "a2_scale"));
  PMOE_TRY(check_ptr(topk_ids, ids_type == PMOE_IDS_INT64 ? 8 : 4, "topk_ids"));
  PMOE_TRY(check_ptr(topk_w, 4, "topk_w"));
  PMOE_TRY(check_ptr(w1_codes, 16, "w1_codes"));
  PMOE_TRY(check_ptr(w1_scales, 16, "w1_scales"));
  PMOE_TRY(check_ptr(w1_alpha, 4, "w1_alpha"));
  PMOE_TRY(check_ptr(w2_codes, 16, "w2_codes"));
  PMOE_TRY(check_ptr(w2_scales, 16, "w2_scales"));
  PMOE_TRY(check_ptr(w2_alpha, 4, "w2_alpha"));
  if (!static_ws) PMOE_TRY(check_ptr(ws, 256, "ws"));  // the static scratch is known good
  PMOE_TRY(check_ptr(out, 16, "out"));
  const MoeLayout L = moe_layout(T, K, E, H, I);
  if (ws_bytes < L.total)
    return fail(PMOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  const int TK = T * K;
  char* base = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);

  RouteBuffers rb;
  rb.rank_local = reinterpret_cast<int*>(base + L.rank_local);
  rb.block_counts = reinterpret_cast<int*>(base + L.block_counts);
  rb.expert_offsets = reinterpret_cast<int*>(base + L.off[PMOE_WS_EXPERT_OFFSETS]);
  rb.tiles = reinterpret_cast<int*>(base + L.tiles);
  rb.counters = reinterpret_cast<int*>(base + L.off[PMOE_WS_COUNTERS]);
  rb.row_of_route = reinterpret_cast<int*>(base + L.off[PMOE_WS_ROW_OF_ROUTE]);
  rb.route_of_row = reinterpret_cast<int*>(base + L.off[PMOE_WS_ROUTE_OF_ROW]);
  auto run = [&](int step) { return first <= step && step <= last; };
  float* acc32 = reinterpret_cast<float*>(base + L.acc32);
  const bool fill_acc = fused && run(PMOE_STEP_FC2);
  const bool quant_in = bf16_input && rc != kW4A16;
  // Two streams for the whole FC1..FC2 range when asked (streams == 2) or by
  // default (streams == 0) once there is enough work to fill the GPU twice.
  bool split = first <= PMOE_STEP_FC1 && last >= PMOE_STEP_FC2 && E >= 2 &&
               (streams == 2 || (streams == 0 && TK >= 2048));
  // One lock for the whole enqueue when the second stream is used, so that the
  // record / wait pairs of concurrent host threads do not interleave.
  std::unique_lock<std::mutex> lock(g_aux_mu, std::defer_lock);
  Aux* aux = nullptr;
  if ((quant_in && !route_quantize_fits(TK)) || split) {
    lock.lock();
    PMOE_TRY(aux_for_current_device(&aux));
    if (!aux_usable(*aux, s)) {  // captured elsewhere: everything on the caller's stream
      aux = nullptr;
      split = false;
    }
  }
  auto record = [&](int i, hipStream_t st) -> int {
    if (step_events && step_events[i]) PMOE_HIP(hipEventRecord(static_cast<hipEvent_t>(step_events[i]), st));
    return PMOE_OK;
  };
  bool s2_after_route = false;  // the second stream already follows the routing
  if (quant_in && route_quantize_fits(TK)) {
    // route and quantize the BF16 activations in one launch on the caller's
    // stream: FC1 can follow on the same stream with no cross-stream wait
    uint8_t* wq = reinterpret_cast<uint8_t*>(base + L.xq);
    uint8_t* wsf = reinterpret_cast<uint8_t*>(base + L.x_sf);
    float* wsc = reinterpret_cast<float*>(base + L.x_scale);
    PMOE_HIP(launch_route_quantize(topk_ids, ids_type == PMOE_IDS_INT64, TK, E, expert_offset, rb, x,
                                   T, H, Hp, rc == kPerTensor ? a1 : nullptr, wq, wsf, wsc, s));
    if (fill_acc) PMOE_HIP(launch_fill_zero(acc32, (long)T * H, s));
    x = wq;
    x_sf = wsf;
    x_scale = rc == kPerToken ? wsc : nullptr;
  } else if (quant_in && !aux) {
    // the second stream is not available: quantize, then route, on the caller's stream
    uint8_t* wq = reinterpret_cast<uint8_t*>(base + L.xq);
    uint8_t* wsf = reinterpret_cast<uint8_t*>(base + L.x_sf);
    float* wsc = reinterpret_cast<float*>(base + L.x_scale);
    PMOE_HIP(launch_quantize_bf16(x, T, H, Hp, rc == kPerTensor ? a1 : nullptr, wq, wsf, wsc, s));
    PMOE_HIP(launch_route(topk_ids, ids_type == PMOE_IDS_INT64, TK, E, expert_offset, rb, s));
    if (fill_acc) PMOE_HIP(launch_fill_zero(acc32, (long)T * H, s));
    x = wq;
    x_sf = wsf;
    x_scale = rc == kPerToken ? wsc : nullptr;
  } else if (quant_in) {
    // quantize the BF16 activations on the second stream while routing runs
    // on the caller's; each stream then waits for the other's part
    uint8_t* wq = reinterpret_cast<uint8_t*>(base + L.xq);
    uint8_t* wsf = reinterpret_cast<uint8_t*>(base + L.x_sf);
    float* wsc = reinterpret_cast<float*>(base + L.x_scale);
    PMOE_HIP(hipEventRecord(aux->fork, s));
    PMOE_HIP(hipStreamWaitEvent(aux->s2, aux->fork, 0));
    PMOE_HIP(launch_quantize_bf16(x, T, H, Hp, rc == kPerTensor ? a1 : nullptr, wq, wsf, wsc, aux->s2));
    PMOE_HIP(launch_route(topk_ids, ids_type == PMOE_IDS_INT64, TK, E, expert_offset, rb, s));
    if (fill_acc) PMOE_HIP(launch_fill_zero(acc32, (long)T * H, s));
    if (split) {
      PMOE_HIP(hipEventRecord(aux->routed, s));
      PMOE_HIP(hipStreamWaitEvent(aux->s2, aux->routed, 0));
      s2_after_route = true;
    }
    PMOE_HIP(hipEventRecord(aux->join, aux->s2));
    PMOE_HIP(hipStreamWaitEvent(s, aux->join, 0));
    x = wq;
    x_sf = wsf;
    x_scale = rc == kPerToken ? wsc : nullptr;
  } else {
    if (run(PMOE_STEP_ROUTE))
      PMOE_HIP(launch_route(topk_ids, ids_type == PMOE_IDS_INT64, TK, E, expert_offset, rb, s));
    if (fill_acc) PMOE_HIP(launch_fill_zero(acc32, (long)T * H, s));
    if (Hp != H && run(PMOE_STEP_FC1)) {
      // canonical FC1 input rows re-laid with zero-padded rows of Hp elements
      if (rc == kW4A16) {
        void* xp = base + L.xpad;
        PMOE_HIP(launch_pad_rows(x, T, 2L * H, 2L * Hp, xp, s));
        x = xp;
      } else {
        uint8_t* wq = reinterpret_cast<uint8_t*>(base + L.xq);
        uint8_t* wsf = reinterpret_cast<uint8_t*>(base + L.x_sf);
        PMOE_HIP(launch_pad_rows(x, T, H / 2, Hp / 2, wq, s));
        PMOE_HIP(launch_pad_rows(x_sf, T, H / 16, Hp / 16, wsf, s));
        x = wq;
        x_sf = wsf;
      }
    }
  }

  void* h = base + L.off[PMOE_WS_H];  // FP32 h, or BF16 h under W4A16
  uint8_t* hq = reinterpret_cast<uint8_t*>(base + L.off[PMOE_WS_HQ]);
  uint8_t* h_sf = reinterpret_cast<uint8_t*>(base + L.off[PMOE_WS_H_SF]);
  float* h_scale = reinterpret_cast<float*>(base + L.off[PMOE_WS_H_SCALE]);
  uint16_t* z = reinterpret_cast<uint16_t*>(base + L.off[PMOE_WS_Z]);
  const bool bf16_a = rc == kW4A16;

  FcParams p1;
  p1.a_codes = static_cast<const uint8_t*>(x);
  p1.a_sf = static_cast<const uint8_t*>(x_sf);
  p1.a_rows = T;
  p1.a_bf16 = bf16_a;
  p1.a_scale = rc == kPerToken ? x_scale : nullptr;
  p1.route_of_row = rb.route_of_row;
  p1.topk = K;
  p1.w_codes = static_cast<const uint8_t*>(w1_codes);
  p1.w_scales = static_cast<const uint8_t*>(w1_scales);
  p1.w_alpha = w1_alpha;
  p1.NB = col_blocks(N1, act == PMOE_ACT_SWIGLU ? I : 0);
  p1.KC = Hp / kChunk;
  p1.tiles = rb.tiles;
  p1.counters = rb.counters;
  p1.max_tiles = L.max_tiles;
  p1.out = h;
  // FP32 h keeps canonical rows for the requant; BF16 h (W4A16) is FC2's A
  // operand, so its rows are padded to Ip (the padding columns compute to 0)
  p1.out_stride = bf16_a ? Ip : I;
  p1.n_out = bf16_a ? Ip : I;
  p1.swiglu_limit = swiglu_limit;
  p1.out_route = nullptr;
  p1.out_w = nullptr;
  p1.part = 0;

  FcParams p2 = p1;
  p2.a_codes = bf16_a ? static_cast<const uint8_t*>(h) : hq;
  p2.a_sf = h_sf;
  p2.a_rows = TK;
  p2.a_scale = rc == kPerToken ? h_scale : nullptr;
  p2.route_of_row = nullptr;
  p2.w_codes = static_cast<const uint8_t*>(w2_codes);
  p2.w_scales = static_cast<const uint8_t*>(w2_scales);
  p2.w_alpha = w2_alpha;
  p2.NB = col_blocks(H, 0);
  p2.KC = Ip / kChunk;
  p2.out = z;
  p2.out_stride = H;
  p2.n_out = H;
  if (fused) {
    p2.out = acc32;
    p2.out_route = rb.route_of_row;
    p2.out_w = topk_w;
  }
  const FcMode m1 = act == PMOE_ACT_SWIGLU ? kFc1Swiglu : kFc1Relu2;
  const FcMode m2 = fused ? kFc2Fused : kFc2;
  const float* static_a2 = rc == kPerTensor ? a2 : nullptr;

  // FC1 -> requant -> FC2 of one part of the experts on one stream.
  auto chain = [&](int part, hipStream_t st, bool fc1, bool requant, bool fc2) -> int {
    FcParams q1 = p1, q2 = p2;
    q1.part = q2.part = part;
    const int* row_begin = part == 2 ? rb.counters + 3 : nullptr;
    const int* row_end = part == 1 ? rb.counters + 3 : rb.counters;
    // timing events: part 1 (or the whole set) at 0, 1 (FC1) and 4, 5 (FC2);
    // part 2 at 2, 3 and 6, 7; one part alone records both pairs
    const int e0 = part == 2 ? 2 : 0;
    if (fc1) {
      PMOE_TRY(record(e0, st));
      if (part == 0) PMOE_TRY(record(2, st));
      PMOE_HIP(launch_fc(m1, q1, st));
      PMOE_TRY(record(e0 + 1, st));
      if (part == 0) PMOE_TRY(record(3, st));
    }
    if (requant && rc != kW4A16)
      PMOE_HIP(launch_quantize_f32(static_cast<const float*>(h), TK, row_begin, row_end, I, Ip,
                                   static_a2, hq, h_sf, h_scale, part != 0, st));
    if (fc2) {
      PMOE_TRY(record(e0 + 4, st));
      if (part == 0) PMOE_TRY(record(6, st));
      PMOE_HIP(launch_fc(m2, q2, st));
      PMOE_TRY(record(e0 + 5, st));
      if (part == 0) PMOE_TRY(record(7, st));
    }
    return PMOE_OK;
  };
  if (split) {
    if (!s2_after_route) {
      PMOE_HIP(hipEventRecord(aux->fork, s));
      PMOE_HIP(hipStreamWaitEvent(aux->s2, aux->fork, 0));
    }
    PMOE_TRY(chain(1, s, true, true, true));
    PMOE_TRY(chain(2, aux->s2, true, true, true));
    PMOE_HIP(hipEventRecord(aux->join, aux->s2));
    PMOE_HIP(hipStreamWaitEvent(s, aux->join, 0));
  } else {
    PMOE_TRY(chain(0, s, run(PMOE_STEP_FC1), run(PMOE_STEP_REQUANT), run(PMOE_STEP_FC2)));
  }

  if (run(PMOE_STEP_FINALIZE)) {
    if (fused)
      PMOE_HIP(launch_f32_to_bf16(acc32, (long)T * H, static_cast<uint16_t*>(out), s));
    else
      PMOE_HIP(launch_finalize(z, rb.row_of_route, topk_w, T, K, H, static_cast<uint16_t*>(out), s));
  }
  return ok();
}

}  // namespace

PMOE_EXPORT int pmoe_routed_moe_steps(int first, int last, const void* xq, const void* x_sf,
                                      const float* x_scale, const void* topk_ids, int ids_type,
                                      const float* topk_w, int T, int K, int E, int H, int I, int N1,
                                      int expert_offset, const void* w1_codes,
                                      const void* w1_scales, const float* w1_alpha,
                                      const void* w2_codes, const void* w2_scales,
                                      const float* w2_alpha, int act, void* ws, size_t ws_bytes,
                                      void* out, void* stream) {
  return moe_path(kPerToken, first, last, xq, x_sf, x_scale, nullptr, topk_ids, ids_type, topk_w, T,
                  K, E, H, I, N1, expert_offset, w1_codes, w1_scales, w1_alpha, w2_codes, w2_scales,
                  w2_alpha, act, ws, ws_bytes, out, stream);
}

PMOE_EXPORT int pmoe_routed_moe(const void* xq, const void* x_sf, const float* x_scale,
                                const void* topk_ids, int ids_type, const float* topk_w, int T,
                                int K, int E, int H, int I, int N1, int expert_offset,
                                const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                                const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                                int act, void* ws, size_t ws_bytes, void* out, void* stream) {
  return moe_path(kPerToken, PMOE_STEP_ROUTE, PMOE_STEP_FINALIZE, xq, x_sf, x_scale, nullptr,
                  topk_ids, ids_type, topk_w, T, K, E, H, I, N1, expert_offset, w1_codes, w1_scales,
                  w1_alpha, w2_codes, w2_scales, w2_alpha, act, ws, ws_bytes, out, stream);
}

PMOE_EXPORT int pmoe_routed_moe_static(const void* xq, const void* x_sf, const float* x_scale,
                                       const void* topk_ids, int ids_type, const float* topk_w,
                                       int T, int K, int E, int H, int I, int N1,
                                       int expert_offset, const void* w1_codes,
                                       const void* w1_scales, const float* w1_alpha,
                                       const void* w2_codes, const void* w2_scales,
                                       const float* w2_alpha, int act, void* out, void* stream) {
  PMOE_TRY(check_moe_shape(T, K, E, H, I, act));
  const size_t need = moe_layout(T, K, E, H, I).total;
  if (need > kScratchBytes)
    return fail(PMOE_ERR_WORKSPACE, "pmoe_routed_moe_static: these sizes need " + std::to_string(need) +
                                        " bytes of scratch; the static scratch holds " +
                                        std::to_string(kScratchBytes) +
                                        " (PMOE_STATIC_SCRATCH_BYTES): use pmoe_routed_moe with a workspace");
  if (T == 0) return ok();
  PMOE_TRY(check_device());
  void* ws = nullptr;
  PMOE_TRY(scratch_for_current_device(&ws));
  // one stream: no library stream or event is created or used
  return moe_path(kPerToken, PMOE_STEP_ROUTE, PMOE_STEP_FINALIZE, xq, x_sf, x_scale, nullptr, topk_ids,
                  ids_type, topk_w, T, K, E, H, I, N1, expert_offset, w1_codes, w1_scales, w1_alpha,
                  w2_codes, w2_scales, w2_alpha, act, ws, kScratchBytes, out, stream, false, 0.0f, 1,
                  false, nullptr, nullptr, true);
}

PMOE_EXPORT int pmoe_routed_moe_per_tensor(const void* xq, const void* x_sf, const void* topk_ids,
                                           int ids_type, const float* topk_w, int T, int K, int E,
                                           int H, int I, int N1, int expert_offset,
                                           const void* w1_codes, const void* w1_scales,
                                           const float* w1_alpha, const void* w2_codes,
                                           const void* w2_scales, const float* w2_alpha,
                                           const float* a2_scale, int act, void* ws,
                                           size_t ws_bytes, void* out, void* stream) {
  return moe_path(kPerTensor, PMOE_STEP_ROUTE, PMOE_STEP_FINALIZE, xq, x_sf, nullptr, a2_scale,
                  topk_ids, ids_type, topk_w, T, K, E, H, I, N1, expert_offset, w1_codes, w1_scales,
                  w1_alpha, w2_codes, w2_scales, w2_alpha, act, ws, ws_bytes, out, stream);
}

PMOE_EXPORT int pmoe_routed_moe_ex(const void* x, const void* x_sf, const float* x_scale,
                                   const void* topk_ids, int ids_type, const float* topk_w, int T,
                                   int K, int E, int H, int I, int N1, int expert_offset,
                                   const void* w1_codes, const void* w1_scales,
                                   const float* w1_alpha, const void* w2_codes,
                                   const void* w2_scales, const float* w2_alpha, int act,
                                   const pmoe_moe_options* options, void* ws, size_t ws_bytes,
                                   void* out, void* stream) {
  pmoe_moe_options o = {PMOE_RECIPE_PER_TOKEN, PMOE_FINALIZE_ORDERED, 0.0f, nullptr, 0, nullptr, nullptr};
  if (options) o = *options;
  if (o.recipe != PMOE_RECIPE_PER_TOKEN && o.recipe != PMOE_RECIPE_PER_TENSOR &&
      o.recipe != PMOE_RECIPE_W4A16)
    return fail(PMOE_ERR_ARG, "unknown recipe");
  if (o.finalize != PMOE_FINALIZE_ORDERED && o.finalize != PMOE_FINALIZE_FUSED)
    return fail(PMOE_ERR_ARG, "unknown finalize mode");
  if (o.swiglu_limit != 0.0f && act != PMOE_ACT_SWIGLU)
    return fail(PMOE_ERR_ARG, "swiglu_limit needs the SwiGLU activation");
  if (o.recipe != PMOE_RECIPE_PER_TENSOR && o.a2_scale)
    return fail(PMOE_ERR_ARG, "a2_scale belongs to the per-tensor recipe");
  if (o.streams < 0 || o.streams > 2) return fail(PMOE_ERR_ARG, "streams must be 0, 1 or 2");
  if (o.a1_scale) return fail(PMOE_ERR_ARG, "a1_scale belongs to pmoe_moe_forward");
  const Recipe rc = static_cast<Recipe>(o.recipe);
  return moe_path(rc, PMOE_STEP_ROUTE, PMOE_STEP_FINALIZE, x, x_sf,
                  rc == kPerToken ? x_scale : nullptr, o.a2_scale, topk_ids, ids_type, topk_w, T, K,
                  E, H, I, N1, expert_offset, w1_codes, w1_scales, w1_alpha, w2_codes, w2_scales,
                  w2_alpha, act, ws, ws_bytes, out, stream, o.finalize == PMOE_FINALIZE_FUSED,
                  o.swiglu_limit, o.streams, false, nullptr, o.step_events);
}

PMOE_EXPORT int pmoe_moe_forward(const void* x, const void* topk_ids, int ids_type,
                                 const float* topk_w, int T, int K, int E, int H, int I, int N1,
                                 int expert_offset, const void* w1_codes, const void* w1_scales,
                                 const float* w1_alpha, const void* w2_codes,
                                 const void* w2_scales, const float* w2_alpha, int act,
                                 const pmoe_moe_options* options, void* ws, size_t ws_bytes,
                                 void* out, void* stream) {
  pmoe_moe_options o = {PMOE_RECIPE_PER_TOKEN, PMOE_FINALIZE_ORDERED, 0.0f, nullptr, 0, nullptr, nullptr};
  if (options) o = *options;
  if (o.recipe != PMOE_RECIPE_PER_TOKEN && o.recipe != PMOE_RECIPE_PER_TENSOR &&
      o.recipe != PMOE_RECIPE_W4A16)
    return fail(PMOE_ERR_ARG, "unknown recipe");
  if (o.finalize != PMOE_FINALIZE_ORDERED && o.finalize != PMOE_FINALIZE_FUSED)
    return fail(PMOE_ERR_ARG, "unknown finalize mode");
  if (o.swiglu_limit != 0.0f && act != PMOE_ACT_SWIGLU)
    return fail(PMOE_ERR_ARG, "swiglu_limit needs the SwiGLU activation");
  if (o.recipe != PMOE_RECIPE_PER_TENSOR && (o.a1_scale || o.a2_scale))
    return fail(PMOE_ERR_ARG, "a1_scale and a2_scale belong to the per-tensor recipe");
  if (o.streams < 0 || o.streams > 2) return fail(PMOE_ERR_ARG, "streams must be 0, 1 or 2");
  const Recipe rc = static_cast<Recipe>(o.recipe);
  return moe_path(rc, PMOE_STEP_ROUTE, PMOE_STEP_FINALIZE, x, nullptr, nullptr, o.a2_scale, topk_ids,
                  ids_type, topk_w, T, K, E, H, I, N1, expert_offset, w1_codes, w1_scales, w1_alpha,
                  w2_codes, w2_scales, w2_alpha, act, ws, ws_bytes, out, stream,
                  o.finalize == PMOE_FINALIZE_FUSED, o.swiglu_limit, o.streams, true, o.a1_scale,
                  o.step_events);
}

PMOE_EXPORT int pmoe_router_topk(const float* logits, int T, int E, int K, int renormalize,
                                 int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0) return fail(PMOE_ERR_SHAPE, "T must be >= 0");
  if (E < 1 || E > kMaxExperts) return fail(PMOE_ERR_SHAPE, "E must be in [1, 1024]");
  if (K < 1 || K > 32 || K > E) return fail(PMOE_ERR_SHAPE, "K must be in [1, min(32, E)]");
  if (renormalize != 0 && renormalize != 1) return fail(PMOE_ERR_ARG, "renormalize must be 0 or 1");
  if (T == 0) return ok();
  PMOE_TRY(check_device());
  PMOE_TRY(check_ptr(logits, 4, "logits"));
  PMOE_TRY(check_ptr(topk_ids, 4, "topk_ids"));
  PMOE_TRY(check_ptr(topk_w, 4, "topk_w"));
  PMOE_HIP(launch_router_topk(logits, T, E, K, renormalize, topk_ids, topk_w,
                              static_cast<hipStream_t>(stream)));
  return ok();
}

PMOE_EXPORT int pmoe_routed_moe_w4a16(const void* x, const void* topk_ids, int ids_type,
                                      const float* topk_w, int T, int K, int E, int H, int I, int N1,
                                      int expert_offset, const void* w1_codes,
                                      const void* w1_scales, const float* w1_alpha,
                                      const void* w2_codes, const void* w2_scales,
                                      const float* w2_alpha, int act, void* ws, size_t ws_bytes,
                                      void* out, void* stream) {
  return moe_path(kW4A16, PMOE_STEP_ROUTE, PMOE_STEP_FINALIZE, x, nullptr, nullptr, nullptr,
                  topk_ids, ids_type, topk_w, T, K, E, H, I, N1, expert_offset, w1_codes, w1_scales,
                  w1_alpha, w2_codes, w2_scales, w2_alpha, act, ws, ws_bytes, out, stream);
}

PMOE_EXPORT int pmoe_finalize(const void* z, const int32_t* row_of_route, const float* topk_w, int T,
                              int K, int H, void* out, void* stream) {
  if (T < 0 || K < 1 || K > 32) return fail(PMOE_ERR_SHAPE, "need T >= 0 and 1 <= K <= 32");
  if (H <= 0 || H % 8 != 0) return fail(PMOE_ERR_SHAPE, "H must be a positive multiple of 8");
  if (T == 0) return ok();
  PMOE_TRY(check_device());
  PMOE_TRY(check_ptr(z, 16, "z"));
  PMOE_TRY(check_ptr(row_of_route, 4, "row_of_route"));
  PMOE_TRY(check_ptr(topk_w, 4, "topk_w"));
  PMOE_TRY(check_ptr(out, 16, "out"));
  PMOE_HIP(launch_finalize(static_cast<const uint16_t*>(z), row_of_route, topk_w, T, K, H,
                           static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
  return ok();
}
