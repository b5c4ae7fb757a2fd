/*
 * pmoe -- per-token NVFP4 routed-MoE expert path for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every compute entry point enqueues HIP kernels on the caller's stream
 * (`stream` is a hipStream_t; NULL means the legacy default stream), returns a
 * status code, and never allocates device memory, synchronizes, or aborts.
 * The routed-MoE entry points may also enqueue work on one library-owned
 * stream per device (created on first use, default priority, kept until the
 * process ends), forked from and joined back into the caller's stream with
 * events, so the call stays ordered on the caller's stream and can be captured
 * in a graph.
 * All tensors are caller-owned device buffers (the library keeps no pointer to
 * them after the call returns and caches nothing about them). All checks run on
 * the host before the first launch; when a call returns an error, no kernel was
 * launched and no output was touched (PMOE_ERR_HIP is the one exception: it
 * reports a failed launch after validation passed).
 *
 * Sources of the contract (three public pages):
 *   [Megatron-LM #8262]  per-token NVFP4 squared-ReLU and SwiGLU MoE via FlashInfer
 *                        CuTe DSL (sections: Background, What is added, How to extend,
 *                        What is tested).
 *   [FlashInfer #5019]   CuTe DSL NVFP4 W4A16 MegaMoE (section: Tensor and numerical
 *                        contract).
 *
 * Notation: T tokens, H hidden size, I intermediate size, E local experts,
 * K top-k, N1 = FC1 output width (2*I gated / SwiGLU, I non-gated / squared ReLU),
 * R = number of valid routes (at most T*K).
 *
 * Number formats (NVFP4): E2M1 codes packed two per byte, element 2i in the low
 * nibble; one E4M3 (fn, max 448) block scale per 16 consecutive elements along
 * the reduction dimension; one FP32 scale per token (activations) or per expert
 * (weights, "alpha") [Megatron-LM #8262 . Background; FlashInfer #5019 . Tensor
 * and numerical contract]. BF16 tensors are passed as raw 16-bit storage.
 *
 * Shape limits of this build: H and I multiples of 16 (one block) in
 * [16, 16384]; 1 <= K <= min(32, E); 1 <= E <= 1024; T >= 0 (T == 0 is a
 * successful no-op); T*Hp and T*K*Ip below 2^31, where Hp and Ip are H and I
 * rounded up to a multiple of 64 (the W4A16 recipe: 2*T*Hp and 2*T*K*Ip). The
 * grouped GEMMs reduce over whole chunks of 64 elements: a reduction length
 * that is not a multiple of 64 is padded inside the library with zero codes
 * and zero block scales, which add exactly zero to every sum; the canonical
 * arrays at this interface are never padded.
 */
#ifndef PMOE_H_
#define PMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define PMOE_OK 0
#define PMOE_ERR_DEVICE 1    /* current device is not gfx950 (MI355X / MI350X)          */
#define PMOE_ERR_POINTER 2   /* null, host, or misaligned pointer                       */
#define PMOE_ERR_SHAPE 3     /* unsupported sizes, or FC1 width neither I nor 2*I         */
#define PMOE_ERR_ACT 4       /* activation kind disagrees with the FC1 shape             */
#define PMOE_ERR_WORKSPACE 5 /* workspace smaller than the queried size                  */
#define PMOE_ERR_HIP 6       /* a HIP runtime call or kernel launch failed               */
#define PMOE_ERR_ARG 7       /* any other invalid argument (unknown enum value, ...)     */

/* Activation kinds. Squared ReLU is the non-gated expert, SwiGLU the gated one;
 * SwiGLU iff FC1 has twice FC2's input width [Megatron-LM #8262 . What is added]. */
#define PMOE_ACT_RELU2 0
#define PMOE_ACT_SWIGLU 1

/* Element type of topk_ids: signed 32- or 64-bit [FlashInfer #5019 . Tensor and
 * numerical contract, 'Inputs/output']. */
#define PMOE_IDS_INT32 0
#define PMOE_IDS_INT64 1

/* Library version (major*10000 + minor*100 + patch). */
int pmoe_version(void);

/* Message of the last error returned on this host thread: "" after a call
 * that succeeded. The pointer stays valid until the next pmoe call on the
 * same thread. */
const char* pmoe_last_error(void);

/* ============================================================ prepared weights
 *
 * Prepared (kernel-native) layout of one FC matrix with logical shape
 * [E, N, Kd] (N output rows, Kd the reduction length; FC1: N = N1, Kd = H;
 * FC2: N = H, Kd = I). Rows are grouped in blocks of 32 ("col blocks" p,
 * NB = ceil(N/32), or 2*ceil(I/32) for a gated FC1; padded with all-zero
 * blocks to NBp = NB rounded up to a multiple of 8), blocks in column tiles
 * of 8 (ct = p/8, pos = p%8, NT = NBp/8), and the reduction in chunks of 64
 * (c, KC = ceil(Kd/64); the elements in [Kd, 64*KC) are zero). Rows of a block
 * past the matrix (past I in each half of a gated FC1) are zero. Chunk c of a column tile --
 * all 8 of its blocks -- is one contiguous slab, so a GEMM workgroup owning
 * the tile streams a single sequential region:
 *
 *   codes  (uint8, E*NBp*32*Kd/2 bytes): byte offset
 *            (((((e*NT + ct)*KC + c)*8 + pos)*64 + lane)*16 + (2*h + s)*4 + i/2
 *          holds element k = c*64 + 32*s + 8*(lane/16) + i (nibble i%2, low first)
 *          of row n(p, 16*h + lane%16), for h, s in 0..1, i in 0..7 (the operand
 *          order of a 16x16x32 MFMA: lane = column, 8 consecutive k per lane).
 *   scales (uint8, E*NBp*32*Kd/16 bytes): byte offset
 *            ((((e*NT + ct)*KC + c)*8 + pos)*32 + d)*4 + 2*h + s
 *          holds the E4M3 scale of 16-block (c*4 + 2*s + d/16) of row
 *          n(p, 16*h + d%16), for d in 0..31.
 *   alpha  (float32, E values).
 *
 * Row map n(p, col): non-gated FC1 and FC2: n = 32*p + col. Gated FC1 (N1 = 2I)
 * interleaves gate and up blocks so one workgroup holds both halves of a SwiGLU
 * output: p even -> gate row 32*(p/2) + col; p odd -> up row I + 32*(p/2) + col
 * (for 32*(p/2) + col < I)
 * (gate rows are [0, I), up rows [I, 2I) of the canonical FC1 [FlashInfer #5019 .
 * Tensor and numerical contract, 'gate-then-up']).
 *
 * The bytes are the canonical codes/scales of the per-expert NVFP4 recipe
 * (packed [E, N, Kd/2], linear scales [E, N, Kd/16]) permuted by this map
 * (padding is zero); no value is changed and alpha is never folded into the
 * block scales.
 */

/* Sizes in bytes of the four prepared arrays: sizes[0] FC1 codes, sizes[1] FC1
 * scales, sizes[2] FC2 codes, sizes[3] FC2 scales (alphas are E floats each).
 * Host only. Returns PMOE_ERR_SHAPE for unsupported sizes. */
int pmoe_weight_bytes(int E, int N1, int H, int I, size_t sizes[4]);

/* Device workspace needed by pmoe_prepare_weights (bytes). 0 on bad shapes. */
size_t pmoe_prepare_workspace_bytes(int E, int N1, int H, int I);

/*
 * Quantize BF16 expert stacks into the prepared NVFP4 layout
 * [Megatron-LM #8262 . What is added, 'prepare_routed_nvfp4_weights'].
 *   w1 : BF16 [E, N1, H], gate rows then up rows when N1 == 2*I.
 *   w2 : BF16 [E, H, I].
 * Per expert and FC: amax over the whole matrix (gate and up together),
 * w_scale = fp32(2688 / amax), alpha = fp32(1 / w_scale); each 16-block gets the
 * E4M3 scale fp32(fp32(amax_b / 6) / alpha) (round to nearest even, saturating
 * at 448) and E2M1 codes of fp32(w / fp32(dec(scale) * alpha)) (round to nearest,
 * ties to the even code, saturating at 6). An all-zero expert gets alpha = 0 and
 * zero bytes.
 * Outputs are written in place, so their addresses stay valid across refreshes
 * (in-place refit) [Megatron-LM #8262 . What is added]. Gating is detected from
 * the shapes: N1 == 2*I gated, N1 == I non-gated, else PMOE_ERR_SHAPE.
 * ws: at least pmoe_prepare_workspace_bytes(...) bytes of device memory.
 * Alignment: every pointer 16-byte aligned.
 */
int pmoe_prepare_weights(const void* w1, const void* w2, int E, int N1, int H, int I,
                         void* w1_codes, void* w1_scales, float* w1_alpha,
                         void* w2_codes, void* w2_scales, float* w2_alpha,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Preparation for the per-tensor NVFP4 recipe [Megatron-LM #8262 . How to
 * extend, 'per_tensor']: codes and block scales exactly as pmoe_prepare_weights,
 * with the static FC1 / FC2 input scales folded into the alphas:
 *   w1_alpha[e] = fp32(1 / fp32(w_scale1[e] * a1)),
 *   w2_alpha[e] = fp32(1 / fp32(w_scale2[e] * a2)).
 *   a1_scale, a2_scale : device float32 scalars (4-byte aligned), read by the
 *                        kernels, so the call never waits on the host. They
 *                        use the weights' convention, a = 2688 / calibrated
 *                        amax, and must be positive and finite (not checked:
 *                        they live on the device).
 * Other arguments, layout and errors as pmoe_prepare_weights.
 */
int pmoe_prepare_weights_per_tensor(const void* w1, const void* w2, int E, int N1, int H, int I,
                                    const float* a1_scale, const float* a2_scale,
                                    void* w1_codes, void* w1_scales, float* w1_alpha,
                                    void* w2_codes, void* w2_scales, float* w2_alpha,
                                    void* ws, size_t ws_bytes, void* stream);

/* ============================================================ activations */

/*
 * Per-token NVFP4 quantization of BF16 activations [Megatron-LM #8262 .
 * Background; What is added, 'quantize_routed_nvfp4_input'; How to extend,
 * 'FC1 input' and 'per_token_scale'].
 *   x       : BF16 [T, H] (row-major, contiguous)
 *   xq      : uint8 [T, H/2] packed E2M1 codes (canonical layout)
 *   x_sf    : uint8 [T, H/16] E4M3 block scales
 *   x_scale : float32 [T] per-token scale
 * Per token: g = fp32(amax * fp32(1/2688)) (the recipe constant 1/(448*6));
 * per 16-block: scale = E4M3(fp32(fp32(amax_b / 6) / g)), codes =
 * E2M1(fp32(x / fp32(dec(scale) * g))); g == 0 (all-zero token) gives zero bytes.
 * Bit-exact IEEE binary32 with denormals. Alignment: xq and x 16 bytes,
 * x_sf 4 bytes, x_scale 4 bytes.
 */
int pmoe_quantize_input_per_token(const void* x, int T, int H,
                                  void* xq, void* x_sf, float* x_scale, void* stream);

/*
 * NVFP4 quantization of BF16 activations with a static, calibrated scale
 * (per-tensor recipe) [Megatron-LM #8262 . How to extend, 'per_tensor', row
 * 'FC1 input']: every row uses g = fp32(1 / a1) in the block steps of
 * pmoe_quantize_input_per_token; blocks beyond the scale's range saturate
 * (scale 448, codes +-6). No per-token scale is produced.
 *   a1_scale : device float32 scalar (a1 = 2688 / calibrated amax), positive and finite
 *   xq, x_sf : as pmoe_quantize_input_per_token.
 */
int pmoe_quantize_input_per_tensor(const void* x, int T, int H, const float* a1_scale,
                                   void* xq, void* x_sf, void* stream);

/*
 * The same per-row NVFP4 quantizer applied to FP32 rows: the requantization of
 * the FP32 expert intermediate before FC2 [Megatron-LM #8262 . How to extend,
 * 'fc2_input_scale'; What is tested, 4. Train-gen parity]. routed_moe runs this
 * quantizer on its intermediate; it is exported so it can be checked alone.
 *   h : float32 [R, L], L a multiple of 16 up to 16384;  hq : uint8 [R, L/2];
 *   h_sf : uint8 [R, L/16];  h_scale : float32 [R].
 */
int pmoe_quantize_rows_f32(const float* h, int R, int L,
                           void* hq, void* h_sf, float* h_scale, void* stream);

/* ============================================================ routed MoE */

/* Device workspace needed by pmoe_routed_moe (bytes). 0 on bad shapes. */
size_t pmoe_moe_workspace_bytes(int T, int K, int E, int H, int I, int act);

/* Fields of the routed_moe workspace, for inspection (offsets in bytes). */
#define PMOE_WS_ROW_OF_ROUTE 0   /* int32 [T*K]   expert-sorted row of route t*K+j, -1 if invalid */
#define PMOE_WS_ROUTE_OF_ROW 1   /* int32 [T*K]   route index of each row (first R valid)        */
#define PMOE_WS_EXPERT_OFFSETS 2 /* int32 [E+1]   first row of each local expert; [E] = R          */
#define PMOE_WS_COUNTERS 3       /* int32 [4]     {R, number of M-tiles, first M-tile and first row
                                    of the experts run on the second stream}                    */
#define PMOE_WS_H 4              /* float32 [T*K, I]   activation output (rows < R valid);
                                    BF16 [T*K, Ip] under pmoe_routed_moe_w4a16 (Ip = I rounded
                                    up to 64; columns past I are 0)                             */
#define PMOE_WS_HQ 5             /* uint8 [T*K, Ip/2]  requantized intermediate codes (past I/2: 0) */
#define PMOE_WS_H_SF 6           /* uint8 [T*K, Ip/16] its E4M3 block scales (past I/16: 0)         */
#define PMOE_WS_H_SCALE 7        /* float32 [T*K]      its per-row scales (per-token recipe only)   */
#define PMOE_WS_Z 8              /* BF16 [T*K, H]      per-route FC2 outputs                         */
#define PMOE_WS_NUM_FIELDS 9

/* Offsets (bytes, from the workspace base) of the fields above. Host only. */
int pmoe_moe_workspace_layout(int T, int K, int E, int H, int I, int act,
                              size_t offsets[PMOE_WS_NUM_FIELDS]);

/*
 * Routed-MoE expert path on per-token-quantized activations: routing, FC1
 * grouped GEMM, activation, per-row requantization, FC2 grouped GEMM, and the
 * deterministic finalize [Megatron-LM #8262 . What is added,
 * 'flashinfer_routed_nvfp4_moe'; FlashInfer #5019 . Tensor and numerical
 * contract, 'Compute order'].
 *   xq, x_sf, x_scale : output of pmoe_quantize_input_per_token for [T, H]
 *   topk_ids          : [T, K] int32 or int64 (ids_type); a route is valid iff
 *                       expert_offset <= id < expert_offset + E, others
 *                       (e.g. -1 fill) contribute nothing
 *   topk_w            : float32 [T, K] routing weights, applied in the finalize
 *   N1                : FC1 width the weights were prepared with (I or 2*I, else
 *                       PMOE_ERR_SHAPE)
 *   weights           : the six prepared arrays of pmoe_prepare_weights
 *   act               : PMOE_ACT_RELU2 (needs N1 == I) or PMOE_ACT_SWIGLU (needs
 *                       N1 == 2*I); a disagreement is PMOE_ERR_ACT
 *   ws                : at least pmoe_moe_workspace_bytes(T, K, E, H, I, act) bytes
 *   out               : BF16 [T, H]
 * Per valid route (token t, expert e), row r:
 *   y = fp32(sum_k dec(xq[t,k]) * dec(W1[e,:,k])) * fp32(x_scale[t] * alpha1[e])
 *   h = max(y,0)^2  or  silu(y_gate) * y_up, in FP32
 *   (hq, h_sf, h_scale) = per-row quantization of h (as pmoe_quantize_rows_f32)
 *   z = bf16(fp32(sum_k dec(hq) * dec(W2[e])) * fp32(h_scale[r] * alpha2[e]))
 * and out[t] = bf16(sum over slots j = 0..K-1 in order of fp32(w[t,j] * z)),
 * accumulated in FP32 from +0 without fused multiply-add. A token with no
 * valid route gets +0. The result of a token depends only on its own inputs
 * (batch invariant): the tiling never depends on T and no split-K is used.
 * Alignment: ws 256 bytes (its fields start on 256-byte boundaries); int64
 * topk_ids 8 bytes, int32 topk_ids, x_scale and topk_w 4 bytes; every other
 * pointer 16 bytes. A misaligned pointer is PMOE_ERR_POINTER. The same rules hold
 * for every entry point below that takes these arguments.
 */
int pmoe_routed_moe(const void* xq, const void* x_sf, const float* x_scale,
                    const void* topk_ids, int ids_type, const float* topk_w,
                    int T, int K, int E, int H, int I, int N1, int expert_offset,
                    const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                    const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                    int act, void* ws, size_t ws_bytes, void* out, void* stream);

/*
 * pmoe_routed_moe for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments without ws / ws_bytes, the same results bit for bit. The
 * workspace is a static device array of PMOE_STATIC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends; the call
 * allocates nothing (no hipMalloc, no library stream or event: everything runs
 * on `stream`). Sizes whose workspace (pmoe_moe_workspace_bytes) exceeds the
 * scratch are PMOE_ERR_WORKSPACE -- at H = 7168, I = 3072 that is about 2300
 * routes (T*K). Every call on one device shares that device's scratch: calls
 * that overlap in time on one device (two streams, two host threads) race and
 * corrupt each other's results; serialize them.
 */
#define PMOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int pmoe_routed_moe_static(const void* xq, const void* x_sf, const float* x_scale,
                           const void* topk_ids, int ids_type, const float* topk_w,
                           int T, int K, int E, int H, int I, int N1, int expert_offset,
                           const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                           const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                           int act, void* out, void* stream);

/* Steps of pmoe_routed_moe, for callers that time or interleave them. */
#define PMOE_STEP_ROUTE 0    /* histogram, scan, tile list, scatter (3 kernels)   */
#define PMOE_STEP_FC1 1      /* FC1 grouped GEMM + activation -> h                */
#define PMOE_STEP_REQUANT 2  /* per-row requantization of h -> hq, h_sf, h_scale  */
#define PMOE_STEP_FC2 3      /* FC2 grouped GEMM -> z                            */
#define PMOE_STEP_FINALIZE 4 /* fixed-order finalize -> out                      */

/*
 * Runs steps first..last (inclusive) of pmoe_routed_moe with the same
 * arguments and workspace; pmoe_routed_moe is steps 0..4. A step reads what the
 * earlier steps left in the workspace, so running the steps one range after
 * another on the same stream gives exactly the result of one full call.
 * PMOE_ERR_ARG unless 0 <= first <= last <= 4.
 */
int pmoe_routed_moe_steps(int first, int last,
                          const void* xq, const void* x_sf, const float* x_scale,
                          const void* topk_ids, int ids_type, const float* topk_w,
                          int T, int K, int E, int H, int I, int N1, int expert_offset,
                          const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                          const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                          int act, void* ws, size_t ws_bytes, void* out, void* stream);

/*
 * The routed path under the per-tensor NVFP4 recipe [Megatron-LM #8262 . How
 * to extend, 'per_tensor']. As pmoe_routed_moe, except:
 *   xq, x_sf   : output of pmoe_quantize_input_per_tensor (no per-token scale)
 *   weights    : output of pmoe_prepare_weights_per_tensor (folded alphas)
 *   a2_scale   : device float32 scalar, the static FC2 input scale
 *   y = fp32(sum_k dec(xq[t,k]) * dec(W1[e,:,k])) * alpha1'[e]
 *   (hq, h_sf) = quantization of h with g = fp32(1 / a2) for every row
 *   z = bf16(fp32(sum_k dec(hq) * dec(W2[e])) * alpha2'[e])
 * The workspace's h_scale field is not written.
 */
int pmoe_routed_moe_per_tensor(const void* xq, const void* x_sf,
                               const void* topk_ids, int ids_type, const float* topk_w,
                               int T, int K, int E, int H, int I, int N1, int expert_offset,
                               const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                               const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                               const float* a2_scale, int act, void* ws, size_t ws_bytes,
                               void* out, void* stream);

/*
 * The routed path with BF16 activations and NVFP4 weights (W4A16, the
 * 'weight_only' recipe) [Megatron-LM #8262 . How to extend, 'weight_only';
 * FlashInfer #5019 . Tensor and numerical contract, 'Compute order'].
 *   x       : BF16 [T, H] activations, not quantized
 *   weights : output of pmoe_prepare_weights (alphas = 1 / w_scale)
 * Per valid route, row r:
 *   y = fp32(sum_k x[t,k] * dec(W1[e,:,k])) * alpha1[e]     (BF16 x BF16 MFMA, FP32 sum)
 *   h = bf16(max(y,0)^2  or  silu(y_gate) * y_up)           (activation in FP32, one rounding)
 *   z = bf16(fp32(sum_k h[r,k] * dec(W2[e,:,k])) * alpha2[e])
 * then the same fixed-order finalize. The workspace's h field holds BF16 h;
 * hq, h_sf and h_scale are not written. Other arguments as pmoe_routed_moe.
 */
int pmoe_routed_moe_w4a16(const void* x, const void* topk_ids, int ids_type, const float* topk_w,
                          int T, int K, int E, int H, int I, int N1, int expert_offset,
                          const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                          const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                          int act, void* ws, size_t ws_bytes, void* out, void* stream);

/* Options of pmoe_routed_moe_ex. */
#define PMOE_RECIPE_PER_TOKEN 0  /* per-token NVFP4 x NVFP4 (x = xq, x_sf, x_scale)        */
#define PMOE_RECIPE_PER_TENSOR 1 /* per-tensor NVFP4 x NVFP4 (x = xq, x_sf; a2_scale)       */
#define PMOE_RECIPE_W4A16 2      /* BF16 x NVFP4 (x = BF16 activations)                     */
#define PMOE_FINALIZE_ORDERED 0  /* fixed slot order, BF16 z per route: batch invariant     */
#define PMOE_FINALIZE_FUSED 1    /* FP32 atomic adds inside FC2: order-free, not invariant  */

typedef struct pmoe_moe_options {
  int recipe;             /* PMOE_RECIPE_*                                                  */
  int finalize;           /* PMOE_FINALIZE_*                                                */
  float swiglu_limit;     /* > 0: SwiGLU clamp, gate <= L and -L <= up <= L; 0: none         */
  const float* a2_scale;  /* per-tensor recipe: device float32 scalar; otherwise NULL       */
  int streams;            /* 0: automatic (two once T*K >= 2048); 1: one stream; 2: the
                             experts are cut at the expert boundary nearest 44 % of the
                             M-tiles and the two parts run FC1 -> requant -> FC2 on the
                             caller's stream and on a second stream, joined before the
                             finalize (same bits either way; needs E >= 2)              */
  const float* a1_scale;  /* pmoe_moe_forward, per-tensor recipe: device float32 scalar
                             (the static FC1 input scale); otherwise NULL               */
  void* const* step_events; /* NULL, or PMOE_STEP_EVENTS caller-created hipEvent_t handles
                             (created with timing enabled, for timing only: not under
                             graph capture), recorded on the stream that runs each
                             grouped GEMM: [0]/[1] before/after FC1 of the first part
                             of the experts, [2]/[3] FC1 of the second part, [4]/[5] FC2
                             of the first part, [6]/[7] FC2 of the second part. With
                             one stream both pairs of a GEMM are recorded around its
                             one launch. A NULL entry is skipped.                     */
} pmoe_moe_options;

#define PMOE_STEP_EVENTS 8

/*
 * The routed path with options; options == NULL means per-token, ordered, no
 * clamp (exactly pmoe_routed_moe).
 *   recipe       : which entry point's contract x / x_sf / x_scale and the
 *                  weights follow (pmoe_routed_moe, pmoe_routed_moe_per_tensor,
 *                  pmoe_routed_moe_w4a16; unused inputs may be NULL).
 *   finalize     : PMOE_FINALIZE_FUSED is the order-free mode the two-stage
 *                  finalize replaces [Megatron-LM #8262 . What is added; Why
 *                  CuTe DSL, 'Controllable determinism']: each route's FC2
 *                  value fp32(acc * scale), times its routing weight, is added
 *                  with FP32 atomics into a per-token FP32 row that is rounded
 *                  to BF16 once. The order of additions is not fixed, so the
 *                  result may differ in the last FP32 bits between runs and is
 *                  not batch invariant; z is not written.
 *   swiglu_limit : the clamp of [FlashInfer #5019 . Tensor and numerical
 *                  contract, 'Compute order']; PMOE_ERR_ARG unless act is
 *                  SwiGLU (or the limit is 0).
 *   streams      : see the struct; automatic means two streams once T*K >= 2048.
 * Other arguments, layout and errors as the recipe's own entry point.
 */
int pmoe_routed_moe_ex(const void* x, const void* x_sf, const float* x_scale,
                       const void* topk_ids, int ids_type, const float* topk_w,
                       int T, int K, int E, int H, int I, int N1, int expert_offset,
                       const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                       const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                       int act, const pmoe_moe_options* options,
                       void* ws, size_t ws_bytes, void* out, void* stream);

/*
 * The whole routed layer from BF16 activations: for the NVFP4 recipes the
 * input is quantized inside the call (per token, or with options->a1_scale for
 * the per-tensor recipe) into the workspace: up to T*K = 8192 routes in the
 * same launch as the routing, on the caller's stream; above that on the
 * library's second stream while the routing runs on the caller's. Then the
 * path of pmoe_routed_moe_ex. For PMOE_RECIPE_W4A16 it is pmoe_routed_moe_ex on x.
 *   x : BF16 [T, H]. Other arguments, options and errors as pmoe_routed_moe_ex
 *   (options == NULL: per-token, ordered, no clamp). The bits of the result
 *   equal quantize + pmoe_routed_moe(_ex) on the same inputs.
 */
int pmoe_moe_forward(const void* x, const void* topk_ids, int ids_type, const float* topk_w,
                     int T, int K, int E, int H, int I, int N1, int expert_offset,
                     const void* w1_codes, const void* w1_scales, const float* w1_alpha,
                     const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                     int act, const pmoe_moe_options* options,
                     void* ws, size_t ws_bytes, void* out, void* stream);

/*
 * Router front: top-k experts and their routing weights from FP32 logits
 * (plain top-k, no group-limited routing [Megatron-LM #8262 . Performance]).
 *   logits    : float32 [T, E], finite, 1 <= E <= 1024
 *   topk_ids  : int32 [T, K] out, 1 <= K <= min(32, E): the K largest logits,
 *               larger first, equal logits ordered by lower expert id (exact:
 *               the choice is made on the logits, and softmax preserves order)
 *   topk_w    : float32 [T, K] out: p = exp(l - max) / sum_e exp(l_e - max) in
 *               FP32 (deterministic order), divided by the sum of the K chosen
 *               p (in slot order) when renormalize == 1
 * Alignment: 4 bytes.
 */
int pmoe_router_topk(const float* logits, int T, int E, int K, int renormalize,
                     int32_t* topk_ids, float* topk_w, void* stream);

/*
 * Deterministic two-stage finalize, standalone [Megatron-LM #8262 . Background,
 * 'two-stage finalize'; FlashInfer #5019 . Tensor and numerical contract]:
 *   out[t, :] = bf16( sum_{j=0..K-1, row(t,j) >= 0} fp32(w[t,j] * z[row(t,j), :]) )
 * in FP32 from +0, slot order, no fused multiply-add, one BF16 rounding.
 *   z : BF16 [R, H];  row_of_route : int32 [T*K] (-1 = skip; values must be < R);
 *   topk_w : float32 [T, K];  out : BF16 [T, H].
 * H must be a multiple of 8. Alignment: z and out 16 bytes, others 4 bytes.
 */
int pmoe_finalize(const void* z, const int32_t* row_of_route, const float* topk_w,
                  int T, int K, int H, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PMOE_H_ */
