"""Seeded synthetic inputs for the routed-MoE path (shared by tests, bench and smoke).

This module holds no arithmetic of the method: it only draws tensors with the
shapes and value distributions of the workloads and rounds them to BF16
storage. Both the GPU path and the CPU oracle take their inputs from here.

Generator. Large tensors (weights, activations) come from a counter-based
generator so that the same bits can be produced by numpy on the host (the
oracle streams single experts) and by torch on the device (the GPU path needs
6+ GB of weights per run):
    h   = mix32(mix32(index ^ k1) + k2)        (32-bit integer hash, wraps mod 2^32)
    z   = NQ[h >> 12]                          (NQ: 2^20 float32 standard-normal
                                                quantiles at (i + 0.5) / 2^20)
    val = bf16_rne(fp32(z * scale))
mix32 is the "lowbias32" integer finalizer (xor-shift / odd multiply rounds).
k1, k2 derive from (base seed 1234, workload, tensor, expert, weight epoch);
the base seed follows the reproduction command of the SM90 NVFP4 scale-ring
page. Integer hashing, table lookup and one FP32 multiply are bit-exact on
both backends. Small tensors (router logits, per-row scales) are drawn with
numpy's PCG64 from the same seed tuple and copied where needed.

Workloads (H hidden, I intermediate, E local experts, K top-k):
  tiny      T=16   H=256  I=128  E=4   K=2 relu2   x~N(0,1), 1% of elements x20
  swiglu    T=256  H=2048 I=768  E=32  K=4 swiglu  x~N(0,1); top-k weights renormalized
  relu2     T=1024 H=4096 I=2048 E=64  K=6 relu2   x~N(0,1) row-scaled by 10^U(-1,1)
  ep4_t512  T=512  H=7168 I=3072 E=96  K=6 swiglu  x~N(0,1); logits +2 on experts 0, 48
  ep4_t1024 T=1024 (same as ep4_t512)
  large     T=4096 H=7168 I=2048 E=256 K=8 swiglu  x~N(0,1), 0.5% of elements x50;
            logits U(0,1), no renormalization
  nemo_swiglu / nemo_relu2  T=64 H=2688 I=1344 E=8 K=2  x~N(0,1): the Nemotron hidden
            width with an intermediate width that is a multiple of 64 but not of 128
  odd_swiglu (T=1100) / odd_relu2 (T=48)  H=2064 I=1040 E=6 K=2  x~N(0,1): widths that
            are multiples of 16 only
Weights ~N(0, 0.02) in BF16; router logits ~N(0,1) unless stated; softmax over
all local experts, top-k by descending probability, lower expert id first.
"""
from dataclasses import dataclass, replace

import numpy as np

BASE_SEED = 1234
T_X, T_LOGITS, T_W1, T_W2, T_OUTLIER, T_ROWSCALE = 0, 1, 2, 3, 4, 5
_M1, _M2 = 0x7FEB352D, 0x846CA68B
_NQ_BITS = 20
_CHUNK = 1 << 20


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    H: int
    I: int
    E: int
    K: int
    act: str                # "relu2" or "swiglu"
    x_kind: str = "normal"  # normal | outliers | rowscale
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    logits: str = "normal"  # normal | uniform
    hot_experts: tuple = ()
    hot_bias: float = 0.0
    renormalize: bool = False
    weight_std: float = 0.02
    weight_epoch: int = 0   # bumped to draw a fresh set of weights (in-place refresh)

    @property
    def N1(self):
        return 2 * self.I if self.act == "swiglu" else self.I

    @property
    def gated(self):
        return self.act == "swiglu"

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 16, 256, 128, 4, 2, "relu2", "outliers", 0.01, 20.0),
    "swiglu": Workload("swiglu", 1, 256, 2048, 768, 32, 4, "swiglu", renormalize=True),
    "relu2": Workload("relu2", 2, 1024, 4096, 2048, 64, 6, "relu2", "rowscale"),
    "ep4_t512": Workload("ep4_t512", 3, 512, 7168, 3072, 96, 6, "swiglu",
                         hot_experts=(0, 48), hot_bias=2.0),
    "ep4_t1024": Workload("ep4_t1024", 3, 1024, 7168, 3072, 96, 6, "swiglu",
                          hot_experts=(0, 48), hot_bias=2.0),
    "large": Workload("large", 4, 4096, 7168, 2048, 256, 8, "swiglu", "outliers", 0.005, 50.0,
                      logits="uniform"),
    # the single-GPU shape of [Megatron-LM #8262 . Performance] (all 256 experts
    # local, squared ReLU, top-8), at 512 tokens: a context point, not a test config
    "dsv3_relu2_t512": Workload("dsv3_relu2_t512", 5, 512, 7168, 2048, 256, 8, "relu2"),
    # the Nemotron hidden width of [Megatron-LM #8262 . Why CuTe DSL] with I = 1344: a
    # SwiGLU FC1 (N1 = 2688) and the FC2 (N = 2688) end in a column tile that is partly
    # padding, and I is a multiple of 64 but not of 128
    "nemo_swiglu": Workload("nemo_swiglu", 6, 64, 2688, 1344, 8, 2, "swiglu"),
    "nemo_relu2": Workload("nemo_relu2", 7, 64, 2688, 1344, 8, 2, "relu2"),
    # widths that are multiples of 16 but not of 64 (H) or 32 (I): the library pads
    # the reductions to whole 64-element chunks and the output columns to whole blocks
    "odd_swiglu": Workload("odd_swiglu", 8, 1100, 2064, 1040, 6, 2, "swiglu"),
    "odd_relu2": Workload("odd_relu2", 9, 48, 2064, 1040, 6, 2, "relu2"),
}


# ----------------------------------------------------------------------------- hashing
def _mix32_int(x):
    x &= 0xFFFFFFFF
    x ^= x >> 16
    x = (x * _M1) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * _M2) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def _keys(w: Workload, tensor: int, expert: int):
    k = _mix32_int(BASE_SEED)
    for v in (w.index, tensor, expert, w.weight_epoch):
        k = _mix32_int(k ^ _mix32_int(v + 0x9E3779B9))
    return k, _mix32_int(k ^ 0x5BD1E995)


def _mix32_np(x):
    x ^= x >> np.uint32(16)
    x *= np.uint32(_M1)
    x ^= x >> np.uint32(15)
    x *= np.uint32(_M2)
    x ^= x >> np.uint32(16)
    return x


def _hash_np(n, k1, k2):
    out = np.empty(n, np.uint32)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = np.arange(s, s + m, dtype=np.uint32)
        x ^= np.uint32(k1)
        x = _mix32_np(x)
        x += np.uint32(k2)
        out[s:s + m] = _mix32_np(x)
    return out


def _mulmod32_t(x, m):
    # (x * m) mod 2^32 for int64 tensors 0 <= x < 2^32, keeping products < 2^49
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * m + (((hi * m) & 0xFFFF) << 16)) & 0xFFFFFFFF


def _mix32_t(x):
    x = x ^ (x >> 16)
    x = _mulmod32_t(x, _M1)
    x = x ^ (x >> 15)
    x = _mulmod32_t(x, _M2)
    return x ^ (x >> 16)


def _hash_t(n, k1, k2, device):
    import torch
    x = torch.arange(n, dtype=torch.int64, device=device)
    x = _mix32_t(x ^ k1)
    x = (x + k2) & 0xFFFFFFFF
    return _mix32_t(x)


_NQ = None


def normal_quantiles():
    """float32 [2^20] standard-normal quantiles at (i + 0.5) / 2^20."""
    global _NQ
    if _NQ is None:
        from scipy.special import ndtri
        n = 1 << _NQ_BITS
        _NQ = ndtri((np.arange(n, dtype=np.float64) + 0.5) / n).astype(np.float32)
    return _NQ


def _bf16_np(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint16)
    for s in range(0, flat.size, _CHUNK):
        u = flat[s:s + _CHUNK].view(np.uint32)
        out[s:s + _CHUNK] = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return out.reshape(x.shape)


def _bf16_t(x):
    """float32 tensor -> BF16 bit patterns as int16 (view as torch.bfloat16 for use)."""
    import torch
    u = x.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = r - ((r >> 15) << 16)                       # two's-complement int16 value of the bits
    return r.to(torch.int16)


def _normal_np(k1, k2, n, scale=None, bf16=False):
    """Chunked numpy backend (keeps the temporaries cache-resident)."""
    nq = normal_quantiles()
    out = np.empty(n, np.uint16 if bf16 else np.float32)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = np.arange(s, s + m, dtype=np.uint32)
        x ^= np.uint32(k1)
        x = _mix32_np(x)
        x += np.uint32(k2)
        x = _mix32_np(x)
        z = np.take(nq, x >> np.uint32(32 - _NQ_BITS))
        if scale is not None:
            z *= scale
        if bf16:
            u = z.view(np.uint32)
            z = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out[s:s + m] = z
    return out


def _normal(w, tensor, expert, n, device, scale=None):
    k1, k2 = _keys(w, tensor, expert)
    if device is None:
        return _normal_np(k1, k2, n, None if scale is None else np.float32(scale))
    import torch
    t = torch.from_numpy(normal_quantiles()).to(device)
    z = t[_hash_t(n, k1, k2, device) >> (32 - _NQ_BITS)]
    return z if scale is None else z * float(np.float32(scale))


def _uniform_u32(w, tensor, expert, n, device):
    k1, k2 = _keys(w, tensor, expert)
    if device is None:
        return _hash_np(n, k1, k2)
    return _hash_t(n, k1, k2, device)


def _as_bf16(x, device):
    return _bf16_np(x) if device is None else _bf16_t(x)


# ----------------------------------------------------------------------------- tensors
def activations(w: Workload, T: int = None, device=None):
    """BF16 activations [T, H]: numpy uint16 bit patterns, or (device given) a torch int16
    tensor of the same bits."""
    T = w.T if T is None else T
    n = T * w.H
    x = _normal(w, T_X, 0, n, device)
    if w.x_kind == "outliers":
        thr = int(w.outlier_frac * 2.0 ** 32)
        m = _uniform_u32(w, T_OUTLIER, 0, n, device) < thr
        mult = np.float32(w.outlier_mult)
        if device is None:
            x = np.where(m, x * mult, x)
        else:
            x = x.clone()
            x[m] = x[m] * float(mult)
    x = x.reshape(T, w.H)
    if w.x_kind == "rowscale":
        g = np.random.Generator(np.random.PCG64([BASE_SEED, w.index, T_ROWSCALE]))
        s = np.power(10.0, g.uniform(-1.0, 1.0, size=(T, 1))).astype(np.float32)
        if device is None:
            x = x * s
        else:
            import torch
            x = x * torch.from_numpy(s).to(device)
    return _as_bf16(x, device)


def router_logits(w: Workload, T: int = None):
    """Seeded FP32 router logits [T, E] (the hot experts get +hot_bias)."""
    T = w.T if T is None else T
    g = np.random.Generator(np.random.PCG64([BASE_SEED, w.index, T_LOGITS]))
    if w.logits == "uniform":
        logits = g.random((T, w.E))
    else:
        logits = g.standard_normal((T, w.E))
    for e in w.hot_experts:
        logits[:, e] += w.hot_bias
    return logits.astype(np.float32)


def router(w: Workload, T: int = None):
    """(topk_ids int32 [T, K], topk_w float32 [T, K]) from softmax over router_logits (numpy)."""
    logits = router_logits(w, T).astype(np.float64)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, : w.K]
    wts = np.take_along_axis(p, ids, axis=1)
    if w.renormalize:
        wts = wts / wts.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), wts.astype(np.float32)


def expert_weights(w: Workload, e: int, device=None):
    """(FC1 [N1, H], FC2 [H, I]) BF16 of local expert e; FC1 rows are gate then up.
    numpy uint16 bit patterns, or (device given) torch int16 tensors of the same bits."""
    if device is None:
        std = np.float32(w.weight_std)
        a = _normal_np(*_keys(w, T_W1, e), w.N1 * w.H, std, bf16=True)
        b = _normal_np(*_keys(w, T_W2, e), w.H * w.I, std, bf16=True)
        return a.reshape(w.N1, w.H), b.reshape(w.H, w.I)
    a = _normal(w, T_W1, e, w.N1 * w.H, device, w.weight_std)
    b = _normal(w, T_W2, e, w.H * w.I, device, w.weight_std)
    return (_as_bf16(a, device).reshape(w.N1, w.H), _as_bf16(b, device).reshape(w.H, w.I))


def all_weights(w: Workload, device=None):
    """Stacked BF16 weights (FC1 [E, N1, H], FC2 [E, H, I])."""
    if device is None:
        w1 = np.empty((w.E, w.N1, w.H), np.uint16)
        w2 = np.empty((w.E, w.H, w.I), np.uint16)
    else:
        import torch
        w1 = torch.empty((w.E, w.N1, w.H), dtype=torch.int16, device=device)
        w2 = torch.empty((w.E, w.H, w.I), dtype=torch.int16, device=device)
    for e in range(w.E):
        a, b = expert_weights(w, e, device)
        w1[e], w2[e] = a, b
    return w1, w2
