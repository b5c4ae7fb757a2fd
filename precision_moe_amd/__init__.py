"""precision_moe_amd -- per-token NVFP4 routed-MoE expert path on AMD MI355X (gfx950).

Thin Python binding over the C ABI of libpmoe.so (include/pmoe.h): every
function here only marshals torch tensors (device memory) and the current HIP
stream into the C calls; all computation runs in the library's HIP kernels.
The library is loaded on first use and its absence raises an error -- there
is no fallback implementation.
"""
import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# PMOE_LIB may point at another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("PMOE_LIB") or os.path.join(_HERE, "_lib", "libpmoe.so")

ACT_RELU2, ACT_SWIGLU = 0, 1
IDS_INT32, IDS_INT64 = 0, 1
RECIPE_PER_TOKEN, RECIPE_PER_TENSOR, RECIPE_W4A16 = 0, 1, 2
FINALIZE_ORDERED, FINALIZE_FUSED = 0, 1
_RECIPES = {"per_token": RECIPE_PER_TOKEN, "per_tensor": RECIPE_PER_TENSOR, "w4a16": RECIPE_W4A16}
_FINALIZE = {"ordered": FINALIZE_ORDERED, "fused": FINALIZE_FUSED}
WS_FIELDS = ("row_of_route", "route_of_row", "expert_offsets", "counters", "h", "hq", "h_sf",
             "h_scale", "z")

_c_size_p = ctypes.POINTER(ctypes.c_size_t)
_vp = ctypes.c_void_p
_i = ctypes.c_int


class MoeOptions(ctypes.Structure):
    """pmoe_moe_options (include/pmoe.h)."""
    _fields_ = [("recipe", ctypes.c_int), ("finalize", ctypes.c_int),
                ("swiglu_limit", ctypes.c_float), ("a2_scale", ctypes.c_void_p),
                ("streams", ctypes.c_int), ("a1_scale", ctypes.c_void_p),
                ("step_events", ctypes.c_void_p)]
STEP_EVENTS = 8
_SIGNATURES = {
    "pmoe_version": (_i, []),
    "pmoe_last_error": (ctypes.c_char_p, []),
    "pmoe_weight_bytes": (_i, [_i, _i, _i, _i, _c_size_p]),
    "pmoe_prepare_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "pmoe_prepare_weights": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]),
    "pmoe_quantize_input_per_token": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp]),
    "pmoe_quantize_rows_f32": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp]),
    "pmoe_moe_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i, _i]),
    "pmoe_moe_workspace_layout": (_i, [_i, _i, _i, _i, _i, _i, _c_size_p]),
    "pmoe_routed_moe": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                             _vp, _vp, _vp, _vp, _i, _vp, ctypes.c_size_t, _vp, _vp]),
    "pmoe_routed_moe_static": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _i, _vp, _vp]),
    "pmoe_routed_moe_steps": (_i, [_i, _i, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, ctypes.c_size_t, _vp, _vp]),
    "pmoe_finalize": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "pmoe_prepare_weights_per_tensor": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "pmoe_quantize_input_per_tensor": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp]),
    "pmoe_routed_moe_per_tensor": (_i, [_vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _i, _vp, ctypes.c_size_t, _vp, _vp]),
    "pmoe_routed_moe_w4a16": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _i, _vp, ctypes.c_size_t, _vp, _vp]),
    "pmoe_routed_moe_ex": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                _vp, _vp, _vp, _vp, _i, ctypes.POINTER(MoeOptions), _vp,
                                ctypes.c_size_t, _vp, _vp]),
    "pmoe_router_topk": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "pmoe_moe_forward": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                              _vp, _i, ctypes.POINTER(MoeOptions), _vp, ctypes.c_size_t, _vp, _vp]),
}
STEP_ROUTE, STEP_FC1, STEP_REQUANT, STEP_FC2, STEP_FINALIZE = range(5)

_lib = None


class PmoeError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"pmoe error {code}: {message}")
        self.code = code


def lib():
    """Load libpmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with precision_moe_amd.build.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(rc):
    if rc != 0:
        raise PmoeError(rc, lib().pmoe_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None, *tensors):
    """The hipStream_t to enqueue on. A `stream` other than torch's current one first
    waits for the current stream (the inputs and the temporaries made here were produced
    there), and every tensor the call touches is recorded as used on `stream`, so the
    caching allocator does not hand its memory out again before that work is done."""
    import torch
    cur = torch.cuda.current_stream()
    if stream is None or stream == cur:
        return ctypes.c_void_p(cur.cuda_stream)
    stream.wait_stream(cur)
    for t in tensors:
        if t is not None and torch.is_tensor(t) and t.is_cuda:
            t.record_stream(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _event_array(events):
    """ctypes array of the raw hipEvent_t handles of STEP_EVENTS torch.cuda.Events (or None)."""
    import torch
    if events is None:
        return None
    if len(events) != STEP_EVENTS:
        raise ValueError(f"step_events needs {STEP_EVENTS} events")
    handles = []
    for ev in events:
        if ev is None:
            handles.append(None)
            continue
        if ev.cuda_event == 0:          # torch creates the event on its first record
            ev.record(torch.cuda.current_stream())
        handles.append(ev.cuda_event)
    return (ctypes.c_void_p * STEP_EVENTS)(*handles)


def _bf16_storage(t):
    import torch
    if t.element_size() != 2:
        raise TypeError("expected a 2-byte (BF16) tensor")
    return t


# ----------------------------------------------------------------------------- weights
@dataclass
class PreparedWeights:
    """Prepared NVFP4 expert weights (layout in include/pmoe.h), all on one device."""
    E: int
    N1: int
    H: int
    I: int
    w1_codes: object
    w1_scales: object
    w1_alpha: object
    w2_codes: object
    w2_scales: object
    w2_alpha: object

    @property
    def act(self):
        return ACT_SWIGLU if self.N1 == 2 * self.I else ACT_RELU2


def weight_bytes(E, N1, H, I):
    sizes = (ctypes.c_size_t * 4)()
    _check(lib().pmoe_weight_bytes(E, N1, H, I, sizes))
    return tuple(int(s) for s in sizes)


def empty_weights(E, N1, H, I, device):
    import torch
    b = weight_bytes(E, N1, H, I)
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return PreparedWeights(E, N1, H, I, torch.empty(b[0], **u8), torch.empty(b[1], **u8),
                           torch.empty(E, **f32), torch.empty(b[2], **u8), torch.empty(b[3], **u8),
                           torch.empty(E, **f32))


def prepare_weights(w1, w2, out=None, workspace=None, stream=None, input_scales=None):
    """BF16 FC1 [E, N1, H] and FC2 [E, H, I] -> PreparedWeights (in place into `out` if given).

    input_scales = (a1, a2), device float32 scalars, selects the per-tensor
    recipe: the static input scales are folded into the alphas.
    """
    import torch
    E, N1, H = w1.shape
    I = w2.shape[2]
    if tuple(w2.shape[:2]) != (E, H):
        raise ValueError("FC2 must be [E, H, I] with FC1's E and H")
    w1, w2 = _bf16_storage(w1.contiguous()), _bf16_storage(w2.contiguous())
    if out is None:
        out = empty_weights(E, N1, H, I, w1.device)
    elif (out.E, out.N1, out.H, out.I) != (E, N1, H, I):
        raise ValueError("`out` was prepared for other shapes")
    need = lib().pmoe_prepare_workspace_bytes(E, N1, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=w1.device)
    if input_scales is None:
        _check(lib().pmoe_prepare_weights(
            _ptr(w1), _ptr(w2), E, N1, H, I, _ptr(out.w1_codes), _ptr(out.w1_scales),
            _ptr(out.w1_alpha), _ptr(out.w2_codes), _ptr(out.w2_scales), _ptr(out.w2_alpha),
            _ptr(workspace), workspace.numel(), _stream(stream, w1, w2, workspace, out.w1_codes, out.w1_scales,
                                                          out.w1_alpha, out.w2_codes, out.w2_scales,
                                                          out.w2_alpha)))
    else:
        a1, a2 = (_f32_scalar(a) for a in input_scales)
        _check(lib().pmoe_prepare_weights_per_tensor(
            _ptr(w1), _ptr(w2), E, N1, H, I, _ptr(a1), _ptr(a2), _ptr(out.w1_codes),
            _ptr(out.w1_scales), _ptr(out.w1_alpha), _ptr(out.w2_codes), _ptr(out.w2_scales),
            _ptr(out.w2_alpha), _ptr(workspace), workspace.numel(),
            _stream(stream, w1, w2, a1, a2, workspace, out.w1_codes, out.w1_scales, out.w1_alpha,
                    out.w2_codes, out.w2_scales, out.w2_alpha)))
    return out


def _f32_scalar(a):
    import torch
    if not (torch.is_tensor(a) and a.dtype == torch.float32 and a.numel() == 1 and a.is_cuda):
        raise TypeError("static scales are device float32 tensors of one element")
    return a


# ----------------------------------------------------------------------------- quantizers
def quantize_input_per_token(x, out=None, stream=None):
    """BF16 [T, H] -> (xq uint8 [T, H/2], x_sf uint8 [T, H/16], x_scale float32 [T])."""
    import torch
    T, H = x.shape
    x = _bf16_storage(x.contiguous())
    if out is None:
        out = (torch.empty((T, H // 2), dtype=torch.uint8, device=x.device),
               torch.empty((T, H // 16), dtype=torch.uint8, device=x.device),
               torch.empty((T,), dtype=torch.float32, device=x.device))
    xq, xsf, xs = out
    _check(lib().pmoe_quantize_input_per_token(_ptr(x), T, H, _ptr(xq), _ptr(xsf), _ptr(xs),
                                               _stream(stream, x, xq, xsf, xs)))
    return xq, xsf, xs


def quantize_input_per_tensor(x, a1, out=None, stream=None):
    """BF16 [T, H] with a static scale a1 (device float32 scalar) -> (xq [T, H/2], x_sf [T, H/16])."""
    import torch
    T, H = x.shape
    x = _bf16_storage(x.contiguous())
    if out is None:
        out = (torch.empty((T, H // 2), dtype=torch.uint8, device=x.device),
               torch.empty((T, H // 16), dtype=torch.uint8, device=x.device))
    xq, xsf = out
    _check(lib().pmoe_quantize_input_per_tensor(_ptr(x), T, H, _ptr(_f32_scalar(a1)), _ptr(xq),
                                                _ptr(xsf), _stream(stream, x, a1, xq, xsf)))
    return xq, xsf


def quantize_rows_f32(h, out=None, stream=None):
    """float32 [R, L] -> (hq uint8 [R, L/2], h_sf uint8 [R, L/16], h_scale float32 [R])."""
    import torch
    R, L = h.shape
    h = h.contiguous()
    if h.dtype != torch.float32:
        raise TypeError("h must be float32")
    if out is None:
        out = (torch.empty((R, L // 2), dtype=torch.uint8, device=h.device),
               torch.empty((R, L // 16), dtype=torch.uint8, device=h.device),
               torch.empty((R,), dtype=torch.float32, device=h.device))
    hq, hsf, hs = out
    _check(lib().pmoe_quantize_rows_f32(_ptr(h), R, L, _ptr(hq), _ptr(hsf), _ptr(hs),
                                        _stream(stream, h, hq, hsf, hs)))
    return hq, hsf, hs


# ----------------------------------------------------------------------------- routed MoE
def moe_workspace_bytes(T, K, E, H, I, act):
    n = lib().pmoe_moe_workspace_bytes(T, K, E, H, I, act)
    if n == 0:
        _check(lib().pmoe_moe_workspace_layout(T, K, E, H, I, act, (ctypes.c_size_t * 9)()))
    return int(n)


def moe_workspace_layout(T, K, E, H, I, act):
    offs = (ctypes.c_size_t * len(WS_FIELDS))()
    _check(lib().pmoe_moe_workspace_layout(T, K, E, H, I, act, offs))
    return dict(zip(WS_FIELDS, (int(o) for o in offs)))


def workspace_views(ws, T, K, E, H, I, act):
    """Typed views of the routed_moe workspace fields (for inspection in tests)."""
    import torch
    off = moe_workspace_layout(T, K, E, H, I, act)
    TK = T * K
    Ip = -(-I // 64) * 64          # the intermediate's rows are padded to whole 64-element chunks

    def view(name, count, dtype):
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return ws[off[name]:off[name] + nbytes].view(dtype)

    return {
        "row_of_route": view("row_of_route", TK, torch.int32),
        "route_of_row": view("route_of_row", TK, torch.int32),
        "expert_offsets": view("expert_offsets", E + 1, torch.int32),
        "counters": view("counters", 4, torch.int32),
        "h": view("h", TK * I, torch.float32).view(TK, I),
        # W4A16: BF16 h in the same field, rows of Ip (zeros past I)
        "h_bf16": view("h", TK * Ip, torch.int16).view(TK, Ip)[:, :I],
        "hq": view("hq", TK * Ip // 2, torch.uint8).view(TK, Ip // 2)[:, :I // 2],
        "h_sf": view("h_sf", TK * Ip // 16, torch.uint8).view(TK, Ip // 16)[:, :I // 16],
        "hq_padded": view("hq", TK * Ip // 2, torch.uint8).view(TK, Ip // 2),
        "h_sf_padded": view("h_sf", TK * Ip // 16, torch.uint8).view(TK, Ip // 16),
        "h_scale": view("h_scale", TK, torch.float32),
        "z": view("z", TK * H, torch.int16).view(TK, H),
    }


def routed_moe(xq, x_sf, x_scale, topk_ids, topk_w, weights: PreparedWeights, act=None,
               expert_offset=0, workspace=None, out=None, stream=None, steps=None):
    """Routing, FC1 + activation, requantization, FC2 and the fixed-order finalize.

    Returns BF16 [T, H] (as torch.bfloat16 unless `out` is given). `steps`
    = (first, last) runs only that range of the five steps (STEP_*), reusing
    `workspace` and `out` from earlier calls.
    """
    import torch
    T, K = topk_ids.shape
    W = weights
    act = W.act if act is None else act
    if topk_ids.dtype == torch.int32:
        ids_type = IDS_INT32
    elif topk_ids.dtype == torch.int64:
        ids_type = IDS_INT64
    else:
        raise TypeError("topk_ids must be int32 or int64")
    topk_ids = topk_ids.contiguous()
    topk_w = topk_w.contiguous()
    if topk_w.dtype != torch.float32:
        raise TypeError("topk_w must be float32")
    if workspace is None:
        workspace = torch.empty(max(moe_workspace_bytes(T, K, W.E, W.H, W.I, act), 256),
                                dtype=torch.uint8, device=xq.device)
    if out is None:
        out = torch.empty((T, W.H), dtype=torch.bfloat16, device=xq.device)
    first, last = (STEP_ROUTE, STEP_FINALIZE) if steps is None else steps
    _check(lib().pmoe_routed_moe_steps(
        first, last, _ptr(xq), _ptr(x_sf), _ptr(x_scale), _ptr(topk_ids), ids_type, _ptr(topk_w), T, K,
        W.E, W.H, W.I, W.N1, expert_offset, _ptr(W.w1_codes), _ptr(W.w1_scales), _ptr(W.w1_alpha),
        _ptr(W.w2_codes), _ptr(W.w2_scales), _ptr(W.w2_alpha), act, _ptr(workspace),
        workspace.numel(), _ptr(out),
        _stream(stream, xq, x_sf, x_scale, topk_ids, topk_w, workspace, out, W.w1_codes, W.w1_scales, W.w1_alpha, W.w2_codes, W.w2_scales, W.w2_alpha)))
    return out


STATIC_SCRATCH_BYTES = 64 << 20


def routed_moe_static(xq, x_sf, x_scale, topk_ids, topk_w, weights: PreparedWeights, act=None,
                      expert_offset=0, out=None, stream=None):
    """routed_moe on the library's static scratch (pmoe_routed_moe_static): no workspace
    argument and no device allocation inside the call; `out` should be given by callers
    that cannot allocate (else one BF16 [T, H] tensor is allocated here)."""
    import torch
    T, K = topk_ids.shape
    W = weights
    act = W.act if act is None else act
    topk_ids, ids_type, topk_w = _routing_args(topk_ids, topk_w)
    if out is None:
        out = torch.empty((T, W.H), dtype=torch.bfloat16, device=xq.device)
    _check(lib().pmoe_routed_moe_static(
        _ptr(xq), _ptr(x_sf), _ptr(x_scale), _ptr(topk_ids), ids_type, _ptr(topk_w), T, K, W.E, W.H,
        W.I, W.N1, expert_offset, _ptr(W.w1_codes), _ptr(W.w1_scales), _ptr(W.w1_alpha),
        _ptr(W.w2_codes), _ptr(W.w2_scales), _ptr(W.w2_alpha), act, _ptr(out),
        _stream(stream, xq, x_sf, x_scale, topk_ids, topk_w, out, W.w1_codes, W.w1_scales,
                W.w1_alpha, W.w2_codes, W.w2_scales, W.w2_alpha)))
    return out


def _routing_args(topk_ids, topk_w):
    import torch
    if topk_ids.dtype == torch.int32:
        ids_type = IDS_INT32
    elif topk_ids.dtype == torch.int64:
        ids_type = IDS_INT64
    else:
        raise TypeError("topk_ids must be int32 or int64")
    if topk_w.dtype != torch.float32:
        raise TypeError("topk_w must be float32")
    return topk_ids.contiguous(), ids_type, topk_w.contiguous()


def _moe_buffers(T, K, W, act, device, workspace, out):
    import torch
    if workspace is None:
        workspace = torch.empty(max(moe_workspace_bytes(T, K, W.E, W.H, W.I, act), 256),
                                dtype=torch.uint8, device=device)
    if out is None:
        out = torch.empty((T, W.H), dtype=torch.bfloat16, device=device)
    return workspace, out


def routed_moe_per_tensor(xq, x_sf, topk_ids, topk_w, weights: PreparedWeights, a2, act=None,
                          expert_offset=0, workspace=None, out=None, stream=None):
    """Per-tensor NVFP4 recipe: (xq, x_sf) from quantize_input_per_tensor, weights prepared
    with input_scales=(a1, a2), a2 the static FC2 input scale (device float32 scalar)."""
    T, K = topk_ids.shape
    W = weights
    act = W.act if act is None else act
    topk_ids, ids_type, topk_w = _routing_args(topk_ids, topk_w)
    workspace, out = _moe_buffers(T, K, W, act, xq.device, workspace, out)
    _check(lib().pmoe_routed_moe_per_tensor(
        _ptr(xq), _ptr(x_sf), _ptr(topk_ids), ids_type, _ptr(topk_w), T, K, W.E, W.H, W.I, W.N1,
        expert_offset, _ptr(W.w1_codes), _ptr(W.w1_scales), _ptr(W.w1_alpha), _ptr(W.w2_codes),
        _ptr(W.w2_scales), _ptr(W.w2_alpha), _ptr(_f32_scalar(a2)), act, _ptr(workspace),
        workspace.numel(), _ptr(out),
        _stream(stream, xq, x_sf, topk_ids, topk_w, a2, workspace, out, W.w1_codes, W.w1_scales, W.w1_alpha, W.w2_codes, W.w2_scales, W.w2_alpha)))
    return out


def routed_moe_w4a16(x, topk_ids, topk_w, weights: PreparedWeights, act=None, expert_offset=0,
                     workspace=None, out=None, stream=None):
    """W4A16 (weight_only) recipe: BF16 activations x [T, H], NVFP4 weights from prepare_weights."""
    T, K = topk_ids.shape
    W = weights
    act = W.act if act is None else act
    x = _bf16_storage(x.contiguous())
    topk_ids, ids_type, topk_w = _routing_args(topk_ids, topk_w)
    workspace, out = _moe_buffers(T, K, W, act, x.device, workspace, out)
    _check(lib().pmoe_routed_moe_w4a16(
        _ptr(x), _ptr(topk_ids), ids_type, _ptr(topk_w), T, K, W.E, W.H, W.I, W.N1, expert_offset,
        _ptr(W.w1_codes), _ptr(W.w1_scales), _ptr(W.w1_alpha), _ptr(W.w2_codes), _ptr(W.w2_scales),
        _ptr(W.w2_alpha), act, _ptr(workspace), workspace.numel(), _ptr(out),
        _stream(stream, x, topk_ids, topk_w, workspace, out, W.w1_codes, W.w1_scales, W.w1_alpha, W.w2_codes, W.w2_scales, W.w2_alpha)))
    return out


def routed_moe_ex(x, x_sf, x_scale, topk_ids, topk_w, weights: PreparedWeights, recipe="per_token",
                  finalize="ordered", swiglu_limit=0.0, a2=None, act=None, expert_offset=0,
                  workspace=None, out=None, stream=None, streams=0, step_events=None):
    """The routed path with options (pmoe_routed_moe_ex): recipe "per_token" (x = xq, x_sf,
    x_scale), "per_tensor" (x = xq, x_sf; a2) or "w4a16" (x = BF16 activations; x_sf, x_scale
    None); finalize "ordered" or "fused"; swiglu_limit > 0 clamps SwiGLU; step_events: None
    or STEP_EVENTS torch.cuda.Events (timing enabled) recorded around the grouped GEMMs."""
    T, K = topk_ids.shape
    W = weights
    act = W.act if act is None else act
    topk_ids, ids_type, topk_w = _routing_args(topk_ids, topk_w)
    if recipe == "w4a16":
        x = _bf16_storage(x.contiguous())
    workspace, out = _moe_buffers(T, K, W, act, x.device, workspace, out)
    evs = _event_array(step_events)
    opt = MoeOptions(_RECIPES[recipe], _FINALIZE[finalize], float(swiglu_limit),
                     _f32_scalar(a2).data_ptr() if a2 is not None else None, int(streams), None,
                     ctypes.cast(evs, ctypes.c_void_p) if evs is not None else None)
    _check(lib().pmoe_routed_moe_ex(
        _ptr(x), _ptr(x_sf), _ptr(x_scale), _ptr(topk_ids), ids_type, _ptr(topk_w), T, K, W.E, W.H,
        W.I, W.N1, expert_offset, _ptr(W.w1_codes), _ptr(W.w1_scales), _ptr(W.w1_alpha),
        _ptr(W.w2_codes), _ptr(W.w2_scales), _ptr(W.w2_alpha), act, ctypes.byref(opt),
        _ptr(workspace), workspace.numel(), _ptr(out),
        _stream(stream, x, x_sf, x_scale, topk_ids, topk_w, a2, workspace, out, W.w1_codes, W.w1_scales, W.w1_alpha, W.w2_codes, W.w2_scales, W.w2_alpha)))
    return out


def moe_forward(x, topk_ids, topk_w, weights: PreparedWeights, recipe="per_token",
                finalize="ordered", swiglu_limit=0.0, a1=None, a2=None, act=None, expert_offset=0,
                workspace=None, out=None, stream=None, streams=0, step_events=None):
    """The whole routed layer from BF16 activations x [T, H] (pmoe_moe_forward): the NVFP4
    recipes quantize x inside the call, overlapped with the routing. step_events: None or
    STEP_EVENTS torch.cuda.Events (timing enabled) recorded around the grouped GEMMs."""
    T, K = topk_ids.shape
    W = weights
    act = W.act if act is None else act
    x = _bf16_storage(x.contiguous())
    topk_ids, ids_type, topk_w = _routing_args(topk_ids, topk_w)
    workspace, out = _moe_buffers(T, K, W, act, x.device, workspace, out)
    evs = _event_array(step_events)
    opt = MoeOptions(_RECIPES[recipe], _FINALIZE[finalize], float(swiglu_limit),
                     _f32_scalar(a2).data_ptr() if a2 is not None else None, int(streams),
                     _f32_scalar(a1).data_ptr() if a1 is not None else None,
                     ctypes.cast(evs, ctypes.c_void_p) if evs is not None else None)
    _check(lib().pmoe_moe_forward(
        _ptr(x), _ptr(topk_ids), ids_type, _ptr(topk_w), T, K, W.E, W.H, W.I, W.N1, expert_offset,
        _ptr(W.w1_codes), _ptr(W.w1_scales), _ptr(W.w1_alpha), _ptr(W.w2_codes), _ptr(W.w2_scales),
        _ptr(W.w2_alpha), act, ctypes.byref(opt), _ptr(workspace), workspace.numel(), _ptr(out),
        _stream(stream, x, topk_ids, topk_w, a1, a2, workspace, out, W.w1_codes, W.w1_scales, W.w1_alpha, W.w2_codes, W.w2_scales, W.w2_alpha)))
    return out


def router_topk(logits, k, renormalize=False, out=None, stream=None):
    """FP32 logits [T, E] -> (topk_ids int32 [T, k], topk_w float32 [T, k])."""
    import torch
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    logits = logits.contiguous()
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=logits.device),
               torch.empty((T, k), dtype=torch.float32, device=logits.device))
    ids, w = out
    _check(lib().pmoe_router_topk(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(ids), _ptr(w),
                                  _stream(stream, logits, ids, w)))
    return ids, w


def finalize(z, row_of_route, topk_w, out=None, stream=None):
    """Fixed-order finalize: z BF16 [R, H], row_of_route int32 [T*K], topk_w float32 [T, K]."""
    import torch
    T, K = topk_w.shape
    H = z.shape[1]
    z = _bf16_storage(z.contiguous())
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=z.device)
    row_of_route = row_of_route.contiguous()
    topk_w = topk_w.contiguous()
    _check(lib().pmoe_finalize(_ptr(z), _ptr(row_of_route), _ptr(topk_w), T, K, H, _ptr(out),
                               _stream(stream, z, row_of_route, topk_w, out)))
    return out
