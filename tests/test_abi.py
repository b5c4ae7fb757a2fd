"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side validation rejects bad arguments before touching any device."""
import ctypes
import os
import re

import pytest

import precision_moe_amd as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pmoe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pmoe_[a-z0-9_]+)\s*\(", src)))


def _header_consts():
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(PMOE_[A-Z0-9_]+)\s+(\d+)", open(HEADER).read())}


def test_library_loads_and_exports_every_declared_symbol():
    lib = pm.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pm._SIGNATURES)


def test_binding_constants_match_header():
    c = _header_consts()
    assert (c["PMOE_ACT_RELU2"], c["PMOE_ACT_SWIGLU"]) == (pm.ACT_RELU2, pm.ACT_SWIGLU)
    assert (c["PMOE_IDS_INT32"], c["PMOE_IDS_INT64"]) == (pm.IDS_INT32, pm.IDS_INT64)
    assert c["PMOE_WS_NUM_FIELDS"] == len(pm.WS_FIELDS)
    assert (c["PMOE_RECIPE_PER_TOKEN"], c["PMOE_RECIPE_PER_TENSOR"], c["PMOE_RECIPE_W4A16"]) == \
        (pm.RECIPE_PER_TOKEN, pm.RECIPE_PER_TENSOR, pm.RECIPE_W4A16)
    assert (c["PMOE_FINALIZE_ORDERED"], c["PMOE_FINALIZE_FUSED"]) == (pm.FINALIZE_ORDERED, pm.FINALIZE_FUSED)
    fields = sorted((v, k) for k, v in c.items() if k.startswith("PMOE_WS_") and k != "PMOE_WS_NUM_FIELDS")
    assert [k[len("PMOE_WS_"):].lower() for _, k in fields] == list(pm.WS_FIELDS)


def test_version_and_sizes():
    assert pm.lib().pmoe_version() >= 100
    E, H, I = 4, 1024, 512
    assert pm.weight_bytes(E, 2 * I, H, I) == (E * 2 * I * H // 2, E * 2 * I * H // 16, E * H * I // 2,
                                              E * H * I // 16)
    # rows are padded to whole column tiles of 8 blocks x 32 rows
    pad = lambda n: -(-n // 256) * 256
    E, H, I = 3, 320, 192
    assert pm.weight_bytes(E, I, H, I) == (E * pad(I) * H // 2, E * pad(I) * H // 16, E * pad(H) * I // 2,
                                          E * pad(H) * I // 16)
    assert pm.lib().pmoe_prepare_workspace_bytes(E, I, H, I) > 0
    # H and I multiples of 16: column blocks of a gated FC1 per half (ceil(I/32) each), and
    # the reduction padded to whole chunks of 64
    E, H, I = 2, 80, 48
    assert pm.weight_bytes(E, 2 * I, H, I) == (E * 256 * 128 // 2, E * 256 * 128 // 16,
                                              E * 256 * 64 // 2, E * 256 * 64 // 16)


def test_workspace_layout_is_aligned_and_large_enough():
    T, K, E, H, I = 100, 6, 96, 7168, 3072
    off = pm.moe_workspace_layout(T, K, E, H, I, pm.ACT_SWIGLU)
    total = pm.moe_workspace_bytes(T, K, E, H, I, pm.ACT_SWIGLU)
    vals = [off[f] for f in pm.WS_FIELDS]
    assert vals == sorted(vals) and all(v % 256 == 0 for v in vals)
    TK = T * K
    assert off["z"] + TK * H * 2 <= total
    assert off["hq"] - off["h"] >= TK * I * 4


@pytest.mark.parametrize("E,N1,H,I", [(4, 256, 100, 128), (4, 200, 256, 100), (4, 384, 256, 128),
                                      (0, 256, 256, 128), (2000, 256, 256, 128), (4, 256, 256, 0)])
def test_weight_shape_errors(E, N1, H, I):
    sizes = (ctypes.c_size_t * 4)()
    assert pm.lib().pmoe_weight_bytes(E, N1, H, I, sizes) == 3
    assert pm.lib().pmoe_last_error().decode() != ""
    assert pm.lib().pmoe_prepare_workspace_bytes(E, N1, H, I) == 0


@pytest.mark.parametrize("T,K,E,H,I,act,code", [
    (-1, 2, 4, 256, 128, 0, 3), (8, 0, 4, 256, 128, 0, 3), (8, 5, 4, 256, 128, 0, 3),
    (8, 33, 64, 256, 128, 0, 3), (8, 2, 4, 250, 128, 0, 3), (8, 2, 4, 256, 100, 0, 3),
    (8, 2, 4, 256, 8, 0, 3), (8, 2, 4, 16400, 128, 0, 3),
    (8, 2, 1025, 256, 128, 0, 3), (8, 2, 4, 256, 128, 7, 4)])
def test_moe_shape_errors(T, K, E, H, I, act, code):
    N1 = 2 * I if act == 1 else I
    rc = pm.lib().pmoe_routed_moe(None, None, None, None, 0, None, T, K, E, H, I, N1, 0, None, None,
                                  None, None, None, None, act, None, 0, None, None)
    assert rc == code, pm.lib().pmoe_last_error()
    assert pm.lib().pmoe_moe_workspace_bytes(T, K, E, H, I, act) == 0


def test_bad_ids_type_and_zero_tokens():
    lib = pm.lib()
    args = [None, None, None, None, 0, None, 8, 2, 4, 256, 128, 128, 0] + [None] * 6 + [0, None, 0, None, None]
    args[4] = 5
    assert lib.pmoe_routed_moe(*args) == 7
    args[4] = 0
    args[11] = 256                 # gated FC1 with the squared-ReLU activation
    assert lib.pmoe_routed_moe(*args) == 4
    args[11] = 200
    assert lib.pmoe_routed_moe(*args) == 3
    args[11] = 128
    args[6] = 0                    # T == 0 is a successful no-op: nothing is touched
    assert lib.pmoe_routed_moe(*args) == 0
    assert lib.pmoe_quantize_input_per_token(None, 0, 256, None, None, None, None) == 0
    assert lib.pmoe_quantize_input_per_token(None, 4, 100, None, None, None, None) == 3
    assert lib.pmoe_finalize(None, None, None, 4, 0, 64, None, None) == 3
    assert lib.pmoe_finalize(None, None, None, 4, 2, 60, None, None) == 3


@pytest.mark.skipif(__import__("conftest").gpu_available(), reason="checks the no-GPU path")
def test_no_device_is_reported_not_crashed():
    rc = pm.lib().pmoe_quantize_input_per_token(None, 4, 256, None, None, None, None)
    assert rc == 1
    assert "gfx950" in pm.lib().pmoe_last_error().decode() or "device" in pm.lib().pmoe_last_error().decode()


def test_options_and_router_validation():
    lib = pm.lib()
    base = [None, None, None, None, 0, None, 8, 2, 4, 256, 128, 256, 0] + [None] * 6 + [1]
    tail = [None, 0, None, None]

    def ex(**kw):
        o = pm.MoeOptions(kw.get("recipe", 0), kw.get("finalize", 0), kw.get("limit", 0.0), None)
        return lib.pmoe_routed_moe_ex(*base, ctypes.byref(o), *tail)

    assert ex(recipe=3) == 7                    # unknown recipe
    assert ex(finalize=2) == 7                  # unknown finalize mode
    assert ex(limit=-1.0) == 7                  # negative clamp limit
    relu = list(base)
    relu[11], relu[19] = 128, 0                 # squared ReLU cannot take a SwiGLU clamp
    o = pm.MoeOptions(0, 0, 10.0, None)
    assert lib.pmoe_routed_moe_ex(*relu, ctypes.byref(o), *tail) == 7
    z = list(base)
    z[6] = 0                                    # T == 0: no-op with any valid options
    assert lib.pmoe_routed_moe_ex(*z, ctypes.byref(pm.MoeOptions(2, 1, 5.0, None)), *tail) == 0
    assert lib.pmoe_routed_moe_ex(*z, None, *tail) == 0
    a1 = ctypes.c_float(1.0)
    o = pm.MoeOptions(0, 0, 0.0, None, 0, ctypes.addressof(a1))
    assert lib.pmoe_routed_moe_ex(*base, ctypes.byref(o), *tail) == 7    # a1 is forward's
    fwd = base[:1] + base[3:]                   # forward: x, ids, ... (no x_sf / x_scale)
    assert lib.pmoe_moe_forward(*fwd, ctypes.byref(o), *tail) == 7      # a1 with per-token
    assert lib.pmoe_moe_forward(*fwd, ctypes.byref(pm.MoeOptions(3, 0, 0.0, None)), *tail) == 7
    zf = list(fwd)
    zf[4] = 0                                   # T == 0
    assert lib.pmoe_moe_forward(*zf, None, *tail) == 0
    o = pm.MoeOptions(1, 0, 0.0, None, 0, ctypes.addressof(a1))
    assert lib.pmoe_moe_forward(*zf, ctypes.byref(o), *tail) == 0
    assert lib.pmoe_router_topk(None, 0, 64, 6, 0, None, None, None) == 0
    assert lib.pmoe_router_topk(None, 4, 64, 0, 0, None, None, None) == 3
    assert lib.pmoe_router_topk(None, 4, 4, 6, 0, None, None, None) == 3
    assert lib.pmoe_router_topk(None, 4, 2000, 6, 0, None, None, None) == 3
    assert lib.pmoe_router_topk(None, 4, 64, 6, 2, None, None, None) == 7
    assert lib.pmoe_quantize_input_per_tensor(None, 4, 100, None, None, None, None) == 3
