"""Pins of the oracle's number formats against hand enumerations, brute force and a library cast."""
import json
import os

import numpy as np
import pytest
import torch

from oracle.formats import (E2M1_MAGNITUDES, bf16_to_f32, e2m1_decode, e2m1_encode, e4m3_decode,
                            e4m3_encode_sat, f32_to_bf16_rne, pack_nibbles, unpack_nibbles)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_decode_all_16():
    want = [0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6]
    got = e2m1_decode(np.arange(16))
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[8])


def test_e2m1_hand_ties():
    cases = json.load(open(os.path.join(GOLD, "e2m1_ties.json")))["cases"]
    v = np.array([c[0] for c in cases], np.float32)
    want = np.array([c[1] for c in cases], np.uint8)
    assert np.array_equal(e2m1_encode(v), want)


def _e2m1_argmin(v):
    """Independent definition: nearest grid magnitude; on a tie the even code."""
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    d = np.abs(a[:, None] - E2M1_MAGNITUDES[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = np.where(a > 6.0, 7, code)
    return (code | (np.signbit(v).astype(int) << 3)).astype(np.uint8)


def test_e2m1_brute_force():
    rng = np.random.default_rng(7)
    v = rng.uniform(-8, 8, 2_000_000).astype(np.float32)
    mids = 0.5 * (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:])
    m32 = mids.astype(np.float32)
    extra = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(10)),
                            E2M1_MAGNITUDES.astype(np.float32)])
    extra = np.concatenate([extra, -extra, np.array([0.0, -0.0, 1e-40, -1e-40, 7.0, 1e38], np.float32)])
    v = np.concatenate([v, extra])
    assert np.array_equal(e2m1_encode(v), _e2m1_argmin(v))


def test_e2m1_decode_encode_roundtrip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(e2m1_encode(e2m1_decode(codes).astype(np.float32)), codes)


def test_pack_order_low_nibble_first():
    assert pack_nibbles(np.array([0x1, 0xF], np.uint8)).tolist() == [0xF1]
    c = np.random.default_rng(1).integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(unpack_nibbles(pack_nibbles(c)), c)


def test_e4m3_hand_cases():
    cases = json.load(open(os.path.join(GOLD, "e4m3_cases.json")))["cases"]
    v = np.array([c[0] for c in cases], np.float64).astype(np.float32)
    want = np.array([int(c[1], 16) for c in cases], np.uint8)
    assert np.array_equal(e4m3_encode_sat(v), want)


def test_e4m3_decode_known():
    assert e4m3_decode(0x7E) == 448.0
    assert e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x08) == 2.0 ** -6
    assert e4m3_decode(0x38) == 1.0
    assert np.isnan(e4m3_decode(0x7F))
    assert e4m3_decode(0xB8) == -1.0


def test_e4m3_against_torch_cast():
    """Special case reducing to a library routine: torch's RNE cast on values clamped to 448."""
    rng = np.random.default_rng(3)
    v = np.concatenate([
        np.exp(rng.uniform(np.log(1e-4), np.log(600), 1_000_000)),
        rng.uniform(0, 2.0 ** -6, 100_000),
        e4m3_decode(np.arange(0x7F)),                                  # every grid point
        0.5 * (e4m3_decode(np.arange(0x7E)) + e4m3_decode(np.arange(1, 0x7F))),   # every midpoint
    ]).astype(np.float32)
    ref = torch.from_numpy(np.minimum(v, np.float32(448.0))).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode_sat(v), ref)


def test_e4m3_saturates_and_rejects():
    assert e4m3_encode_sat(np.array([np.inf], np.float32)).tolist() == [0x7E]
    with pytest.raises(ValueError):
        e4m3_encode_sat(np.array([-1.0], np.float32))
    with pytest.raises(ValueError):
        e4m3_encode_sat(np.array([np.nan], np.float32))


def test_bf16_against_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-45], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x), ref)
    assert np.array_equal(bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())
