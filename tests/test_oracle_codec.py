"""Pins of the oracle's number codecs against the OCP FP8 table and torch's own casts.

The oracle's e4m3 decoder/encoder and its bf16/fp16 rounding are checked
against values fixed outside the oracle: the OCP FP8 specification's special
values (tests/golden/e4m3_special_values.json) and torch's CPU conversions
(``float8_e4m3fn``, ``bfloat16``, ``float16``), which round to nearest even.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _torch_e4m3_encode(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    want = _torch_e4m3_decode(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert nan.sum() == 2  # 0x7F and 0xFF only


def test_e4m3_special_values_from_spec(orc):
    spec = json.load(open(os.path.join(GOLD, "e4m3_special_values.json")))
    for row in spec["decode"]:
        v = orc.e4m3_decode(np.array([int(row["code"], 16)], np.uint8))[0]
        if row["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == row["value"] and math.copysign(1, v) == math.copysign(1, row["value"])
    for row in spec["encode_rne"]:
        c = orc.e4m3_encode(np.array([row["value"]], np.float32))[0]
        assert c == int(row["code"], 16), row


def test_e4m3_encode_strided_fp32_space_matches_torch(orc):
    # every 97th fp32 bit pattern with |v| <= 448 (positive and negative), ~23.5M values
    top = np.float32(448.0).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 97, dtype=np.uint32)
    for sign in (0, 0x80000000):
        v = (bits | np.uint32(sign)).view(np.float32)
        got = orc.e4m3_encode(v)
        want = _torch_e4m3_encode(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_encode_near_every_midpoint_matches_torch(orc):
    # exhaustive +-64 ulps around every midpoint between adjacent finite codes, and around each code
    vals = _torch_e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    centers = np.concatenate([vals, mids])
    offs = np.arange(-64, 65, dtype=np.int64)
    b = centers.view(np.uint32).astype(np.int64)[:, None] + offs[None, :]
    b = b[(b >= 0) & (b <= np.int64(np.float32(448.0).view(np.uint32)))].astype(np.uint32)
    for sign in (0, 0x80000000):
        v = (b | np.uint32(sign)).view(np.float32)
        assert np.array_equal(orc.e4m3_encode(v), _torch_e4m3_encode(v))


def test_e4m3_encode_saturates_like_clamped_torch(orc):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(448, 1e6, 10000), -rng.uniform(448, 1e6, 10000),
                        [448.0, 449.0, 463.99, 464.0, 465.0, 1e38, -1e38]]).astype(np.float32)
    got = orc.e4m3_encode(v)
    want = _torch_e4m3_encode(np.clip(v, -448, 448))
    assert np.array_equal(got, want)
    assert set(np.unique(got)) <= {0x7E, 0xFE}


def test_bf16_encode_matches_torch(orc):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    v = np.concatenate([v, np.array([0.0, -0.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38], np.float32)])
    got = orc.bf16_encode(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_encode_matches_torch(orc):
    rng = np.random.default_rng(6)
    v = np.concatenate([
        rng.standard_normal(500_000).astype(np.float32) * np.exp2(rng.integers(-30, 18, 500_000)).astype(np.float32),
        np.array([65504.0, 65519.99, 65520.0, 70000.0, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8, 0.0, -0.0], np.float32),
    ]).astype(np.float32)
    got = orc.f16_encode(v)
    want = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
