"""Pins of the oracle's E4M3FN codec and tile quantiser.

Independent checks: the landmark values of the OCP OFP8 specification
(tests/golden/e4m3_ocp_values.json), torch's own float8_e4m3fn conversion
(a separate implementation of the same format), exhaustive round trips over
all 256 codes, and round-half-to-even at every midpoint.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_ocp_landmark_values(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_ocp_values.json")) as f:
        fx = json.load(f)
    for row in fx["codes"]:
        c = int(row["code"], 16)
        v = e4m3.e4m3_value(c)
        if row["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == row["value"], row


def test_decode_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_round_trip_all_codes():
    vals = e4m3.DECODE_TABLE[FINITE]
    back = e4m3.e4m3_encode_rne(vals)
    assert np.array_equal(back, np.array(FINITE, dtype=np.uint8))


def test_positive_values_increase_with_code():
    pos = e4m3.DECODE_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_midpoints_round_to_even_code():
    pos = e4m3.DECODE_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2               # exact in fp64
    got = e4m3.e4m3_encode_rne(mids).astype(int)
    lo = np.arange(len(mids))
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    # and the negative side mirrors it with the sign bit
    assert np.array_equal(e4m3.e4m3_encode_rne(-mids).astype(int), want | 0x80)


def test_saturation_and_tiny_values():
    enc = e4m3.e4m3_encode_rne
    assert enc(np.array([449.0, 1000.0, 1e30]))[0] == 0x7E
    assert np.all(enc(np.array([449.0, 1000.0, 1e30])) == 0x7E)
    assert np.all(enc(np.array([-449.0, -1e9])) == 0xFE)
    assert enc(np.array([2.0 ** -10]))[0] == 0x00            # half of 2^-9 ties to 0
    assert enc(np.array([3 * 2.0 ** -11]))[0] == 0x01        # 0.75 * 2^-9 -> 2^-9
    assert enc(np.array([1.0625]))[0] == 0x38                # between 1 and 1.125: tie -> even (1.0)
    assert enc(np.array([1.1875]))[0] == 0x3A                # between 1.125 and 1.25: tie -> 1.25


def test_encode_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.normal(0, 1, 20000),
        rng.normal(0, 100, 20000),
        rng.uniform(-463, 463, 20000),
        rng.normal(0, 2.0 ** -8, 20000),
    ]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.e4m3_encode_rne(x), ref)


def test_quantize_zero_tile_has_unit_scale():
    q, sc = e4m3.quantize_tiles(np.zeros((2, 256)), 1, 128)
    assert np.all(sc == 1.0) and np.all(q == 0)


def test_pow2_scale_definition():
    # smallest power of two with amax <= 448 * scale
    assert e4m3.pow2_scale(448.0) == 1.0
    assert e4m3.pow2_scale(448.0001) == 2.0
    assert e4m3.pow2_scale(224.0) == 0.5
    assert e4m3.pow2_scale(225.0) == 1.0
    assert e4m3.pow2_scale(1.0) == 2.0 ** -8          # 448 * 2^-9 = 0.875 < 1 <= 1.75
    assert e4m3.pow2_scale(0.0) == 1.0
    assert e4m3.pow2_scale(1e-45) == 2.0 ** -126


def test_vectorised_pow2_scale_matches_search():
    rng = np.random.default_rng(21)
    amax = np.concatenate([
        np.abs(rng.standard_t(2, 3000)) * np.exp2(rng.integers(-40, 40, 3000)),
        448.0 * np.exp2(np.arange(-30, 30)), 0.875 * 448.0 * np.exp2(np.arange(-5, 5)),
        np.nextafter(448.0 * np.exp2(np.arange(-5, 5)), np.inf), [0.0, 1e-45, 1e-39],
    ]).astype(np.float32).astype(np.float64)
    got = e4m3.pow2_scales(amax)
    want = np.array([e4m3.pow2_scale(float(a)) for a in amax])
    assert np.array_equal(got, want)


def test_quantize_tiles_scale_and_codes_match_torch():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (256, 384)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (256, 1))).astype(np.float32)
    x[5, :128] = 0.0
    for tr, tc in ((1, 128), (128, 128)):
        q, sc = e4m3.quantize_tiles(x, tr, tc)
        assert sc.dtype == np.float32 and sc.shape == (256 // tr, 384 // tc)
        amax = np.abs(x.reshape(256 // tr, tr, 3, tc)).max(axis=(1, 3)).astype(np.float64)
        # scales are powers of two and put amax in (224, 448] (or 1 for a zero tile)
        m, _ = np.frexp(sc.astype(np.float64))
        assert np.all(m == 0.5)
        nz = amax > 0
        ratio = amax[nz] / sc[nz]
        assert np.all(ratio <= 448.0) and np.all(ratio > 224.0)
        assert np.all(sc[~nz] == 1.0)
        # codes: torch's own E4M3 conversion of the (exactly) scaled values
        scaled = torch.from_numpy(x.astype(np.float64)) / torch.from_numpy(np.repeat(np.repeat(sc, tr, 0), tc, 1).astype(np.float64))
        ref = scaled.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, ref)


def test_dequantize_error_within_half_ulp():
    rng = np.random.default_rng(11)
    x = rng.standard_t(3, (64, 512)).astype(np.float32)
    q, sc = e4m3.quantize_tiles(x, 1, 128)
    deq = e4m3.dequantize_tiles(q, sc, 1, 128)
    s = np.repeat(sc.astype(np.float64), 128, axis=1)
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s)   # half an ulp, normal or subnormal
    assert np.all(err <= bound)


def test_quantize_rejects_ragged_shapes():
    with pytest.raises(ValueError):
        e4m3.quantize_tiles(np.zeros((3, 100)), 1, 128)
    with pytest.raises(ValueError):
        e4m3.quantize_tiles(np.zeros((100, 128)), 128, 128)
