"""Oracle e4m3fn codec against torch's float8_e4m3fn and the format's landmarks."""

import numpy as np
import pytest
import torch

from oracle import decode_e4m3fn, encode_e4m3fn_rne, E4M3_MAX


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3fn(codes)
    ref = _torch_decode(codes)
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    # signed zeros are kept apart
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))


def test_format_landmarks():
    d = lambda c: float(decode_e4m3fn(np.array([c], dtype=np.uint8))[0])
    assert d(0x7E) == 448.0 == E4M3_MAX          # largest finite
    assert d(0x38) == 1.0
    assert d(0x08) == 2.0 ** -6                   # smallest normal
    assert d(0x01) == 2.0 ** -9                   # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9               # largest subnormal
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0xFE) == -448.0
    # no infinities anywhere
    assert not np.isinf(decode_e4m3fn(np.arange(256, dtype=np.uint8))).any()


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3fn_rne(decode_e4m3fn(codes)), codes)


def test_encoder_matches_torch_on_midpoints_and_random():
    """fp32 inputs (what the quantiser feeds): exact ties, their fp32
    neighbours, and random values over many magnitudes.  (torch narrows a
    float64 through float32 first, so float64 inputs would round twice.)"""
    vals = np.sort(decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)  # exact ties, exact in fp32
    nudged = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    rng = np.random.default_rng(7)
    rand = (rng.standard_normal(20000) * rng.choice([1e-3, 0.1, 1, 30, 300], 20000)).astype(np.float32)
    x = np.concatenate([nudged, -nudged, rand, np.array([0.0, -0.0, 447.9, 448.0, -448.0], np.float32)])
    # torch turns out-of-range values into NaN; the quantiser clamps to +-448
    # before encoding, so compare on the representable range only.
    x = x[np.abs(x) <= 448.0]
    ours = encode_e4m3fn_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encoder_saturates():
    out = encode_e4m3fn_rne(np.array([1e6, -1e6, 460.0, -500.0]))
    assert list(out) == [0x7E, 0xFE, 0x7E, 0xFE]


def test_decode_rejects_wrong_dtype():
    with pytest.raises(TypeError):
        decode_e4m3fn(np.arange(4, dtype=np.int32))
