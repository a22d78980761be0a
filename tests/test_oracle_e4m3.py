"""Pins for the oracle's e4m3 codec (CPU only).

Pinned against: the OCP e4m3fn constants, torch's own float8_e4m3fn cast (a
library routine the oracle does not use), and brute-force nearest-code search.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(y32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_spec_constants():
    t = e4m3.DECODE_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0 and t[0x40] == 2.0
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2


def test_decode_matches_torch_all_codes():
    ours, ref = e4m3.DECODE_TABLE, torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _fp32_neighbours(x):
    x = np.asarray(x, dtype=np.float32)
    return np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))])


def test_encode_matches_torch_on_ties_and_random():
    pos = e4m3.DECODE_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0            # every rounding boundary (exact in fp32)
    pts = np.concatenate([pos, mids]).astype(np.float32)
    pts = _fp32_neighbours(pts)
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-14, 9, 200_000))).astype(np.float32)
    y = np.concatenate([pts, -pts, rnd, np.float32([0.0, -0.0])])
    y = y[np.abs(y) <= 448.0]
    assert np.array_equal(e4m3.encode_rne(y), torch_encode(y))


def test_encode_matches_torch_all_bf16_in_range():
    b = np.arange(65536, dtype=np.uint32)
    y = (b << np.uint32(16)).view(np.float32)
    y = y[np.isfinite(y) & (np.abs(y) <= 448.0)]
    assert np.array_equal(e4m3.encode_rne(y), torch_encode(y))


def test_encode_brute_force_nearest_even():
    finite_codes = np.array([c for c in range(256) if not np.isnan(e4m3.DECODE_TABLE[c])])
    vals = e4m3.DECODE_TABLE[finite_codes]
    rng = np.random.default_rng(1)
    y = np.concatenate([(rng.uniform(-1, 1, 3000) * np.exp2(rng.uniform(-12, 8.8, 3000))),
                        (e4m3.DECODE_TABLE[:0x7E] + e4m3.DECODE_TABLE[1:0x7F]) / 2]).astype(np.float32)
    got = e4m3.encode_rne(y)
    for yi, gi in zip(y, got):
        d = np.abs(vals - np.float64(yi))
        best = finite_codes[d == d.min()]
        if len(best) > 1:                       # tie (or +-0): even mantissa, sign of y
            best = [c for c in best if c % 2 == 0 and (c >= 0x80) == bool(np.signbit(yi))] or best
        assert gi in best and (gi % 2 == 0 or len(best) == 1), (yi, gi, best)
        assert bool(gi & 0x80) == bool(np.signbit(yi))


def test_sign_kept_on_underflow_and_saturation():
    y = np.float32([-1e-30, -0.0009765625, 0.0009765625, 500.0, -1e9, 447.99, 432.0, 431.99997])
    got = e4m3.encode_rne(y)
    assert list(got) == [0x80, 0x80, 0x00, 0x7E, 0xFE, 0x7E, 0x7E, 0x7D]
