"""Pins for the oracle's amax and quantization (CPU only).

Pinned against: exact rational arithmetic (fractions) for the division and the
nearest-even choice, torch's float8_e4m3fn cast (a library routine the oracle
does not use), brute-force max, and invariants of per-tensor scaling.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, quant, scales
from synth import f32_to_bf16_bits, make_qkv
from tests.golden.make_descale_examples import rn_fp32

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE_BF16 = ALL_BF16[np.isfinite(quant.bf16_to_f32(ALL_BF16))]

# descales: floor, powers of two, printed-example descales, awkward mantissas
DESCALES = [np.float32(1e-10), np.float32(2.0 ** -20), np.float32(1 / 448), np.float32(0.5),
            np.float32(198 / 448), np.float32(15 / 32), np.float32(0.0091552734375),
            np.float32(1.2345678e-3), np.float32(3.3333333), np.float32(0.99999994), np.float32(7.0e5)]


def test_bf16_widening_exact():
    x = np.float32([1.0, -2.5, 3.140625, 0.0, -0.0])
    assert np.array_equal(quant.bf16_to_f32(f32_to_bf16_bits(x)), x)


def test_amax_brute_force():
    q, k, v = make_qkv(7, 37, 3, 8, outlier_frac=0.01)
    for t in (q, k, v):
        vals = [abs(float(x)) for x in quant.bf16_to_f32(t).ravel()]
        assert quant.amax(t) == np.float32(max(vals))
    assert quant.amax(np.zeros((0, 3, 8), np.uint16)) == 0.0


@pytest.mark.parametrize("descale", DESCALES)
def test_quantize_all_bf16_matches_torch_formula(descale):
    ours = quant.quantize(FINITE_BF16, descale)
    x = torch.from_numpy(quant.bf16_to_f32(FINITE_BF16))
    ref = (x / torch.tensor(descale, dtype=torch.float32)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    assert np.array_equal(ours, ref.view(torch.uint8).numpy())


def _exact_code(x: float, d: float) -> int:
    """Exact-arithmetic reference for one element: RN_fp32(x/d), clamp, nearest-even code."""
    if x == 0.0:
        return 0x80 if np.signbit(np.float32(x)) else 0x00
    qf = Fraction(abs(x)) / Fraction(float(d))
    if qf >= Fraction(2) ** 128:
        y = Fraction(448)
    else:
        b = rn_fp32(qf) if qf >= Fraction(2) ** -126 else None
        if b is None:                           # subnormal fp32 quotient -> far below e4m3 range
            y = Fraction(0)
        else:
            y = Fraction(float(np.uint32(b).view(np.float32)))
        y = min(y, Fraction(448))
    cands = [(abs(Fraction(float(e4m3.DECODE_TABLE[c])) - y), c) for c in range(0x7F)]
    best = min(c[0] for c in cands)
    codes = [c for dist, c in cands if dist == best]
    code = codes[0] if len(codes) == 1 else [c for c in codes if c % 2 == 0][0]
    return code | (0x80 if x < 0 else 0)


def test_quantize_exact_rational_sample():
    rng = np.random.default_rng(3)
    idx = rng.choice(len(FINITE_BF16), 400, replace=False)
    for d in (np.float32(198 / 448), np.float32(1.2345678e-3), np.float32(1e-10)):
        got = quant.quantize(FINITE_BF16[idx], d)
        xs = quant.bf16_to_f32(FINITE_BF16[idx])
        for xi, gi in zip(xs, got):
            assert gi == _exact_code(float(xi), d), (xi, d, gi)


def test_zero_tensor_floor_path():
    z = np.zeros((4, 2, 8), np.uint16)
    d = scales.descale_from_amax(quant.amax(z))
    assert d == np.float32(1e-10)
    assert np.all(quant.quantize(z, d) == 0)


def test_per_tensor_invariants():
    q, _, _ = make_qkv(11, 64, 2, 8)
    d = scales.descale_from_amax(quant.amax(q))
    c = quant.quantize(q, d)
    # amax element maps to +-448 exactly
    x = quant.bf16_to_f32(q)
    i = np.argmax(np.abs(x))
    assert c.ravel()[i] & 0x7F == 0x7E
    # doubling the tensor doubles amax and descale exactly: identical codes
    q2 = f32_to_bf16_bits(x * np.float32(2))
    d2 = scales.descale_from_amax(quant.amax(q2))
    assert d2 == 2 * d
    assert np.array_equal(quant.quantize(q2, d2), c)
    # permuting elements permutes codes
    perm = np.random.default_rng(0).permutation(q.size)
    assert np.array_equal(quant.quantize(q.ravel()[perm], d), c.ravel()[perm])


def test_dequantize_exact():
    codes = np.arange(256, dtype=np.uint8)
    d = np.float32(198 / 448)
    v = quant.dequantize(codes, d)
    fin = ~np.isnan(v)
    for c in np.nonzero(fin)[0][::7]:
        assert Fraction(float(v[c])) == Fraction(float(e4m3.DECODE_TABLE[c])) * Fraction(float(d))


def test_quantize_f32_matches_torch_formula_and_exact_rationals():
    """quantize_f32 (used for the fp8 attention output) on fp32 values with full
    24-bit mantissas: torch's float8 cast of the same formula, and the exact
    rational reference on a sample."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 4, 20000)).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 448.0, -1e30, 3.4e38])])
    for d in (np.float32(1e-10), np.float32(0.0123456), np.float32(3.3333333), np.float32(0.5)):
        ours = quant.quantize_f32(x, d)
        ref = (torch.from_numpy(x) / torch.tensor(d)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        assert np.array_equal(ours, ref.view(torch.uint8).numpy())
        for xi, gi in zip(x[:300], ours[:300]):
            assert gi == _exact_code(float(xi), d), (xi, d, gi)


def test_quantize_f32_agrees_with_bf16_path():
    for d in DESCALES:
        assert np.array_equal(quant.quantize_f32(quant.bf16_to_f32(FINITE_BF16), d), quant.quantize(FINITE_BF16, d))
