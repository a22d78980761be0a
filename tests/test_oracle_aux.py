"""Pins of the oracle's diagnostics: the saturation count (oracle.quant) and
the cu_seqlens validity bits (oracle.varlen), against closed forms, exact
rational arithmetic and hand-made cases; plus planted mistakes that must fail
a pin."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, varlen
from synth import f32_to_bf16_bits


def _all_bf16_in(lo_exp, hi_exp):
    """Every positive bf16 value in [2^lo_exp, 2^hi_exp) and its negative, as bits."""
    vals = [2.0 ** e * (1 + m / 128) for e in range(lo_exp, hi_exp) for m in range(128)]
    x = np.array(vals + [-v for v in vals], dtype=np.float32)
    return f32_to_bf16_bits(x)


def test_saturated_count_closed_form():
    # descale 2^-3: quotient = 8 x exactly; clamped iff |x| > 56 = 1.75 * 2^5.
    # In [32, 64) the values 32 (1 + m/128) > 56 are m = 97..127 (31 of them);
    # [64, 1024) holds 4 * 128 more; both signs.
    bits = _all_bf16_in(0, 10)
    assert quant.saturated_count(bits, np.float32(0.125)) == 2 * (31 + 4 * 128)
    # exactly 448 is not clamped; the next bf16 value up is
    assert quant.saturated_count(f32_to_bf16_bits(np.array([56.0, -56.0], np.float32)), np.float32(0.125)) == 0
    assert quant.saturated_count(f32_to_bf16_bits(np.array([56.25, -56.25], np.float32)), np.float32(0.125)) == 2
    assert quant.saturated_count(np.zeros(0, np.uint16), np.float32(1.0)) == 0


def _exact_count(bits, d):
    """Clamped iff the fp32 quotient exceeds 448: with RNE, iff the exact
    quotient exceeds 448 + half an fp32 ulp at 448 (2^-16; the tie rounds to
    448, whose significand is even)."""
    x = quant.bf16_to_f32(bits)
    lim = Fraction(448) + Fraction(1, 2 ** 16)
    dd = Fraction(float(np.float32(d)))
    return sum(1 for v in x.reshape(-1) if abs(Fraction(float(v)) / dd) > lim)


@pytest.mark.parametrize("d", [0.3, 1.0 / 3.0, 0.0071, 2.5e-4])
def test_saturated_count_exact_rationals(d):
    rng = np.random.default_rng(int(d * 1e6))
    d32 = np.float32(d)
    # values spread around the clamp point 448 * d, plus the bf16 neighbours of it
    x = (448 * d32 * rng.uniform(0.9, 1.1, 400)).astype(np.float32) * rng.choice([-1, 1], 400).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    c = int(np.float32(448 * d32).view(np.uint32) >> 16)
    near = np.array([c - 1, c, c + 1, c + 2, (c - 1) | 0x8000, c | 0x8000, (c + 1) | 0x8000], np.uint16)
    bits = np.concatenate([bits, near])
    assert quant.saturated_count(bits, d32) == _exact_count(bits, d32)


CU_CASES = [
    # (cu, T, max_seqlen, bits)
    ([0, 3, 3, 10], 10, 7, 0),
    ([0], 0, 0, 0),
    ([0, 0, 0], 0, 0, 0),
    ([1, 3, 10], 10, 7, varlen.CU_FIRST_NOT_ZERO),
    ([0, 5, 4, 10], 10, 6, varlen.CU_DECREASING),
    ([0, 3, 9], 10, 7, varlen.CU_LAST_NOT_T),
    ([0, 3, 11], 10, 8, varlen.CU_LAST_NOT_T),
    ([0, 3, 10], 10, 6, varlen.CU_LONGER_THAN_MAX),
    ([2, 1, 12], 10, 3, varlen.CU_FIRST_NOT_ZERO | varlen.CU_DECREASING | varlen.CU_LAST_NOT_T
     | varlen.CU_LONGER_THAN_MAX),
]


@pytest.mark.parametrize("cu,T,m,bits", CU_CASES)
def test_cu_seqlens_errors_cases(cu, T, m, bits):
    assert varlen.cu_seqlens_errors(cu, T, m) == bits


def test_planted_mistakes_fail_a_pin(monkeypatch):
    def fails(fn, *a):
        try:
            fn(*a)
        except AssertionError:
            return True
        return False

    orig = quant.saturated_count
    # >= 448 instead of > 448
    monkeypatch.setattr(quant, "saturated_count",
                        lambda b, d: orig(b, d) + int(np.count_nonzero(
                            np.abs((quant.bf16_to_f32(b) / np.float32(d)).astype(np.float32)) == 448)))
    assert fails(test_saturated_count_closed_form)
    # threshold applied to x instead of x / descale
    monkeypatch.setattr(quant, "saturated_count",
                        lambda b, d: int(np.count_nonzero(np.abs(quant.bf16_to_f32(b)) > 448)))
    assert fails(test_saturated_count_closed_form)
    monkeypatch.setattr(quant, "saturated_count", orig)
    # a check that forgets the length bound
    orig_cu = varlen.cu_seqlens_errors
    monkeypatch.setattr(varlen, "cu_seqlens_errors",
                        lambda cu, T, m: orig_cu(cu, T, 1 << 30))
    assert fails(test_cu_seqlens_errors_cases, [0, 3, 10], 10, 6, varlen.CU_LONGER_THAN_MAX)
