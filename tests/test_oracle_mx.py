"""Pins of the block-scaled (MX) e4m3 oracle (oracle/mx.py) against brute
force, a closed-form special case shared with the per-tensor path, and the
block structure. Mutation checks plant plausible mistakes in a copy of the
oracle's arithmetic and require a pin to fail."""
import numpy as np
import pytest

import oracle
from oracle import e4m3, mx
from synth import f32_to_bf16_bits, make_qkv


def brute_scale_exponent(a: float) -> int:
    """Smallest s in [-127, 127] with 448 * 2^s >= a (a == 0 -> -127), by search."""
    if a == 0:
        return -127
    for s in range(-127, 128):
        if 448.0 * 2.0 ** s >= a:
            return s
    return 127


def brute_nearest(y: float, s: int) -> int:
    """Nearest of all finite e4m3 values times 2^s (ties to the even code), sign kept."""
    vals = e4m3.DECODE_TABLE[:0x7F] * 2.0 ** s
    a = abs(y)
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if np.signbit(y) else 0)


def test_scale_exponent_brute_force():
    rng = np.random.default_rng(0)
    amax = [0.0, 448.0, 448.0 * 2.0 ** -5, 1.75, 1.7578125, 0.875, 1e-38, 2.0 ** -130, 3.0e38]
    amax += list(np.abs(rng.standard_normal(200)) * 10.0 ** rng.integers(-30, 30, 200))
    amax = np.float32(amax).astype(np.float64)          # values the GPU sees are float32 (from bf16)
    got = mx.scale_exponent(amax)
    for a, s in zip(amax, got):
        assert int(s) == brute_scale_exponent(float(a)), a
        if a > 0 and s > -127:
            assert a <= 448.0 * 2.0 ** s and a > 448.0 * 2.0 ** (s - 1)   # the smallest such power of two


def test_elements_are_nearest_codes_without_saturation():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((3, 2, 72)) * np.exp(rng.normal(0, 3, (3, 2, 72)))).astype(np.float32)
    x[0, 0, :32] = 0.0                                   # an all-zero block
    x[1, 1, 64:] = x[1, 1, 64:] * 1e-30                  # a tiny partial block
    bits = f32_to_bf16_bits(x)
    codes, scales = mx.quantize(bits)
    xf = oracle.quant.bf16_to_f32(bits).astype(np.float64)
    for t in range(3):
        for h in range(2):
            for j in range(72):
                s = int(scales[t, h, j // 32]) - 127
                assert codes[t, h, j] == brute_nearest(xf[t, h, j], s), (t, h, j)
    deq = mx.dequantize(codes, scales)
    # no element saturates: the largest magnitude of every block is within e4m3's step of itself
    amax = mx.block_amax(xf)
    damax = mx.block_amax(deq)
    assert np.all(damax <= amax * (1 + 2.0 ** -4) + 1e-300)
    assert np.all(scales[..., 3] == 0)                   # head_dim 72: three blocks, pad byte 0
    assert np.all(scales[0, 0, 0] == 0) and np.all(codes[0, 0, :32] & 0x7F == 0)


def test_uniform_blocks_equal_the_per_tensor_path():
    """Closed-form special case: when every block's amax is 448 * 2^k, each block
    scale is 2^k, and the codes are the per-tensor path's codes with descale 2^k."""
    rng = np.random.default_rng(2)
    k = -4
    x = (rng.uniform(-1, 1, (5, 3, 128)) * 448.0 * 2.0 ** k).astype(np.float32)
    for b in range(4):
        x[:, :, 32 * b] = 448.0 * 2.0 ** k                # pin each block's amax
    bits = f32_to_bf16_bits(x)
    codes, scales = mx.quantize(bits)
    assert np.all(scales == 127 + k)
    assert np.array_equal(codes, oracle.quant.quantize(bits, np.float32(2.0 ** k)))


def test_block_structure():
    q, _, _ = make_qkv(3, 16, 2, 72)
    codes, scales = mx.quantize(q)
    q2 = q.copy()
    q2[5, 1, 40] = f32_to_bf16_bits(np.float32([1000.0]))[0]   # only block 1 of row (5, 1) changes
    c2, s2 = mx.quantize(q2)
    diff_rows = np.argwhere(np.any(c2 != codes, axis=-1))
    assert diff_rows.tolist() == [[5, 1]]
    assert s2[5, 1, 1] != scales[5, 1, 1] and s2[5, 1, 0] == scales[5, 1, 0] and s2[5, 1, 2] == scales[5, 1, 2]
    assert np.array_equal(c2[5, 1, :32], codes[5, 1, :32]) and np.array_equal(c2[5, 1, 64:], codes[5, 1, 64:])
    # permuting elements inside a block permutes the codes
    p = q.copy()
    perm = np.random.default_rng(4).permutation(32)
    p[..., 32:64] = q[..., 32:64][..., perm]
    cp, sp = mx.quantize(p)
    assert np.array_equal(sp, scales) and np.array_equal(cp[..., 32:64], codes[..., 32:64][..., perm])


def test_mutations_fail_a_pin(monkeypatch):
    """A floor instead of the round-up (saturating block maxima), or 24-element
    blocks, must each fail one of the pins above."""
    orig = mx.scale_exponent

    def floor_rule(amax):
        a = np.asarray(amax, dtype=np.float64)
        s = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64) - 8
        return np.clip(np.where(a > 0, s, -127), -127, 127)
    monkeypatch.setattr(mx, "scale_exponent", floor_rule)
    with pytest.raises(AssertionError):
        test_scale_exponent_brute_force()
    monkeypatch.setattr(mx, "scale_exponent", orig)
    monkeypatch.setattr(mx, "BLOCK", 24)
    with pytest.raises(AssertionError):
        test_block_structure()
