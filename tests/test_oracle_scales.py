"""Pins for the oracle's scale bookkeeping (CPU only).

Pinned against: the printed scale-file example values (vLLM page "FP8 ViT
Encoder Attention", Scale File Format) divided by 448 with exact rational
arithmetic (tests/golden/descale_examples.txt), the 1e-10 floor of the
atrex-bench per_token_group_quant_fp8 formula, and closed forms of the
16-slot sliding maximum.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import scales
from tests.golden.make_descale_examples import rn_fp32


def _bits(x):
    return int(np.float32(x).view(np.uint32))


def test_descale_printed_example(golden_dir):
    with open(os.path.join(golden_dir, "descale_examples.txt")) as f:
        rows = [ln.split() for ln in f if not ln.startswith("#")]
    assert len(rows) == 6
    for val, bits, _ in rows:
        assert _bits(scales.descale_from_amax(float(val))) == int(bits, 16)
    # closed forms visible by eye
    assert scales.descale_from_amax(224.0) == np.float32(0.5)
    assert scales.descale_from_amax(210.0) == np.float32(15 / 32)


def test_descale_is_correctly_rounded_division():
    rng = np.random.default_rng(2)
    A = (rng.uniform(1, 2, 2000) * np.exp2(rng.integers(-20, 40, 2000))).astype(np.float32)
    for a in A:
        assert _bits(scales.descale_from_amax(a)) == rn_fp32(Fraction(float(a)) / 448)


def test_descale_floor():
    assert scales.descale_from_amax(0.0) == np.float32(1e-10)
    assert scales.descale_from_amax(4.0e-8) == np.float32(1e-10)       # 4e-8/448 < 1e-10
    assert scales.descale_from_amax(1.0e-7) > np.float32(1e-10)


def _window_closed_form(seq, t):
    """Max of the last 16 observations up to and including t (zeros before start)."""
    return max(seq[max(0, t - 15): t + 1])


@pytest.mark.parametrize("pattern", ["ramp_up", "ramp_down", "spike", "zeros"])
def test_ring_sliding_max(pattern):
    n = 40
    if pattern == "ramp_up":
        seq = [float(t + 1) for t in range(n)]
    elif pattern == "ramp_down":
        seq = [float(100 - t) for t in range(n)]
    elif pattern == "spike":
        seq = [1000.0 if t == 3 else 1.0 for t in range(n)]
    else:
        seq = [0.0] * n
    ring = scales.AmaxRing()
    for t in range(n):
        got = ring.push([seq[t], 2 * seq[t], 0.5 * seq[t]])
        assert got[0] == np.float32(_window_closed_form(seq, t))
        assert got[1] == np.float32(2 * _window_closed_form(seq, t))
        assert got[2] == np.float32(0.5 * _window_closed_form(seq, t))
    if pattern == "ramp_up":
        assert ring.window_max()[0] == n            # current value always wins
    if pattern == "ramp_down":
        assert ring.window_max()[0] == 100 - (n - 16)   # value 15 steps back
    assert ring.count == n


def test_spike_visible_exactly_16_forwards():
    ring = scales.AmaxRing()
    seen = []
    for t in range(25):
        a = 1000.0 if t == 3 else 1.0
        seen.append(float(ring.push([a, a, a])[0]))
    assert all(seen[t] == 1000.0 for t in range(3, 19))
    assert seen[19] == 1.0 and seen[2] == 1.0


def test_first_forward_uses_its_own_amax():
    ring = scales.AmaxRing()
    d = scales.dynamic_descales(ring, [224.0, 198.0, 210.0])
    assert d[0] == np.float32(0.5) and d[2] == np.float32(15 / 32)


def test_static_path_no_extra_margin_and_calibration():
    d = scales.static_descales([224.0, 198.0, 210.0])
    assert d[0] == np.float32(0.5)
    ring = scales.AmaxRing()
    for t in range(16):
        ring.push([1.0 + t, 2.0, 3.0 + (t == 7) * 10])
    v = scales.calibrated_values(ring, 1.5)
    assert list(v) == [np.float32(24.0), np.float32(3.0), np.float32(19.5)]
