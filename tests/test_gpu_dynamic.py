"""Dynamic mode's two passes against the oracle's ring, forward by forward.

Pass 1 quantizes at the window over the other 15 ring slots; pass 2 redoes a
tensor only where this forward's amax changes the descale. The inputs here are
one seeded tensor triple scaled by powers of two (exact in bf16), so the
sequence forces both branches: a growing amax (redo), a repeated or smaller
amax (no redo), a single tensor raising its window (redo of that tensor only),
and the ring wrapping around. Codes, descales, ring and count must equal the
oracle's after every forward, with the clamp counts on."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_qkv
from tests.gpu_helpers import codes_np, f32bits, fv, require_gpu, to_dev

pytestmark = pytest.mark.gpu

# per forward: power-of-two exponent applied to q, k, v
SEQ = [(0, 0, 0), (1, 1, 1), (1, 1, 1), (0, 0, 0), (-2, -2, -2), (2, 0, 0), (0, 3, 0), (0, 0, -4)] + \
      [(k % 3 - 1, (k * 5) % 4 - 2, 0) for k in range(14)] + [(5, 5, 5), (0, 0, 0)]


def _scaled(bits, e):
    x = oracle.quant.bf16_to_f32(bits) * np.float32(2.0 ** e)
    return (x.view(np.uint32) >> 16).astype(np.uint16)   # exact: a power-of-two scale of bf16 values


@pytest.mark.parametrize("H,d", [(4, 72), (2, 128)])
def test_dynamic_sequence_matches_oracle(H, d):
    dev = require_gpu()
    T = 513
    base = make_qkv(300 + d, T, H, d, outlier_frac=0.002)
    st = fv.new_state(dev)
    fv.state_set_flags(st, fv.FP8VIT_FLAG_COUNT_SATURATION)
    ring = oracle.scales.AmaxRing()
    sat = np.zeros(3, np.int64)
    for i, ex in enumerate(SEQ):
        bits = [_scaled(b, e) for b, e in zip(base, ex)]
        got = fv.quantize_qkv(*(to_dev(b, dev) for b in bits), st, "dynamic")
        codes, ds, _ = oracle.pipeline.quantize_step(*bits, "dynamic", ring=ring)
        for name, g, c in zip("qkv", got, codes):
            assert np.array_equal(codes_np(g), c), (i, name)
        view = fv.state_read(st)
        assert np.array_equal(f32bits(view["descale_used"]), f32bits(ds)), i
        assert np.array_equal(f32bits(view["ring"]), f32bits(ring.ring)) and view["count"] == ring.count, i
        sat += [oracle.quant.saturated_count(b, dd) for b, dd in zip(bits, ds)]
        assert view["saturated"] == sat.tolist(), i


def test_dynamic_mx_v_pass_sequence():
    """The block-scaled quantizer's V pass follows the same ring (all three
    amaxes enter it; only V is quantized per tensor)."""
    dev = require_gpu()
    T, H, d = 300, 3, 72
    base = make_qkv(77, T, H, d)
    st = fv.new_state(dev)
    ring = oracle.scales.AmaxRing()
    for i, ex in enumerate(SEQ[:10]):
        bits = [_scaled(b, e) for b, e in zip(base, ex)]
        q8, k8, v8, qs, ks = fv.quantize_qkv_mx(*(to_dev(b, dev) for b in bits), st, "dynamic")
        ref = oracle.pipeline.forward_mx(*bits, None, "dynamic", ring=ring, attend=False)
        assert np.array_equal(codes_np(v8), ref.v_codes), i
        assert np.array_equal(codes_np(q8), ref.q[0]) and np.array_equal(codes_np(ks), ref.k[1]), i
        assert np.float32(fv.state_read(st)["descale_used"][2]) == ref.v_descale, i
        assert np.array_equal(f32bits(fv.state_read(st)["ring"]), f32bits(ring.ring)), i
