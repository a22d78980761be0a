"""Pins for the oracle's fp64 varlen attention and the full pipeline (CPU only).

Pinned against: pure-Python brute force (math.exp / math.fsum loops) on tiny
inputs, torch's scaled_dot_product_attention in fp64 per segment (a library
routine the oracle does not use), closed forms and invariants. The pages print
no attention output values, so there is nothing printed to pin against.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, pipeline, quant, scales
from synth import f32_to_bf16_bits, make_qkv, make_cu_seqlens

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def brute_force(q, k, v, cu, sigma):
    T, H, d = q.shape
    out = np.zeros_like(q, dtype=np.float64)
    for i in range(len(cu) - 1):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        for h in range(H):
            for t in range(s0, s1):
                scores = [math.fsum(float(q[t, h, c]) * float(k[j, h, c]) for c in range(d)) * sigma
                          for j in range(s0, s1)]
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = math.fsum(w)
                for c in range(v.shape[2]):
                    out[t, h, c] = math.fsum(w[j - s0] * float(v[j, h, c]) for j in range(s0, s1)) / z
    return out


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("seglens", [(5,), (3, 0, 4, 1), (2, 6, 3)])
def test_attention_brute_force(seglens):
    cu = make_cu_seqlens(seglens)
    T = int(cu[-1])
    q, k, v = rand((T, 2, 5), 1), rand((T, 2, 5), 2), rand((T, 2, 5), 3)
    sigma = float(np.float32(0.37))
    got = attention.attention(q, k, v, cu, softmax_scale=np.float32(0.37))
    ref = brute_force(q, k, v, cu, sigma)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_attention_matches_torch_sdpa():
    seglens = (17, 1, 40, 0, 9)
    cu = make_cu_seqlens(seglens)
    T, H, d = int(cu[-1]), 3, 72
    q, k, v = rand((T, H, d), 4), rand((T, H, d), 5), rand((T, H, d), 6)
    got = attention.attention(q, k, v, cu)
    sigma = float(attention.default_softmax_scale(d))
    for i in range(len(seglens)):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        if s1 == s0:
            continue
        tq = torch.from_numpy(q[s0:s1]).permute(1, 0, 2)
        tk = torch.from_numpy(k[s0:s1]).permute(1, 0, 2)
        tv = torch.from_numpy(v[s0:s1]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sigma).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[s0:s1], ref, rtol=1e-10, atol=1e-12)


def test_default_scale():
    assert attention.default_softmax_scale(72) == np.float32(1 / math.sqrt(72))
    assert attention.default_softmax_scale(128) == np.float32(0.08838834764831845)


def test_invariants():
    seglens = (7, 1, 12, 0, 5)
    cu = make_cu_seqlens(seglens)
    T, H, d = int(cu[-1]), 2, 8
    q, k, v = rand((T, H, d), 7), rand((T, H, d), 8), rand((T, H, d), 9)
    base = attention.attention(q, k, v, cu)
    # equal keys -> segment mean of V
    k_eq = k.copy()
    for i in range(len(seglens)):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        k_eq[s0:s1] = k[s0:s0 + 1] if s1 > s0 else k_eq[s0:s1]
    o = attention.attention(q, k_eq, v, cu)
    for i in range(len(seglens)):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        if s1 > s0:
            np.testing.assert_allclose(o[s0:s1], np.broadcast_to(v[s0:s1].mean(axis=0), o[s0:s1].shape), atol=1e-12)
    # one-token segment -> its v
    np.testing.assert_array_equal(base[7], v[7])
    # V == 1 -> 1
    np.testing.assert_allclose(attention.attention(q, k, np.ones_like(v), cu), 1.0, atol=1e-14)
    # Q == 0 -> segment mean of V
    oz = attention.attention(np.zeros_like(q), k, v, cu)
    np.testing.assert_allclose(oz[8:20], np.broadcast_to(v[8:20].mean(axis=0), (12, H, d)), atol=1e-12)
    # permuting segments leaves each segment's output unchanged
    order = [2, 4, 0, 3, 1]
    segs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(seglens))]
    idx = np.concatenate([np.arange(*segs[i]) for i in order])
    cu2 = make_cu_seqlens([seglens[i] for i in order])
    o2 = attention.attention(q[idx], k[idx], v[idx], cu2)
    np.testing.assert_allclose(o2, base[idx], rtol=1e-13, atol=1e-14)
    # heads are independent
    q3 = q.copy()
    q3[:, 1] = rand((T, d), 10)
    o3 = attention.attention(q3, k, v, cu)
    np.testing.assert_array_equal(o3[:, 0], base[:, 0])
    # zero-length segments are inert
    cu4 = make_cu_seqlens((7, 0, 0, 1, 12, 0, 5, 0))
    np.testing.assert_array_equal(attention.attention(q, k, v, cu4), base)


def test_attention_rows_match_full():
    seglens = (30, 50)
    cu = make_cu_seqlens(seglens)
    q, k, v = rand((80, 2, 8), 11), rand((80, 2, 8), 12), rand((80, 2, 8), 13)
    full = attention.attention(q, k, v, cu)
    rows = [(0, 0), (29, 1), (30, 0), (79, 1), (55, 0)]
    got = attention.attention_rows(q, k, v, cu, rows)
    for n, (t, h) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[t, h], rtol=1e-12, atol=1e-14)


def test_pipeline_dynamic_first_forward_and_scaling_invariant():
    cu = make_cu_seqlens((40, 24))
    q, k, v = make_qkv(21, 64, 2, 72)
    ring = scales.AmaxRing()
    r = pipeline.forward(q, k, v, cu, "dynamic", ring=ring)
    for x, d, c in zip((q, k, v), r.descales, r.codes):
        assert d == scales.descale_from_amax(quant.amax(x))
        assert np.array_equal(c, quant.quantize(x, d))
    # V x 2 (fresh ring): identical codes, output x 2 exactly
    v2 = f32_to_bf16_bits(quant.bf16_to_f32(v) * np.float32(2))
    r2 = pipeline.forward(q, k, v2, cu, "dynamic", ring=scales.AmaxRing())
    assert all(np.array_equal(a, b) for a, b in zip(r.codes, r2.codes))
    np.testing.assert_array_equal(r2.out, 2 * r.out)


def test_pipeline_error_vs_unquantized_in_expected_band():
    """The quantize-then-attend oracle must sit a few percent from fp64 attention
    on N(0,1) data (e4m3 keeps 3 mantissa bits); a transposed operand, a dropped
    scale or a wrong segment table lands far outside this band."""
    cu = make_cu_seqlens((256,))
    q, k, v = make_qkv(1, 256, 4, 72)
    r = pipeline.forward(q, k, v, cu, "dynamic", ring=scales.AmaxRing())
    ref = pipeline.reference_unquantized(q, k, v, cu)
    rel = np.linalg.norm(r.out - ref) / np.linalg.norm(ref)
    assert 0.02 < rel < 0.06


def test_calibration_values():
    draws = [make_qkv(100 + i, 16, 2, 8) for i in range(16)]
    vals = pipeline.calibrate(draws, 1.5)
    for j in range(3):
        m = max(quant.amax(d[j]) for d in draws)
        assert vals[j] == np.float32(np.float32(1.5) * m)


def test_output_quantization_is_the_input_formula_on_fp32_O():
    """pipeline.quantize_output: O rounded to fp32, then the per-tensor formula."""
    import oracle
    rng = np.random.default_rng(9)
    out = rng.standard_normal((37, 3, 8)) * 0.3
    s = np.float32(0.0021)
    codes = oracle.pipeline.quantize_output(out, s)
    assert codes.shape == out.shape and codes.dtype == np.uint8
    assert np.array_equal(codes, oracle.quant.quantize_f32(out.astype(np.float32), s))
    # round trip: decoding lands within half an e4m3 step (3 mantissa bits) of O
    dec = oracle.e4m3.decode(codes) * np.float64(s)
    big = np.abs(out) > 2.0 ** -6 * float(s)
    assert np.all(np.abs(dec - out)[big] <= np.abs(out)[big] * 2.0 ** -4 * 1.0001)
