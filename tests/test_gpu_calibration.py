"""Calibration export and state resume in the library, through the C ABI.

vLLM page "FP8 ViT Encoder Attention", Calibrate-Once Reuse Workflow: dynamic
scaling runs over the calibration passes, then the learned values times a
margin (default 1.5) go to the JSON scale file that static scaling reads. Here
fp8vit_calibrated_values must give the oracle's values bit for bit, the file
written by fp8vit_save_static_scales must read back to the same floats, and a
static forward with them must quantize as the oracle does. fp8vit_state_write
must resume a dynamic ring so that later forwards are the ones the original
state would have produced."""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import make_qkv
from tests.gpu_helpers import codes_np, f32bits, fv, require_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

T, H, D = 300, 4, 72
LAYER = "visual.blocks.0.attn.attn"


def _draw(i):
    # outliers on some draws, so the window maximum moves as the ring fills
    return make_qkv(500 + i, T, H, D, outlier_frac=1e-3 if i % 5 == 2 else 0.0, outlier_scale=4.0 + i)


def _dyn(st, bits, dev):
    q, k, v = (to_dev(x, dev) for x in bits)
    return [codes_np(c) for c in fv.quantize_qkv(q, k, v, st, "dynamic")]


def test_calibrate_save_load_static_forward(tmp_path):
    dev = require_gpu()
    draws = [_draw(i) for i in range(16)]
    st = fv.new_state(dev)
    with pytest.raises(fv.Fp8VitError):
        fv.calibrated_values(st, 1.5)                        # empty ring: nothing to calibrate
    for bits in draws:
        _dyn(st, bits, dev)
    want = oracle.pipeline.calibrate(draws, 1.5)
    got = np.float32(fv.calibrated_values(st, 1.5))
    print("calibrated", got, "oracle", want, flush=True)
    assert np.array_equal(f32bits(got), f32bits(want))
    # another margin: still one fp32 product of the window max
    ring = oracle.scales.AmaxRing()
    for bits in draws:
        ring.push([oracle.quant.amax(x) for x in bits])
    assert np.array_equal(f32bits(fv.calibrated_values(st, 1.1)), f32bits(oracle.scales.calibrated_values(ring, 1.1)))

    path = str(tmp_path / "scales.json")
    with open(path, "w") as f:
        f.write('{"visual.blocks.1.attn.attn": {"q": 3, "k": 4, "v": 5}}')
    fv.save_static_scales(path, LAYER, got)
    loaded = np.float32(fv.load_static_scales(path, LAYER))
    assert np.array_equal(f32bits(loaded), f32bits(got))
    assert fv.load_static_scales(path, "visual.blocks.1.attn.attn") == (3.0, 4.0, 5.0)

    sst = fv.new_state(dev)
    fv.state_set_static(sst, loaded)
    probe = make_qkv(999, T, H, D, outlier_frac=1e-3, outlier_scale=30.0)   # saturates somewhere
    q, k, v = (to_dev(x, dev) for x in probe)
    codes = [codes_np(c) for c in fv.quantize_qkv(q, k, v, sst, "static")]
    ref_codes, ref_ds, _ = oracle.pipeline.quantize_step(*probe, "static", static_values=loaded)
    for name, c, r in zip("qkv", codes, ref_codes):
        assert np.array_equal(c, r), name
    assert np.array_equal(f32bits(fv.state_read(sst)["descale_used"]), f32bits(ref_ds))


def test_state_write_resumes_the_ring():
    dev = require_gpu()
    draws = [_draw(i) for i in range(26)]
    a = fv.new_state(dev)
    ring = oracle.scales.AmaxRing()
    for bits in draws[:9]:
        _dyn(a, bits, dev)
        ring.push([oracle.quant.amax(x) for x in bits])
    snap = fv.state_read(a)
    b = fv.new_state(dev)
    fv.state_write(b, snap)
    assert fv.state_read(b) == snap
    # both continue past the ring's wrap-around; every forward must agree
    for i, bits in enumerate(draws[9:]):
        ca = _dyn(a, bits, dev)
        cb = _dyn(b, bits, dev)
        ref_codes, ref_ds, _ = oracle.pipeline.quantize_step(*bits, "dynamic", ring=ring)
        for name, x, y, r in zip("qkv", ca, cb, ref_codes):
            assert np.array_equal(x, y), (i, name)
            assert np.array_equal(x, r), (i, name)
        sa, sb = fv.state_read(a), fv.state_read(b)
        assert sa == sb, i
        assert np.array_equal(f32bits(sa["descale_used"]), f32bits(ref_ds)), i
    assert fv.state_read(b)["count"] == len(draws)
    assert np.array_equal(f32bits(fv.state_read(b)["ring"]), f32bits(ring.ring))


def test_state_write_then_static_and_reset():
    dev = require_gpu()
    st = fv.new_state(dev)
    snap = {"ring": [[float(x + 16 * i) for i in range(16)] for x in range(3)], "count": 37,
            "static_values": [1.0, 2.0, 3.0], "descale_used": [0.5, 0.25, 0.125], "amax_last": [7.0, 8.0, 9.0],
            "flags": 0, "cu_check": 0, "saturated": [0, 0, 0]}
    fv.state_write(st, snap)
    assert fv.state_read(st) == snap
    # a dynamic forward after the write pushes into slot 37 % 16 = 5
    bits = _draw(3)
    _dyn(st, bits, dev)
    r = fv.state_read(st)
    amax = [float(oracle.quant.amax(x)) for x in bits]
    assert r["count"] == 38 and [r["ring"][x][5] for x in range(3)] == amax
    with pytest.raises(fv.Fp8VitError):
        fv.state_write(st, dict(snap, ring=[[-1.0] * 16] * 3))
    assert fv.state_read(st) == r                           # a rejected write changes nothing
    fv.state_init(st)
    torch.cuda.synchronize()
    assert fv.state_read(st)["count"] == 0
