"""GPU parity of the fused quantizer and the scale bookkeeping against the oracle.
Bar: e4m3 bytes and fp32 descales bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, f32_to_bf16_bits, make_qkv
from tests.gpu_helpers import codes_np, f32bits, fv, require_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = ALL[np.isfinite(oracle.quant.bf16_to_f32(ALL))]

# static file values: the printed example, the floor region, awkward mantissas, huge
STATIC_VALUES = [224.0, 198.0, 210.0, 1e-12, 4.0e-8, 1.0, 3.7e-3, 0.07, 5.5, 448.0, 1.2e5, 3.3333333, 1e30]


def _all_bf16_tensor(shift: int):
    x = np.roll(FINITE, shift)
    n = (len(x) + 7) // 8 * 8
    x = np.concatenate([x, np.zeros(n - len(x), np.uint16)])
    return x.reshape(-1, 1, 8)


def test_quantize_static_exhaustive_bf16():
    dev = require_gpu()
    xs = [_all_bf16_tensor(s) for s in (0, 1000, 20000)]
    td = [to_dev(x, dev) for x in xs]
    st = fv.new_state(dev)
    for i in range(0, len(STATIC_VALUES), 3):
        vals = (STATIC_VALUES + STATIC_VALUES[:2])[i:i + 3]
        fv.state_set_static(st, vals)
        q8, k8, v8 = fv.quantize_qkv(td[0], td[1], td[2], st, "static")
        torch.cuda.synchronize()
        ds = oracle.scales.static_descales(vals)
        s = fv.state_read(st)
        assert np.array_equal(f32bits(s["descale_used"]), f32bits(ds)), (vals, s["descale_used"], ds)
        for x, c, d in zip(xs, (q8, k8, v8), ds):
            ref = oracle.quant.quantize(x, d)
            got = codes_np(c)
            bad = np.nonzero(got.ravel() != ref.ravel())[0]
            assert bad.size == 0, f"descale {d!r}: {bad.size} mismatches, first input bits " \
                                  f"{hex(int(x.ravel()[bad[0]]))} got {hex(got.ravel()[bad[0]])} want {hex(ref.ravel()[bad[0]])}"
        assert s["count"] == 0 and s["ring"] == [[0.0] * 16] * 3


def _random_static_values(n=60, seed=7):
    """Seeded fp32 file values with random 24-bit mantissas over 18 decades,
    plus neighbours of powers of two and of 448 * 2^k."""
    rng = np.random.Generator(np.random.PCG64(seed))
    vals = list((10.0 ** rng.uniform(-9, 9, n)).astype(np.float32))
    for k in (-20, -3, 0, 5, 17):
        p = np.float32(2.0 ** k)
        vals += [np.nextafter(p, np.float32(0)), p, np.nextafter(p, np.float32(np.inf)), np.float32(448.0) * p]
    return [float(v) for v in vals]


def test_quantize_static_exhaustive_bf16_random_descales():
    """Every finite bf16 pattern against many unrelated descales: the kernel's
    quotient RN32(x * RN64(1/descale)) must equal the IEEE fp32 division."""
    dev = require_gpu()
    xs = [_all_bf16_tensor(s) for s in (0, 7, 333)]
    td = [to_dev(x, dev) for x in xs]
    st = fv.new_state(dev)
    vals_all = _random_static_values()
    for i in range(0, len(vals_all) - 2, 3):
        vals = vals_all[i:i + 3]
        fv.state_set_static(st, vals)
        codes = fv.quantize_qkv(td[0], td[1], td[2], st, "static")
        torch.cuda.synchronize()
        ds = oracle.scales.static_descales(vals)
        for x, c, d in zip(xs, codes, ds):
            ref = oracle.quant.quantize(x, d)
            got = codes_np(c)
            bad = np.nonzero(got.ravel() != ref.ravel())[0]
            assert bad.size == 0, f"descale {d!r}: {bad.size} mismatches, first input bits " \
                                  f"{hex(int(x.ravel()[bad[0]]))} got {hex(got.ravel()[bad[0]])} want {hex(ref.ravel()[bad[0]])}"


def test_quantize_dynamic_sequence_matches_ring():
    dev = require_gpu()
    st = fv.new_state(dev)
    ring = oracle.scales.AmaxRing()
    for step in range(21):
        T = [37, 256, 1, 100][step % 4]
        scale = [1.0, 30.0, 0.001, 5.0, 1e-9][step % 5]
        qb, kb, vb = make_qkv(500 + step, T, 3, 8, outlier_frac=0.02)
        bits = [f32_to_bf16_bits(oracle.quant.bf16_to_f32(x) * np.float32(scale)) for x in (qb, kb, vb)]
        q8, k8, v8 = fv.quantize_qkv(*(to_dev(b, dev) for b in bits), st, "dynamic")
        torch.cuda.synchronize()
        codes, ds, a = oracle.pipeline.quantize_step(*bits, "dynamic", ring=ring)
        s = fv.state_read(st)
        assert np.array_equal(f32bits(s["amax_last"]), f32bits(a)), step
        assert np.array_equal(f32bits(s["descale_used"]), f32bits(ds)), step
        assert np.array_equal(f32bits(s["ring"]), f32bits(ring.ring)), step
        assert s["count"] == ring.count and s["flags"] == 0
        for c, r in zip((q8, k8, v8), codes):
            assert np.array_equal(codes_np(c), r), step


def test_quantize_strided_views_of_fused_qkv():
    dev = require_gpu()
    T, H, d = 300, 4, 72
    qb, kb, vb = make_qkv(77, T, H, d)
    fused = np.stack([qb, kb, vb], axis=1)            # [T, 3, H, d]
    tf = to_dev(fused, dev)
    views = [tf[:, i] for i in range(3)]
    assert views[0].stride(0) == 3 * H * d
    for mode in ("dynamic", "static"):
        st = fv.new_state(dev)
        if mode == "static":
            fv.state_set_static(st, [5.0, 6.0, 7.0])
        q8, k8, v8 = fv.quantize_qkv(*views, st, mode)
        torch.cuda.synchronize()
        ring = oracle.scales.AmaxRing()
        codes, ds, _ = oracle.pipeline.quantize_step(qb, kb, vb, mode, ring=ring, static_values=[5.0, 6.0, 7.0])
        for c, r in zip((q8, k8, v8), codes):
            assert np.array_equal(codes_np(c), r), mode


def test_quantize_empty_and_zero_tensors():
    dev = require_gpu()
    st = fv.new_state(dev)
    e = torch.empty((0, 2, 8), dtype=torch.bfloat16, device=dev)
    fv.quantize_qkv(e, e, e, st, "dynamic")
    z = torch.zeros((16, 2, 8), dtype=torch.bfloat16, device=dev)
    q8, _, _ = fv.quantize_qkv(z, z, z, st, "dynamic")
    torch.cuda.synchronize()
    s = fv.state_read(st)
    assert s["count"] == 2 and s["amax_last"] == [0.0, 0.0, 0.0]
    assert np.float32(s["descale_used"][0]) == np.float32(1e-10)
    assert np.all(codes_np(q8) == 0)


def test_scales_update_closed_forms():
    dev = require_gpu()
    st = fv.new_state(dev)
    ring = oracle.scales.AmaxRing()
    seqs = [float(t + 1) for t in range(20)] + [float(100 - t) for t in range(20)] + \
           [1000.0 if t == 3 else 0.5 for t in range(20)] + [0.0] * 3
    for t, a in enumerate(seqs):
        trip = np.float32([a, 2 * a, a / 3])
        fv.scales_update(st, torch.from_numpy(trip).to(dev))
        torch.cuda.synchronize()
        ds = oracle.scales.dynamic_descales(ring, trip)
        s = fv.state_read(st)
        assert np.array_equal(f32bits(s["descale_used"]), f32bits(ds)), t
        assert np.array_equal(f32bits(s["ring"]), f32bits(ring.ring)), t
    # a fused dynamic quantize after standalone updates continues the same ring
    qb, kb, vb = make_qkv(9, 64, 2, 8)
    fv.quantize_qkv(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, "dynamic")
    torch.cuda.synchronize()
    _, ds, _ = oracle.pipeline.quantize_step(qb, kb, vb, "dynamic", ring=ring)
    assert np.array_equal(f32bits(fv.state_read(st)["descale_used"]), f32bits(ds))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_quantize_full_size_workloads(name):
    """Every workload at its full size, in the scaling mode the bench uses."""
    dev = require_gpu()
    w = WORKLOADS[name]
    qb, kb, vb = w.inputs()
    st = fv.new_state(dev)
    static_vals = [3.0, 4.0, 5.0] if w.mode == "static" else None
    if static_vals:
        fv.state_set_static(st, static_vals)
    tq, tk, tv = (to_dev(x, dev) for x in (qb, kb, vb))
    q8, k8, v8 = fv.quantize_qkv(tq, tk, tv, st, w.mode)
    torch.cuda.synchronize()
    codes, ds, _ = oracle.pipeline.quantize_step(qb, kb, vb, w.mode, ring=oracle.scales.AmaxRing(),
                                                 static_values=static_vals)
    assert np.array_equal(f32bits(fv.state_read(st)["descale_used"]), f32bits(ds))
    for c, r in zip((q8, k8, v8), codes):
        assert np.array_equal(codes_np(c), r)


def test_quantize_writes_only_its_outputs():
    """Each code tensor is a view inside a larger buffer filled with a canary:
    the views hold the same codes as a contiguous run and nothing else changes."""
    dev = require_gpu()
    T, H, d = 777, 3, 72
    qb, kb, vb = make_qkv(61, T, H, d)
    q, k, v = (to_dev(x, dev) for x in (qb, kb, vb))
    n = T * H * d
    outs, bigs = [], []
    for x in range(3):
        big = torch.full((n + 4096,), 0xA5, dtype=torch.uint8, device=dev)
        bigs.append(big)
        outs.append(big[2048:2048 + n].view(T, H, d))
    for mode in ("dynamic", "static"):
        st = fv.new_state(dev)
        if mode == "static":
            fv.state_set_static(st, [3.0, 4.0, 5.0])
        fv.quantize_qkv(q, k, v, st, mode, out=tuple(outs))
        st2 = fv.new_state(dev)
        if mode == "static":
            fv.state_set_static(st2, [3.0, 4.0, 5.0])
        ref = fv.quantize_qkv(q, k, v, st2, mode)
        torch.cuda.synchronize()
        for x in range(3):
            assert torch.equal(outs[x], ref[x])
            assert torch.all(bigs[x][:2048] == 0xA5) and torch.all(bigs[x][2048 + n:] == 0xA5)
