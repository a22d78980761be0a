"""Full-size parity in the bench's own launch configuration and scaling
sequence (the workspace attention entry point; calibration or dynamic
warm-ups exactly as bench.py runs them before its timed steps):

* L=8192, 16 heads, hd72, static 1.5 x calibrated: every row of the output
  against the oracle (element by element) and against unquantized fp64;
* L=256, 16 heads, hd72, dynamic on an empty ring (first forward): every row;
* L=2304, 16 heads, hd72, dynamic after its 16 warm-ups: every row (the
  workspace entry point, whose plan does not split this shape);
* L=8192, 16 heads, hd128, dynamic after its 16 warm-ups: 2048 sampled rows
  plus the first and last row of every head.

The ring the GPU holds after the warm-ups, the descales and the codes are
compared bit for bit with the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from tests.gpu_helpers import ATOL_FRAC_OF_VMAX, REL_RMS_VS_FP64, codes_np, fv, rel_rms, require_gpu, to_dev, vmax_of

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _amax3(x):
    return [oracle.quant.amax(t) for t in x]


def _bench_forward(name, dev):
    """Scaling sequence and launch of bench.py for workload `name`; returns the
    GPU output (fp64 numpy), the codes, the GPU state and the oracle's codes and
    descales for the measured input."""
    w = WORKLOADS[name]
    st = fv.new_state(dev)
    ring = oracle.scales.AmaxRing()
    static_values = None
    if w.mode == "static":
        cal = fv.new_state(dev)
        for s in w.warm_seeds:
            x = w.inputs(s)
            fv.quantize_qkv(*(to_dev(t, dev) for t in x), cal, "dynamic")
            ring.push(_amax3(x))
        static_values = fv.calibrated_values(cal, 1.5)
        assert np.array_equal(np.float32(static_values), oracle.scales.calibrated_values(ring, 1.5))
        fv.state_set_static(st, static_values)
    else:
        for s in w.warm_seeds:
            x = w.inputs(s)
            fv.quantize_qkv(*(to_dev(t, dev) for t in x), st, "dynamic")
            ring.push(_amax3(x))
    qb, kb, vb = w.inputs()
    codes = fv.quantize_qkv(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, w.mode)
    ref_codes, ref_ds, _ = oracle.pipeline.quantize_step(qb, kb, vb, w.mode, ring=ring, static_values=static_values)
    T, H, d = qb.shape
    L = max(w.seglens)
    cu_d = torch.from_numpy(np.asarray(w.cu_seqlens, np.int32)).to(dev)
    ws = fv.attn_workspace(len(w.seglens), L, T, H, d, device=dev)
    out = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
    fv.attn_varlen_ws(*codes, cu_d, L, st, ws, out=out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(o)), "unwritten output elements"
    for c, r in zip(codes, ref_codes):
        assert np.array_equal(codes_np(c), r)
    sv = fv.state_read(st)
    assert np.array_equal(np.float32(sv["descale_used"]), ref_ds)
    if w.mode == "dynamic":
        assert np.array_equal(np.float32(sv["ring"]), ring.ring) and sv["count"] == ring.count
    return w, (qb, kb, vb), o, ref_codes, ref_ds


def _all_rows(name):
    dev = require_gpu()
    w, (qb, kb, vb), o, ref_codes, ref_ds = _bench_forward(name, dev)
    deq = [oracle.quant.dequantize(c, d) for c, d in zip(ref_codes, ref_ds)]
    ref = oracle.attention.attention(deq[0], deq[1], deq[2], w.cu_seqlens)
    err = np.abs(o - ref).max() / vmax_of(vb)
    assert err <= ATOL_FRAC_OF_VMAX, err
    unq = oracle.pipeline.reference_unquantized(qb, kb, vb, w.cu_seqlens)
    r_gpu, r_orc = rel_rms(o, unq), rel_rms(ref, unq)
    assert r_gpu <= REL_RMS_VS_FP64, (r_gpu, r_orc)
    assert abs(r_gpu - r_orc) <= 0.02 * r_orc, (r_gpu, r_orc)


@pytest.mark.parametrize("name", ["small_l256_hd72_dyn", "l2304_hd72_dyn", "l8192_hd72_static"])
def test_full_size_every_row(name):
    _all_rows(name)


def test_full_size_hd128_after_warmups_sampled():
    dev = require_gpu()
    w, (qb, kb, vb), o, ref_codes, ref_ds = _bench_forward("l8192_hd128_dyn", dev)
    T, H, d = qb.shape
    rng = np.random.default_rng(5)
    rows = list(zip(rng.integers(0, T, 2048).tolist(), rng.integers(0, H, 2048).tolist()))
    rows += [(0, h) for h in range(H)] + [(T - 1, h) for h in range(H)]
    deq = [oracle.quant.dequantize(c, ds) for c, ds in zip(ref_codes, ref_ds)]
    ref = oracle.attention.attention_rows(deq[0], deq[1], deq[2], w.cu_seqlens, rows)
    got = np.stack([o[t, h] for t, h in rows])
    err = np.abs(got - ref).max() / vmax_of(vb)
    assert err <= ATOL_FRAC_OF_VMAX, err
    fp = [oracle.quant.bf16_to_f32(x) for x in (qb, kb, vb)]
    unq = oracle.attention.attention_rows(fp[0], fp[1], fp[2], w.cu_seqlens, rows)
    assert rel_rms(got, unq) <= REL_RMS_VS_FP64
