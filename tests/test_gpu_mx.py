"""GPU parity of the block-scaled (MX) variant against the oracle
(oracle.mx, oracle.pipeline.forward_mx): codes and E8M0 scales of Q and K bit
for bit, V and the state as the per-tensor path, and the attention within
max-abs 1e-2 * max|V| of the quantization-emulating oracle and relative RMS
5e-2 of unquantized fp64 (block-scaled e4m3 is as accurate as per-tensor
e4m3 on these inputs)."""
import numpy as np
import pytest
import torch

import oracle
from synth import f32_to_bf16_bits, make_cu_seqlens, make_qkv
from tests.gpu_helpers import ATOL_FRAC_OF_VMAX, REL_RMS_VS_FP64, codes_np, fv, rel_rms, require_gpu, to_dev, vmax_of

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _edge_tensor(T, H, d, seed):
    """Blocks spanning many binades, zero blocks, subnormal-only blocks, and
    block maxima at and around the scale boundaries (448 * 2^k and a mantissa
    of 1.75 against the next bf16 value)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, H, d)) * np.exp2(rng.integers(-40, 40, (T, H, 1)))).astype(np.float32)
    x *= np.exp2(rng.normal(0, 4, (T, H, d))).astype(np.float32)
    x[0, 0, :] = 0.0
    if T > 1:
        x[1, 0, :] = np.float32(2.0 ** -130) * rng.integers(-3, 4, d)
    for r in range(2, min(T, 12)):
        k = int(rng.integers(-20, 20))
        m = [1.75, 1.7578125, 1.0, 1.9921875, 1.5][r % 5]
        blk = r % ((d + 31) // 32)
        x[r, 0, 32 * blk] = np.float32(m * 2.0 ** (k + 8)) * (1 if r % 2 else -1)
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("d", [72, 128])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_mx_quantize_bit_exact(d, mode):
    dev = require_gpu()
    T, H = 97, 3
    qb, kb = _edge_tensor(T, H, d, 1 + d), _edge_tensor(T, H, d, 2 + d)
    _, _, vb = make_qkv(3, T, H, d)
    st = fv.new_state(dev)
    if mode == "static":
        fv.state_set_static(st, [2.0, 3.0, 5.0])
    q8, k8, v8, qs, ks = fv.quantize_qkv_mx(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, mode)
    torch.cuda.synchronize()
    for got_c, got_s, bits in ((q8, qs, qb), (k8, ks, kb)):
        rc, rs = oracle.mx.quantize(bits)
        assert np.array_equal(codes_np(got_s), rs)
        assert np.array_equal(codes_np(got_c), rc)
    ring = oracle.scales.AmaxRing()
    ref = oracle.pipeline.forward_mx(qb, kb, vb, make_cu_seqlens([T]), mode, ring=ring,
                                     static_values=[2.0, 3.0, 5.0], attend=False)
    assert np.array_equal(codes_np(v8), ref.v_codes)
    assert np.float32(fv.state_read(st)["descale_used"][2]) == ref.v_descale


def test_mx_quantize_strided_views():
    dev = require_gpu()
    T, H, d = 40, 4, 72
    qb, kb, vb = make_qkv(9, T, H, d)
    fused = np.stack([qb, kb, vb], axis=1)          # [T, 3, H, d]
    f = to_dev(fused, dev)
    st = fv.new_state(dev)
    q8, k8, v8, qs, ks = fv.quantize_qkv_mx(f[:, 0], f[:, 1], f[:, 2], st, "dynamic")
    torch.cuda.synchronize()
    rc, rs = oracle.mx.quantize(qb)
    assert np.array_equal(codes_np(q8), rc) and np.array_equal(codes_np(qs), rs)
    rc, rs = oracle.mx.quantize(kb)
    assert np.array_equal(codes_np(k8), rc) and np.array_equal(codes_np(ks), rs)


# (segment lengths, heads, head_dim): narrow hd72, narrow hd128, wide hd128 (64 heads),
# wide hd72 (attn_w32_kernel: 64 heads)
MX_CASES = [((130, 1, 0, 257, 64), 3, 72), ((300, 129, 1), 2, 128), ((300, 129), 64, 128), ((700,), 16, 72),
            ((300, 129, 0, 513), 64, 72)]


@pytest.mark.parametrize("seglens,H,d", MX_CASES)
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_mx_attention_matches_oracle(seglens, H, d, mode):
    dev = require_gpu()
    cu = make_cu_seqlens(seglens)
    T = int(cu[-1])
    qb, kb, vb = make_qkv(sum(seglens) + H + d, T, H, d)
    st = fv.new_state(dev)
    sv = [4.5, 4.5, 4.5]
    if mode == "static":
        fv.state_set_static(st, sv)
    q8, k8, v8, qs, ks = fv.quantize_qkv_mx(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, mode)
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
    out = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
    fv.attn_varlen_mx(q8, k8, v8, qs, ks, cu_d, max(seglens), st, out=out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(o)), "unwritten output elements"
    ref = oracle.pipeline.forward_mx(qb, kb, vb, cu, mode, ring=oracle.scales.AmaxRing(), static_values=sv)
    assert np.array_equal(codes_np(q8), ref.q[0]) and np.array_equal(codes_np(ks), ref.k[1])
    err = np.abs(o - ref.out).max() / vmax_of(vb)
    assert err <= ATOL_FRAC_OF_VMAX, err
    if T >= 256:
        assert rel_rms(o, oracle.pipeline.reference_unquantized(qb, kb, vb, cu)) <= REL_RMS_VS_FP64
    # run-to-run determinism
    o2 = fv.attn_varlen_mx(q8, k8, v8, qs, ks, cu_d, max(seglens), st).float().cpu().numpy()
    assert np.array_equal(o2, o)


def test_mx_attention_block_scales_matter():
    """Scaling one block of K by 2^8 (exactly) moves its E8M0 byte by 8 and
    leaves its codes and the attention output unchanged up to the same 2^8 in
    that block's share of the scores: checked against the oracle, which a
    wrong per-lane scale mapping in the kernel would fail."""
    dev = require_gpu()
    T, H, d = 300, 2, 128
    qb, kb, vb = make_qkv(77, T, H, d)
    kf = oracle.quant.bf16_to_f32(kb).copy()
    kf[:, :, 64:96] *= np.float32(2.0 ** -8)
    kb2 = f32_to_bf16_bits(kf)
    st = fv.new_state(dev)
    q8, k8, v8, qs, ks = fv.quantize_qkv_mx(to_dev(qb, dev), to_dev(kb2, dev), to_dev(vb, dev), st, "dynamic")
    cu = make_cu_seqlens([T])
    o = fv.attn_varlen_mx(q8, k8, v8, qs, ks, torch.from_numpy(np.asarray(cu, np.int32)).to(dev), T, st)
    torch.cuda.synchronize()
    ref = oracle.pipeline.forward_mx(qb, kb2, vb, cu, "dynamic", ring=oracle.scales.AmaxRing())
    err = np.abs(o.float().cpu().numpy() - ref.out).max() / vmax_of(vb)
    assert err <= ATOL_FRAC_OF_VMAX, err


@pytest.mark.parametrize("H,d", [(2, 72), (2, 128), (64, 128), (64, 72)])
def test_mx_attention_random_block_scales(H, d):
    """Scale bytes drawn independently per (token, head, block) for Q and K
    (2^-8 .. 2^-4) over the quantizer's codes: the attention must match the
    oracle's attention of exactly these codes and scales, so every block scale
    must reach the bytes of its own block (the scaled MFMA takes block j's
    scale from lane group j, which is not the lane group holding d 32j..)."""
    dev = require_gpu()
    T = 300
    qb, kb, vb = make_qkv(500 + H + d, T, H, d)
    st = fv.new_state(dev)
    q8, k8, v8, _, _ = fv.quantize_qkv_mx(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, "dynamic")
    rng = np.random.default_rng(H * 1000 + d)
    nb = (d + 31) // 32
    scales = []
    for _ in range(2):
        s = np.zeros((T, H, 4), np.uint8)
        s[..., :nb] = rng.integers(119, 124, (T, H, nb))
        scales.append(s)
    cu = make_cu_seqlens([T])
    o = fv.attn_varlen_mx(q8, k8, v8, *(torch.from_numpy(s).to(dev) for s in scales),
                          torch.from_numpy(np.asarray(cu, np.int32)).to(dev), T, st)
    torch.cuda.synchronize()
    dv = np.float32(fv.state_read(st)["descale_used"][2])
    vdeq = oracle.quant.dequantize(codes_np(v8), dv)
    ref = oracle.attention.attention(oracle.mx.dequantize(codes_np(q8), scales[0]),
                                     oracle.mx.dequantize(codes_np(k8), scales[1]), vdeq, cu)
    err = np.abs(o.float().cpu().numpy() - ref).max() / np.abs(vdeq).max()
    assert err <= ATOL_FRAC_OF_VMAX, err


@pytest.mark.parametrize("name", ["l8192_hd72_static", "l8192_hd128_dyn"])
def test_mx_full_size_sampled(name):
    """The block-scaled path at full size in the launch configuration of
    `bench.py --scaling mx` (static values calibrated over the workload's 16
    calibration inputs, or the ring filled by its 16 warm-ups): codes and
    scales bit for bit, V's descale, and 2048 sampled rows plus the first and
    last row of every head against the MX oracle and unquantized fp64."""
    from synth import WORKLOADS
    dev = require_gpu()
    w = WORKLOADS[name]
    st = fv.new_state(dev)
    ring = oracle.scales.AmaxRing()
    static_values = None
    if w.mode == "static":
        cal = fv.new_state(dev)
        cal_ring = oracle.scales.AmaxRing()
        for s in w.warm_seeds:
            x = w.inputs(s)
            fv.quantize_qkv(*(to_dev(t, dev) for t in x), cal, "dynamic")
            cal_ring.push([oracle.quant.amax(t) for t in x])
        static_values = fv.calibrated_values(cal, 1.5)
        assert np.array_equal(np.float32(static_values), oracle.scales.calibrated_values(cal_ring, 1.5))
        fv.state_set_static(st, static_values)
    else:
        for s in w.warm_seeds:
            x = w.inputs(s)
            fv.quantize_qkv(*(to_dev(t, dev) for t in x), st, "dynamic")
            ring.push([oracle.quant.amax(t) for t in x])
    qb, kb, vb = w.inputs()
    q8, k8, v8, qs, ks = fv.quantize_qkv_mx(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, w.mode)
    T, H, d = qb.shape
    L = max(w.seglens)
    cu_d = torch.from_numpy(np.asarray(w.cu_seqlens, np.int32)).to(dev)
    out = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
    fv.attn_varlen_mx(q8, k8, v8, qs, ks, cu_d, L, st, out=out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(o)), "unwritten output elements"
    ref = oracle.pipeline.forward_mx(qb, kb, vb, w.cu_seqlens, w.mode, ring=ring, static_values=static_values,
                                     attend=False)
    assert np.array_equal(codes_np(q8), ref.q[0]) and np.array_equal(codes_np(qs), ref.q[1])
    assert np.array_equal(codes_np(k8), ref.k[0]) and np.array_equal(codes_np(ks), ref.k[1])
    assert np.array_equal(codes_np(v8), ref.v_codes)
    assert np.float32(fv.state_read(st)["descale_used"][2]) == ref.v_descale
    rng = np.random.default_rng(11)
    rows = list(zip(rng.integers(0, T, 2048).tolist(), rng.integers(0, H, 2048).tolist()))
    rows += [(0, h) for h in range(H)] + [(T - 1, h) for h in range(H)]
    deq = [oracle.mx.dequantize(*ref.q), oracle.mx.dequantize(*ref.k), oracle.quant.dequantize(ref.v_codes, ref.v_descale)]
    want = oracle.attention.attention_rows(deq[0], deq[1], deq[2], w.cu_seqlens, rows)
    got = np.stack([o[t, h] for t, h in rows])
    err = np.abs(got - want).max() / vmax_of(vb)
    assert err <= ATOL_FRAC_OF_VMAX, err
    fp = [oracle.quant.bf16_to_f32(x) for x in (qb, kb, vb)]
    unq = oracle.attention.attention_rows(fp[0], fp[1], fp[2], w.cu_seqlens, rows)
    assert rel_rms(got, unq) <= REL_RMS_VS_FP64
