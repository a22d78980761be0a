"""GPU parity at the largest sizes the library accepts.

The entry points reject calls past two 31-bit limits (include/fp8vit.h): the
quantizer's chunk indices (T*H*d/8 < 2^31) and the attention kernels' buffer
offsets ((T + 384)*H*d < 2^31 bytes per e4m3 tensor). These tests run just
under each limit, so the highest offsets of every index computation are used,
and check sampled slices bit-exactly (codes) or to the usual attention bar
against the CPU oracle. Static scales keep the oracle's inputs to the slices
it checks. Inputs come from torch's seeded generator on the device
(`synth.device_randn_bf16`); the oracle reads back the same bf16 bits.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import device_randn_bf16, make_cu_seqlens
from tests.gpu_helpers import ATOL_FRAC_OF_VMAX, codes_np, fv, require_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_quantize_at_the_chunk_index_limit():
    dev = require_gpu()
    H, d = 16, 72
    T = 14_913_000                       # T * H * d / 8 = 2^31 - 11648 chunks
    assert T * H * d // 8 < 2 ** 31 and (T + 1000) * H * d // 8 >= 2 ** 31
    x = device_randn_bf16((T, H, d), 81, dev)
    values = [4.0, 5.0, 6.0]
    st = fv.new_state(dev)
    fv.state_set_static(st, values)
    codes = fv.quantize_qkv(x, x, x, st, "static")   # Q, K and V share one input
    torch.cuda.synchronize()
    descales = [oracle.scales.descale_from_amax(v) for v in values]
    assert fv.state_read(st)["descale_used"] == [float(dd) for dd in descales]
    rng = np.random.Generator(np.random.PCG64(82))
    windows = [(0, 4096), (T // 2, T // 2 + 4096), (T - 4096, T)]
    windows += [(int(t), int(t) + 64) for t in rng.integers(0, T - 64, size=6)]
    for t0, t1 in windows:
        bits = _bits(x[t0:t1])
        for c, dd in zip(codes, descales):
            assert np.array_equal(codes_np(c[t0:t1]), oracle.quant.quantize(bits, dd)), (t0, t1)
    del x, codes


def test_attention_at_the_buffer_offset_limit():
    dev = require_gpu()
    H, d, L = 16, 72, 1000
    nseg = 1863
    T = nseg * L                         # (T + 384) * H * d = 2^31 - 865,280
    assert (T + 384) * H * d < 2 ** 31 and (T + 384 + 800) * H * d >= 2 ** 31
    q, k, v = (device_randn_bf16((T, H, d), s, dev) for s in (91, 92, 93))
    values = [5.0, 5.0, 5.0]
    st = fv.new_state(dev)
    fv.state_set_static(st, values)
    q8, k8, v8 = fv.quantize_qkv(q, k, v, st, "static")
    cu = make_cu_seqlens([L] * nseg)
    out = fv.attn_varlen(q8, k8, v8, torch.from_numpy(cu).to(dev), L, st)
    torch.cuda.synchronize()
    ds = [oracle.scales.descale_from_amax(x) for x in values]
    for seg in (0, nseg // 2, nseg - 1):
        t0, t1 = seg * L, (seg + 1) * L
        qb, kb, vb = _bits(q[t0:t1]), _bits(k[t0:t1]), _bits(v[t0:t1])
        cq, ck, cv = (oracle.quant.quantize(b, dd) for b, dd in zip((qb, kb, vb), ds))
        for c_gpu, c_ref in zip((q8, k8, v8), (cq, ck, cv)):
            assert np.array_equal(codes_np(c_gpu[t0:t1]), c_ref), seg
        ref = oracle.attention.attention(oracle.quant.dequantize(cq, ds[0]), oracle.quant.dequantize(ck, ds[1]),
                                         oracle.quant.dequantize(cv, ds[2]), [0, L])
        o = out[t0:t1].float().cpu().numpy().astype(np.float64)
        vmax = np.abs(oracle.quant.bf16_to_f32(vb)).max()
        err = np.abs(o - ref).max() / vmax
        assert err <= ATOL_FRAC_OF_VMAX, (seg, err)
