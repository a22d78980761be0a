"""The whole hot path on the CPU, step by step, in the order the pages give.

Oracle code: used only by tests, smoke() and the bench's CPU baseline.

forward(): bf16 Q/K/V -> (dynamic: amax of each tensor, pushed into the ring;
static: the file values) -> descale per tensor -> e4m3 codes -> attention over
the dequantized values, per segment, in fp64 ("Q/K/V are quantized to FP8 right
before the attention call", vLLM page "FP8 ViT Encoder Attention", intro).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import quant, scales, attention, mx


@dataclass
class ForwardResult:
    codes: tuple            # (q8, k8, v8) uint8 [T, H, d]
    descales: np.ndarray    # fp32 [3]
    amax: Optional[np.ndarray]  # fp32 [3] (dynamic only)
    out: Optional[np.ndarray]   # fp64 [T, H, d] (None when attend=False)


def quantize_step(q, k, v, mode: str, ring: Optional[scales.AmaxRing] = None, static_values=None):
    """Scale bookkeeping + quantization for one forward."""
    if mode == "dynamic":
        a = np.array([quant.amax(q), quant.amax(k), quant.amax(v)], dtype=np.float32)
        ds = scales.dynamic_descales(ring, a)
    elif mode == "static":
        a = None
        ds = scales.static_descales(static_values)
    else:
        raise ValueError(mode)
    codes = tuple(quant.quantize(x, d) for x, d in zip((q, k, v), ds))
    return codes, ds, a


def forward(q, k, v, cu_seqlens, mode: str, ring: Optional[scales.AmaxRing] = None,
            static_values=None, softmax_scale=None, attend: bool = True) -> ForwardResult:
    codes, ds, a = quantize_step(q, k, v, mode, ring, static_values)
    out = None
    if attend:
        deq = [quant.dequantize(c, d) for c, d in zip(codes, ds)]
        out = attention.attention(deq[0], deq[1], deq[2], cu_seqlens, softmax_scale)
    return ForwardResult(codes, ds, a, out)


def quantize_output(out: np.ndarray, out_descale) -> np.ndarray:
    """FP8 output of the attention (the fused fp8-output feature request on the
    vLLM issue page "Add support for fused fp8 output to FlashAttention 3"):
    the per-tensor input formula applied to O. Reading: O is first rounded to
    fp32, the precision the kernel forms it in, then divided by the static
    output descale (IEEE fp32), clamped to +-448 and rounded to e4m3."""
    return quant.quantize_f32(np.asarray(out, dtype=np.float64).astype(np.float32), out_descale)


def reference_unquantized(q, k, v, cu_seqlens, softmax_scale=None) -> np.ndarray:
    """Attention on the bf16 values themselves (no quantization), fp64."""
    return attention.attention(quant.bf16_to_f32(q), quant.bf16_to_f32(k), quant.bf16_to_f32(v),
                               cu_seqlens, softmax_scale)


def calibrate(draws, margin: float = 1.5) -> np.ndarray:
    """16 dynamic passes over the draws, then fp32(margin x window max) per tensor."""
    ring = scales.AmaxRing()
    for (q, k, v) in draws:
        ring.push([quant.amax(q), quant.amax(k), quant.amax(v)])
    return scales.calibrated_values(ring, margin)


@dataclass
class MxForwardResult:
    q: tuple                # (e4m3 codes uint8 [T, H, d], E8M0 scales uint8 [T, H, 4])
    k: tuple
    v_codes: np.ndarray     # per-tensor e4m3 codes of V
    v_descale: np.float32
    out: Optional[np.ndarray]


def forward_mx(q, k, v, cu_seqlens, mode: str, ring: Optional[scales.AmaxRing] = None, static_values=None,
               softmax_scale=None, attend: bool = True) -> MxForwardResult:
    """Block-scaled variant: Q and K quantized with one power-of-two scale per
    32-element block of head_dim (oracle.mx, readings R25-R27), V with its
    per-tensor scale as in forward() (R28: dynamic ring or static value), then
    the same fp64 attention over the dequantized values."""
    qc, qs = mx.quantize(q)
    kc, ks = mx.quantize(k)
    if mode == "dynamic":
        a = np.array([quant.amax(q), quant.amax(k), quant.amax(v)], dtype=np.float32)
        dv = scales.dynamic_descales(ring, a)[2]
    elif mode == "static":
        dv = scales.static_descales(static_values)[2]
    else:
        raise ValueError(mode)
    vc = quant.quantize(v, dv)
    out = None
    if attend:
        out = attention.attention(mx.dequantize(qc, qs), mx.dequantize(kc, ks), quant.dequantize(vc, dv),
                                  cu_seqlens, softmax_scale)
    return MxForwardResult((qc, qs), (kc, ks), vc, np.float32(dv), out)
