"""Per-tensor amax and e4m3 quantization of bf16 tensors.

Oracle code: used only by tests, smoke() and the bench's CPU baseline.

Sources: atrex-bench #025 per_token_group_quant_fp8, Reference Implementation
(the only printed FP8 quantization formula): divide the fp32 input by the scale,
clamp to +-fp8_max, cast to e4m3fn. The ViT path applies it with one group per
tensor (per-tensor scaling, the "pertensor" AITER entry point named in the
Requirements section of the vLLM "FP8 ViT Encoder Attention" page).

Readings:
  R6  rounding is nearest-even from the fp32 quotient; the clamp comes before
      the cast, so out-of-range quotients saturate to +-448.
  R7  the quotient is an IEEE fp32 division (numpy float32 division is
      correctly rounded), not a multiplication by a reciprocal.
  R8  inputs are finite (non-finite inputs are outside the contract).
  R9  the amax runs over the whole packed tensor: all segments, all heads.
"""
from __future__ import annotations

import numpy as np

from . import e4m3


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact: a 16-bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def amax(bits: np.ndarray) -> np.float32:
    """max |x| over every element of the tensor (0 for an empty tensor)."""
    x = bf16_to_f32(bits)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def quantize_f32(x: np.ndarray, descale) -> np.ndarray:
    """e4m3 codes of the fp32 values x / descale (IEEE fp32 division), clamped to
    +-448 then rounded to nearest even."""
    x = np.asarray(x, dtype=np.float32)
    d = np.float32(descale)
    with np.errstate(over="ignore"):
        y = (x / d).astype(np.float32)
    y = np.clip(y, -e4m3.E4M3_MAX, e4m3.E4M3_MAX).astype(np.float32)
    return e4m3.encode_rne(y)


def quantize(bits: np.ndarray, descale) -> np.ndarray:
    """e4m3 codes of x / descale for bf16 bit patterns x."""
    return quantize_f32(bf16_to_f32(bits), descale)


def dequantize(codes: np.ndarray, descale) -> np.ndarray:
    """Exact fp64 value of each code times the descale (3-bit x 24-bit fits in 53)."""
    return e4m3.decode(codes) * np.float64(np.float32(descale))


def saturated_count(bits: np.ndarray, descale) -> int:
    """Number of elements the clamp of the quantizer changes: those whose fp32
    quotient x / descale (IEEE division) is larger than 448 in magnitude.

    A diagnostic of static scales (vLLM page "FP8 ViT Encoder Attention",
    Calibrate-Once Reuse Workflow: the saved values carry a margin that leaves
    headroom for activations beyond the calibration maximum; an element past
    that headroom is clamped to +-448 and counted here). A quotient of exactly
    448 is not clamped."""
    x = bf16_to_f32(bits)
    d = np.float32(descale)
    with np.errstate(over="ignore"):
        y = (x / d).astype(np.float32)
    return int(np.count_nonzero(np.abs(y) > e4m3.E4M3_MAX))
