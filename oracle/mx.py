"""Block-scaled ("MX") e4m3 quantization of Q and K -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU baseline use this.

Sources (cited by title and section):
  * FlashInfer PR 5283 analysis ("experimental NVFP4 attention"), Code
    analysis §1: the head dimension is cut into blocks (SF_VEC elements), each
    block gets its own scale from the block's absolute maximum divided by the
    element format's largest value, and the elements are stored in a narrow
    float format.
  * FlashInfer PR 3684 analysis ("asymmetric VO-split NVFP4"), §3: one scale
    factor per block of elements; a split of the computation must respect the
    block boundaries.

The gfx950 matrix cores apply block scales natively to 32-element blocks of
the contraction dimension, with power-of-two (E8M0) scales. Readings taken:
  R25 block = 32 consecutive elements along head_dim within one (token, head)
      row; a trailing partial block (head_dim 72: elements 64..71) is a block
      of its own.
  R26 the block scale is the smallest power of two >= block amax / 448 (the
      page's amax / format-max, rounded up to a power of two so that no
      element saturates), stored as an E8M0 byte (exponent + 127), within
      2^-127 .. 2^127; an all-zero block gets 2^-127 (byte 0).
  R27 elements: e4m3 round-to-nearest-even of clamp(x / scale, -448, 448), the
      per-tensor path's clamp-then-cast; x / scale is exact (a power of two).
  R28 V keeps its per-tensor scale: in P.V the contraction runs over keys,
      while V's blocks would run along head_dim.

Scales are returned as uint8 [T, H, 4]: block b's E8M0 byte at [..., b], the
unused bytes (head_dim 72 has three blocks) zero.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .quant import bf16_to_f32

BLOCK = 32
E8M0_BIAS = 127
SCALE_BYTES = 4


def n_blocks(head_dim: int) -> int:
    return (head_dim + BLOCK - 1) // BLOCK


def block_amax(x: np.ndarray) -> np.ndarray:
    """max |x| per block of the last axis: [..., n_blocks] float64."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    d = x.shape[-1]
    return np.stack([x[..., b * BLOCK:min(d, (b + 1) * BLOCK)].max(axis=-1) for b in range(n_blocks(d))], axis=-1)


def scale_exponent(amax) -> np.ndarray:
    """R26: the smallest integer s with 448 * 2^s >= amax, clamped to [-127, 127];
    -127 for amax == 0. Computed exactly from frexp (amax = f * 2^e, f in [0.5, 1))."""
    a = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(np.where(a > 0, a, 1.0))
    # amax / 448 = (f / 0.875) * 2^(e - 9); f / 0.875 <= 1 exactly when f <= 0.875
    s = np.where(f <= 0.875, e - 9, e - 8).astype(np.int64)
    s = np.where(a > 0, s, -127)
    return np.clip(s, -127, 127)


def quantize(bits: np.ndarray):
    """bf16 bit patterns [T, H, d] -> (e4m3 codes uint8 [T, H, d], E8M0 scales uint8 [T, H, 4])."""
    x = bf16_to_f32(bits).astype(np.float64)
    T, H, d = x.shape
    nb = n_blocks(d)
    assert nb <= SCALE_BYTES
    s = scale_exponent(block_amax(x)) if x.size else np.zeros((T, H, nb), np.int64)
    codes = np.empty((T, H, d), dtype=np.uint8)
    for b in range(nb):
        b0, b1 = b * BLOCK, min(d, (b + 1) * BLOCK)
        y = x[..., b0:b1] * np.ldexp(1.0, -s[..., b:b + 1])        # exact: a power of two
        y = np.clip(y, -e4m3.E4M3_MAX, e4m3.E4M3_MAX)
        codes[..., b0:b1] = e4m3.encode_rne(y.astype(np.float32))
    scales = np.zeros((T, H, SCALE_BYTES), dtype=np.uint8)
    scales[..., :nb] = (s + E8M0_BIAS).astype(np.uint8)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 value of each code times its block's power-of-two scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    out = e4m3.decode(codes).copy()
    for b in range(n_blocks(d)):
        b0, b1 = b * BLOCK, min(d, (b + 1) * BLOCK)
        s = scales[..., b:b + 1].astype(np.int64) - E8M0_BIAS
        out[..., b0:b1] *= np.ldexp(1.0, s)
    return out
