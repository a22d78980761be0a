"""Seeded synthetic workloads for FP8 ViT-encoder attention.

This module only *makes inputs*: shapes, segment tables and bf16 bit patterns
drawn from a seeded generator. It holds none of the method's arithmetic (no
amax, no scales, no quantization, no attention), so both the HIP path's tests
and the CPU oracle may use it without sharing any computation.

Workload shapes follow the pages' own measurements of ViT encoder attention:
16 heads, head_dim 72 (the MI300X AITER table on the vLLM "FP8 ViT Encoder
Attention" page, Performance section) and head_dim 128 at sequence length 8192
(the cuDNN kernel table on the same page); packed image + video-frame batches
(same page, note on packed variable-length batches). Inputs are standard
normal, as in the input-generation snippet of the atrex-bench page for
per_token_group_quant_fp8.

Recipe (host numpy, PCG64):
  * rng = numpy.random.Generator(numpy.random.PCG64(seed))
  * for X in (q, k, v), in that order: x = rng.standard_normal((T, H, d), float32)
  * optional outliers: exactly round(frac * T*H*d) flat positions drawn without
    replacement from the same generator (after that tensor's normals), whose
    float32 values are multiplied by `outlier_scale` before rounding
  * bf16 by round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_qkv",
    "make_cu_seqlens",
    "device_randn_bf16",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest, ties to even) and return uint16 bits.

    Inputs here are always finite (normal samples), so no NaN handling."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (used to build inputs)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def device_randn_bf16(shape: Sequence[int], seed: int, device, chunk: int = 1 << 28):
    """Standard-normal bf16 tensor made on the device by torch's seeded
    generator, a chunk of float32 samples at a time (rounded to nearest even).
    For the sizes at the library's limits, which are too large to make on the
    host; tests read back the slices they check."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def make_cu_seqlens(seglens: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(seglens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(seglens, dtype=np.int64))
    return cu


def make_qkv(seed: int, T: int, H: int, d: int, outlier_frac: float = 0.0,
             outlier_scale: float = 20.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Return q, k, v as uint16 bf16 bit arrays of shape [T, H, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    E = T * H * d
    for _ in range(3):
        x = rng.standard_normal((T, H, d), dtype=np.float32)
        if outlier_frac > 0.0 and E > 0:
            n_out = int(round(outlier_frac * E))
            if n_out > 0:
                idx = rng.choice(E, size=n_out, replace=False)
                flat = x.reshape(-1)
                flat[idx] *= np.float32(outlier_scale)
        out.append(f32_to_bf16_bits(x))
    return out[0], out[1], out[2]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: segment lengths, heads, head_dim and scaling recipe."""

    name: str
    seglens: Tuple[int, ...]
    heads: int
    head_dim: int
    mode: str                 # "dynamic" or "static"
    seed: int                 # seed of the measured input
    warm_seeds: Tuple[int, ...] = ()   # dynamic warm-ups / static calibration draws
    outlier_frac: float = 0.0
    description: str = ""

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seglens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return make_cu_seqlens(self.seglens)

    @property
    def flops(self) -> int:
        """Useful attention flops: two matmuls per (query, key) pair, 2*d each."""
        return int(4 * self.heads * self.head_dim * sum(L * L for L in self.seglens))

    def inputs(self, seed: Optional[int] = None):
        s = self.seed if seed is None else seed
        return make_qkv(s, self.total_tokens, self.heads, self.head_dim, self.outlier_frac)


def _range(a: int, n: int = 16) -> Tuple[int, ...]:
    return tuple(range(a, a + n))


# The five workloads. Sizes: ViT attention with 16 heads; L=2304..16384 mirrors
# the MI300X AITER table; hd128 at L=8192 mirrors the cuDNN kernel table; the
# packed batch mixes three 14400-token images with eight 1024-token frames and
# runs once with static scales and once with the dynamic ring.
WORKLOADS = {
    "small_l256_hd72_dyn": Workload(
        "small_l256_hd72_dyn", (256,), 16, 72, "dynamic", 1, (),
        description="single segment L=256, 16 heads, hd72, dynamic scaling on an empty ring"),
    "l2304_hd72_dyn": Workload(
        "l2304_hd72_dyn", (2304,), 16, 72, "dynamic", 2, _range(2001),
        description="single segment L=2304, 16 heads, hd72, dynamic scaling after 16 warm-ups"),
    "l8192_hd72_static": Workload(
        "l8192_hd72_static", (8192,), 16, 72, "static", 3, _range(3001),
        description="single segment L=8192, 16 heads, hd72, static scales = 1.5 x calibrated"),
    "l16384_hd72_static": Workload(
        "l16384_hd72_static", (16384,), 16, 72, "static", 4, _range(4001),
        description="single segment L=16384, 16 heads, hd72, static scales = 1.5 x calibrated"),
    "l8192_hd128_dyn": Workload(
        "l8192_hd128_dyn", (8192,), 16, 128, "dynamic", 5, _range(5001),
        description="single segment L=8192, 16 heads, hd128, dynamic scaling after 16 warm-ups"),
    "packed_3x14400_8x1024_hd72": Workload(
        "packed_3x14400_8x1024_hd72", (14400, 14400, 14400) + (1024,) * 8, 16, 72, "static", 6,
        _range(6001), outlier_frac=0.001,
        description="packed batch 3x14400 + 8x1024 tokens, 16 heads, hd72, 0.1% outliers x20"),
    "packed_3x14400_8x1024_hd72_dyn": Workload(
        "packed_3x14400_8x1024_hd72_dyn", (14400, 14400, 14400) + (1024,) * 8, 16, 72, "dynamic", 6,
        _range(6001), outlier_frac=0.001,
        description="the same packed batch and input, dynamic scaling after 16 warm-ups"),
}
