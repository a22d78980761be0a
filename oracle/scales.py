"""Per-tensor scale bookkeeping: dynamic amax ring, static values, descale.

Oracle code: used only by tests, smoke() and the bench's CPU baseline.

Sources:
  * vLLM page "FP8 ViT Encoder Attention", Usage: without a scale file the
    scales are dynamic -- a 16-entry circular buffer of the observed Q/K/V amax
    values drives the per-forward scale update.
  * same page, Calibrate-Once Reuse Workflow: calibration runs dynamic scaling
    for 16 passes and saves the learned scales multiplied by a margin
    (default 1.5); Scale File Format: one q/k/v triple per attention layer.
  * atrex-bench #025 per_token_group_quant_fp8, Reference Implementation:
    scale = clamp(amax / fp8_max, min=1e-10), fp8_max = 448 for e4m3fn.

Readings (the pages leave these open):
  R1  file values are amax-like numbers that already carry the margin, so the
      descale is value / 448 (224/448 = 0.5 for the page's example).
  R2  the ring is current-inclusive: this forward's amax is pushed first and
      the window max over all 16 slots (including it) sets this forward's scale.
  R3  the ring starts as zeros; amax >= 0 so empty slots never win the max.
  R4  the 1e-10 floor of the page's formula applies to the per-tensor descale.
  R13 the static path does not multiply by the margin again.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = np.float32(448.0)
DESCALE_FLOOR = np.float32(1e-10)
RING_SLOTS = 16


def descale_from_amax(A) -> np.float32:
    """descale = max(fp32(A / 448), fp32(1e-10)), IEEE fp32 division."""
    A = np.float32(A)
    with np.errstate(over="ignore", invalid="ignore"):
        d = np.float32(A / FP8_MAX)
    return np.float32(max(d, DESCALE_FLOOR))


class AmaxRing:
    """The 16-slot circular buffer of observed (q, k, v) amax values."""

    def __init__(self):
        self.ring = np.zeros((3, RING_SLOTS), dtype=np.float32)
        self.count = 0

    def push(self, amax_qkv) -> np.ndarray:
        """Record this forward's amax triple; return the window max per tensor."""
        a = np.asarray(amax_qkv, dtype=np.float32).reshape(3)
        self.ring[:, self.count % RING_SLOTS] = a
        self.count += 1
        return self.window_max()

    def window_max(self) -> np.ndarray:
        return self.ring.max(axis=1).astype(np.float32)


def dynamic_descales(ring: AmaxRing, amax_qkv) -> np.ndarray:
    """One dynamic forward: push, then descale from the 16-slot window max."""
    A = ring.push(amax_qkv)
    return np.array([descale_from_amax(a) for a in A], dtype=np.float32)


def static_descales(values_qkv) -> np.ndarray:
    """Static forward: descale straight from the file values (margin included)."""
    v = np.asarray(values_qkv, dtype=np.float32).reshape(3)
    return np.array([descale_from_amax(x) for x in v], dtype=np.float32)


def calibrated_values(ring: AmaxRing, margin: float = 1.5) -> np.ndarray:
    """Values to save after calibration: fp32(margin * window max) per tensor."""
    return (np.float32(margin) * ring.window_max()).astype(np.float32)
