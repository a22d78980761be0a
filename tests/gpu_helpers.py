"""Helpers shared by the GPU tests: move seeded bf16 bits to the device, run the
HIP path through the C ABI binding, and compare with the CPU oracle."""
import numpy as np
import pytest
import torch

try:
    import fp8_quantized_varlen_amd as fv
except ImportError as e:  # the GPU tests need the built library
    fv = None
    _IMPORT_ERROR = e

import oracle

# Tolerances (stated in the design notes): attention output vs the
# quantization-emulating oracle, max-abs relative to max|V|; and relative RMS
# vs unquantized fp64 attention.
ATOL_FRAC_OF_VMAX = 1e-2
REL_RMS_VS_FP64 = 5e-2


def require_gpu():
    if fv is None:
        pytest.fail(f"HIP library not importable: {_IMPORT_ERROR}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def codes_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().astype(np.uint8)


def f32bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def vmax_of(vbits: np.ndarray) -> float:
    return float(np.abs(oracle.quant.bf16_to_f32(vbits)).max())


def rel_rms(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))
