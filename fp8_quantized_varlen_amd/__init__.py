"""fp8_quantized_varlen_amd: FP8 ViT-encoder attention on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libfp8vit.so`` (include/fp8vit.h).
Argument marshalling only: every step of the hot path (amax, scale
bookkeeping, e4m3 quantization, varlen attention) runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream.

If the shared library has not been built, the first call raises
ImportError: there is no CPU fallback. (Importing the package itself works
without it, so that the build module can run.)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "LIB_PATH", "FP8VIT_DYNAMIC", "FP8VIT_STATIC", "Fp8VitError",
    "state_bytes", "new_state", "state_init", "state_set_static", "scales_update",
    "quantize_qkv", "attn_varlen", "attn_varlen_fp8out", "state_read", "state_write", "calibrated_values",
    "load_static_scales", "save_static_scales", "status_str",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8vit.so")
FP8VIT_DYNAMIC = 0
FP8VIT_STATIC = 1
_MODES = {"dynamic": FP8VIT_DYNAMIC, "static": FP8VIT_STATIC}

class _StateView(ctypes.Structure):
    _fields_ = [("ring", (ctypes.c_float * 16) * 3), ("count", ctypes.c_uint32),
                ("static_values", ctypes.c_float * 3), ("descale_used", ctypes.c_float * 3),
                ("amax_last", ctypes.c_float * 3), ("flags", ctypes.c_uint32)]


_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "fp8vit_state_bytes": (ctypes.c_size_t, []),
    "fp8vit_state_init": (ctypes.c_int, [_vp, _vp]),
    "fp8vit_load_static_scales": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(_f32)]),
    "fp8vit_state_set_static": (ctypes.c_int, [_vp, ctypes.POINTER(_f32), _vp]),
    "fp8vit_scales_update": (ctypes.c_int, [_vp, _vp, _vp]),
    "fp8vit_quantize_qkv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                           _vp, _vp, _vp, _vp, _vp]),
    "fp8vit_attn_varlen": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                          _vp, _i64, _vp]),
    "fp8vit_attn_varlen_fp8out": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                                 _vp, _vp, _i64, _vp]),
    "fp8vit_state_read": (ctypes.c_int, [_vp, ctypes.POINTER(_StateView), _vp]),
    "fp8vit_state_write": (ctypes.c_int, [_vp, ctypes.POINTER(_StateView), _vp]),
    "fp8vit_calibrated_values": (ctypes.c_int, [_vp, _f32, ctypes.POINTER(_f32), _vp]),
    "fp8vit_save_static_scales": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(_f32)]),
    "fp8vit_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}
_LIB = None


def _lib_handle():
    """Load libfp8vit.so on first use; raise ImportError if it was never built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m fp8_quantized_varlen_amd.build` "
                              "(the HIP library is required; there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


class _Lazy:
    def __getattr__(self, name):
        return getattr(_lib_handle(), name)


_lib = _Lazy()

EXPORTED_SYMBOLS = tuple(_SIGS)


class Fp8VitError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} (status {status})")
        self.status = status


def status_str(status: int) -> str:
    return _lib.fp8vit_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8VitError(fn, status)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def state_bytes() -> int:
    return int(_lib.fp8vit_state_bytes())


def state_init(state: torch.Tensor) -> torch.Tensor:
    _check("fp8vit_state_init", _lib.fp8vit_state_init(_ptr(state), _stream(state.device)))
    return state


def new_state(device="cuda") -> torch.Tensor:
    """Allocate and reset one layer's scale state (device bytes, 256-B aligned)."""
    st = torch.empty(state_bytes(), dtype=torch.uint8, device=device)
    return state_init(st)


def state_set_static(state: torch.Tensor, values_qkv: Sequence[float]) -> None:
    arr = (_f32 * 3)(*[float(x) for x in values_qkv])
    _check("fp8vit_state_set_static", _lib.fp8vit_state_set_static(_ptr(state), arr, _stream(state.device)))


def scales_update(state: torch.Tensor, amax_qkv: torch.Tensor) -> None:
    """Push a device float32[3] amax triple into the ring (bookkeeping only)."""
    assert amax_qkv.dtype == torch.float32 and amax_qkv.numel() == 3 and amax_qkv.is_contiguous()
    _check("fp8vit_scales_update", _lib.fp8vit_scales_update(_ptr(state), _ptr(amax_qkv), _stream(state.device)))


def _token_stride(x: torch.Tensor) -> int:
    T, H, d = x.shape
    if x.stride(2) != 1 or x.stride(1) != d:
        raise ValueError("expected [T, H, d] with heads and head_dim contiguous")
    return x.stride(0) if T > 0 else H * d


def quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, mode="dynamic",
                 out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """bf16 [T, H, d] (token stride may exceed H*d) -> e4m3 codes as uint8 [T, H, d]."""
    for x in (q, k, v):
        if x.dtype != torch.bfloat16 or x.dim() != 3:
            raise ValueError("q, k, v must be bf16 [T, H, d]")
    T, H, d = q.shape
    if out is None:
        out = tuple(torch.empty((T, H, d), dtype=torch.uint8, device=q.device) for _ in range(3))
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    st = _lib.fp8vit_quantize_qkv(_ptr(q), _ptr(k), _ptr(v), _token_stride(q), _token_stride(k), _token_stride(v),
                                  T, H, d, m, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(state),
                                  _stream(q.device))
    _check("fp8vit_quantize_qkv", st)
    return out


def attn_varlen(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                state: torch.Tensor, softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Non-causal FP8 attention per packed segment; returns bf16 [T, H, d]."""
    T, H, d = q8.shape
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 device tensor")
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=q8.device)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                 int(max_seqlen), T, H, d, float(softmax_scale), _ptr(state), _ptr(out), ld_out,
                                 _stream(q8.device))
    _check("fp8vit_attn_varlen", st)
    return out


def attn_varlen_fp8out(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens: torch.Tensor,
                       max_seqlen: int, state: torch.Tensor, out_descale: torch.Tensor, softmax_scale: float = 0.0,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """As attn_varlen, with e4m3 codes of O / out_descale (device float32[1]) as uint8 [T, H, d]."""
    T, H, d = q8.shape
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 device tensor")
    if out_descale.dtype != torch.float32 or out_descale.numel() != 1:
        raise ValueError("out_descale must be a float32 device tensor of one element")
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.uint8, device=q8.device)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen_fp8out(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                        int(max_seqlen), T, H, d, float(softmax_scale), _ptr(state),
                                        _ptr(out_descale), _ptr(out), ld_out, _stream(q8.device))
    _check("fp8vit_attn_varlen_fp8out", st)
    return out


def state_read(state: torch.Tensor) -> dict:
    view = _StateView()
    _check("fp8vit_state_read", _lib.fp8vit_state_read(_ptr(state), ctypes.byref(view), _stream(state.device)))
    return {
        "ring": [[view.ring[x][i] for i in range(16)] for x in range(3)],
        "count": int(view.count),
        "static_values": list(view.static_values),
        "descale_used": list(view.descale_used),
        "amax_last": list(view.amax_last),
        "flags": int(view.flags),
    }


def state_write(state: torch.Tensor, snapshot: dict) -> None:
    """Restore a state from a dict shaped like state_read's result (synchronous)."""
    view = _StateView()
    for x in range(3):
        for i in range(16):
            view.ring[x][i] = float(snapshot["ring"][x][i])
        view.static_values[x] = float(snapshot["static_values"][x])
        view.descale_used[x] = float(snapshot["descale_used"][x])
        view.amax_last[x] = float(snapshot["amax_last"][x])
    view.count = int(snapshot["count"])
    view.flags = int(snapshot.get("flags", 0))
    _check("fp8vit_state_write", _lib.fp8vit_state_write(_ptr(state), ctypes.byref(view), _stream(state.device)))


def calibrated_values(state: torch.Tensor, margin: float = 1.5) -> Tuple[float, float, float]:
    """fp32(margin x ring window max) per tensor, as a calibration saves them."""
    arr = (_f32 * 3)()
    _check("fp8vit_calibrated_values",
           _lib.fp8vit_calibrated_values(_ptr(state), float(margin), arr, _stream(state.device)))
    return (arr[0], arr[1], arr[2])


def save_static_scales(json_path: str, layer_name: str, values_qkv: Sequence[float]) -> None:
    arr = (_f32 * 3)(*[float(x) for x in values_qkv])
    _check("fp8vit_save_static_scales",
           _lib.fp8vit_save_static_scales(os.fsencode(json_path), layer_name.encode("utf-8"), arr))


def load_static_scales(json_path: str, layer_name: str) -> Tuple[float, float, float]:
    arr = (_f32 * 3)()
    st = _lib.fp8vit_load_static_scales(os.fsencode(json_path), layer_name.encode("utf-8"), arr)
    _check("fp8vit_load_static_scales", st)
    return (arr[0], arr[1], arr[2])
