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
    "quantize_qkv", "attn_varlen", "attn_varlen_fp8out", "attn_workspace_bytes", "attn_workspace",
    "attn_varlen_ws", "attn_varlen_noalloc", "quantize_qkv_mx", "attn_varlen_mx", "state_read", "state_write",
    "state_set_flags", "check_cu_seqlens", "FP8VIT_FLAG_COUNT_SATURATION", "calibrated_values",
    "load_static_scales", "save_static_scales", "status_str",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8vit.so")
FP8VIT_DYNAMIC = 0
FP8VIT_STATIC = 1
FP8VIT_FLAG_COUNT_SATURATION = 1
FP8VIT_CU_FIRST_NOT_ZERO, FP8VIT_CU_DECREASING, FP8VIT_CU_LAST_NOT_T, FP8VIT_CU_LONGER_THAN_MAX = 1, 2, 4, 8
_MODES = {"dynamic": FP8VIT_DYNAMIC, "static": FP8VIT_STATIC}

class _StateView(ctypes.Structure):
    _fields_ = [("ring", (ctypes.c_float * 16) * 3), ("count", ctypes.c_uint32),
                ("static_values", ctypes.c_float * 3), ("descale_used", ctypes.c_float * 3),
                ("amax_last", ctypes.c_float * 3), ("flags", ctypes.c_uint32), ("cu_check", ctypes.c_uint32),
                ("saturated", ctypes.c_uint64 * 3)]


_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "fp8vit_state_bytes": (ctypes.c_size_t, []),
    "fp8vit_state_init": (ctypes.c_int, [_vp, _vp]),
    "fp8vit_load_static_scales": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(_f32)]),
    "fp8vit_state_set_static": (ctypes.c_int, [_vp, ctypes.POINTER(_f32), _vp]),
    "fp8vit_scales_update": (ctypes.c_int, [_vp, _vp, _vp]),
    "fp8vit_state_set_flags": (ctypes.c_int, [_vp, ctypes.c_uint32, _vp]),
    "fp8vit_check_cu_seqlens": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "fp8vit_quantize_qkv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                           _vp, _vp, _vp, _vp, _vp]),
    "fp8vit_attn_varlen": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                          _vp, _i64, _vp]),
    "fp8vit_attn_varlen_fp8out": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                                 _vp, _vp, _i64, _vp]),
    "fp8vit_attn_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32]),
    "fp8vit_quantize_qkv_mx": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                              _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp8vit_attn_varlen_mx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                             _vp, _vp, _i64, _vp]),
    "fp8vit_attn_varlen_ws": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                             _vp, _i64, _vp, ctypes.c_size_t, _vp]),
    "fp8vit_attn_varlen_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                                  _vp, _i64, _vp]),
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
    # First access to a name loads the library and keeps the function as an
    # attribute, so later calls skip this method.
    def __getattr__(self, name):
        fn = getattr(_lib_handle(), name)
        setattr(self, name, fn)
        return fn


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


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device) -> int:
    """The current stream of `device` as a raw hipStream_t."""
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


_STATE_BYTES = None


def state_bytes() -> int:
    global _STATE_BYTES
    if _STATE_BYTES is None:
        _STATE_BYTES = int(_lib.fp8vit_state_bytes())
    return _STATE_BYTES


def state_init(state: torch.Tensor) -> torch.Tensor:
    state = _state_tensor(state)
    _check("fp8vit_state_init", _lib.fp8vit_state_init(_ptr(state), _stream(_same_gpu(state=state))))
    return state


def new_state(device="cuda") -> torch.Tensor:
    """Allocate and reset one layer's scale state (device bytes, 256-B aligned)."""
    st = torch.empty(state_bytes(), dtype=torch.uint8, device=device)
    return state_init(st)


def state_set_static(state: torch.Tensor, values_qkv: Sequence[float]) -> None:
    state = _state_tensor(state)
    arr = (_f32 * 3)(*[float(x) for x in values_qkv])
    _check("fp8vit_state_set_static", _lib.fp8vit_state_set_static(_ptr(state), arr, _stream(_same_gpu(state=state))))


def scales_update(state: torch.Tensor, amax_qkv: torch.Tensor) -> None:
    """Push a device float32[3] amax triple into the ring (bookkeeping only)."""
    state = _state_tensor(state)
    amax_qkv = _tensor("amax_qkv", amax_qkv)
    if amax_qkv.dtype != torch.float32 or amax_qkv.numel() != 3 or not amax_qkv.is_contiguous():
        raise ValueError("amax_qkv must be a contiguous float32 tensor of 3 elements")
    dev = _same_gpu(state=state, amax_qkv=amax_qkv)
    _check("fp8vit_scales_update", _lib.fp8vit_scales_update(_ptr(state), _ptr(amax_qkv), _stream(dev)))


# Argument checks. They run before any library call, so a caller's mistake
# raises ValueError here instead of reaching a kernel with a wrong pointer,
# shape or stride. The library checks sizes and alignment again on its side.
_CODE_DTYPES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))


def _tensor(name: str, t) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    return t


def _bhd(name: str, t, dtypes, shape=None, contiguous=False) -> torch.Tensor:
    """A [T, H, d] tensor with heads and head_dim contiguous (token stride free
    unless `contiguous`)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(x) for x in dtypes)}, got {t.dtype}")
    sh = t.shape
    if len(sh) != 3:
        raise ValueError(f"{name} must be 3-D [tokens, heads, head_dim], got shape {tuple(sh)}")
    if shape is not None and sh != shape:
        raise ValueError(f"{name} has shape {tuple(sh)}, expected {tuple(shape)}")
    T, H, d = sh
    if T > 0 and H > 0 and d > 0:
        s0, s1, s2 = t.stride()
        if (H > 1 and s1 != d) or (d > 1 and s2 != 1):
            raise ValueError(f"{name}: heads and head_dim must be contiguous (strides {t.stride()})")
        # with heads and head_dim contiguous, [T, H, d] is contiguous iff the
        # token stride is H*d (or there is one token)
        if contiguous and T > 1 and s0 != H * d:
            raise ValueError(f"{name} must be contiguous [T, H, d]")
        if s0 < H * d:
            raise ValueError(f"{name}: token stride {s0} is below H*d = {H * d}")
    return t


def _state_tensor(state) -> torch.Tensor:
    state = _tensor("state", state)
    if state.dtype != torch.uint8 or not state.is_contiguous() or state.numel() < state_bytes():
        raise ValueError(f"state must be a contiguous uint8 tensor of at least {state_bytes()} bytes "
                         "(use new_state())")
    return state


def _same_gpu(**tensors) -> torch.device:
    """All tensors on one device, and that device a GPU."""
    first = None
    for t in tensors.values():
        if t is None:
            continue
        if first is None:
            first = t.device
        elif t.device != first:
            raise ValueError("tensors are on different devices: " +
                             ", ".join(f"{n}={t.device}" for n, t in tensors.items() if t is not None))
    if first.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {first}")
    return first


def _token_stride(x: torch.Tensor) -> int:
    T, H, d = x.shape
    return x.stride(0) if T > 0 else H * d


def _cu_seqlens(cu, T: int) -> torch.Tensor:
    cu = _tensor("cu_seqlens", cu)
    if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 1 or not cu.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor of num_segments + 1 entries")
    return cu


def quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, mode="dynamic",
                 out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """bf16 [T, H, d] (token stride may exceed H*d) -> e4m3 codes as uint8 [T, H, d]."""
    q = _bhd("q", q, (torch.bfloat16,))
    k = _bhd("k", k, (torch.bfloat16,), shape=q.shape)
    v = _bhd("v", v, (torch.bfloat16,), shape=q.shape)
    T, H, d = q.shape
    state = _state_tensor(state)
    if mode not in _MODES and mode not in (FP8VIT_DYNAMIC, FP8VIT_STATIC):
        raise ValueError(f"mode must be 'dynamic' or 'static', got {mode!r}")
    if out is not None:
        if not isinstance(out, (tuple, list)) or len(out) != 3:
            raise ValueError("out must be a tuple of three [T, H, d] uint8 tensors")
        out = tuple(_bhd(n, o, _CODE_DTYPES, shape=q.shape, contiguous=True) for n, o in zip(("q8", "k8", "v8"), out))
    dev = _same_gpu(q=q, k=k, v=v, state=state, **({} if out is None else dict(zip(("q8", "k8", "v8"), out))))
    if out is None:
        out = tuple(torch.empty((T, H, d), dtype=torch.uint8, device=dev) for _ in range(3))
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    st = _lib.fp8vit_quantize_qkv(_ptr(q), _ptr(k), _ptr(v), _token_stride(q), _token_stride(k), _token_stride(v),
                                  T, H, d, m, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(state),
                                  _stream(dev))
    _check("fp8vit_quantize_qkv", st)
    return out


def _attn_inputs(q8, k8, v8, cu_seqlens, max_seqlen, state):
    q8 = _bhd("q8", q8, _CODE_DTYPES, contiguous=True)
    k8 = _bhd("k8", k8, _CODE_DTYPES, shape=q8.shape, contiguous=True)
    v8 = _bhd("v8", v8, _CODE_DTYPES, shape=q8.shape, contiguous=True)
    cu_seqlens = _cu_seqlens(cu_seqlens, q8.shape[0])
    if int(max_seqlen) < 0:
        raise ValueError("max_seqlen must be >= 0")
    return q8, k8, v8, cu_seqlens, _state_tensor(state)


def attn_varlen(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                state: torch.Tensor, softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Non-causal FP8 attention per packed segment; returns bf16 [T, H, d]."""
    q8, k8, v8, cu_seqlens, state = _attn_inputs(q8, k8, v8, cu_seqlens, max_seqlen, state)
    T, H, d = q8.shape
    if out is not None:
        out = _bhd("out", out, (torch.bfloat16,), shape=q8.shape)
    dev = _same_gpu(q8=q8, k8=k8, v8=v8, cu_seqlens=cu_seqlens, state=state, out=out)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                 int(max_seqlen), T, H, d, float(softmax_scale), _ptr(state), _ptr(out), ld_out,
                                 _stream(dev))
    _check("fp8vit_attn_varlen", st)
    return out


def attn_workspace_bytes(num_segments: int, max_seqlen: int, total_tokens: int, num_heads: int,
                         head_dim: int) -> int:
    """Workspace fp8vit_attn_varlen_ws would use for this problem (0: it does not split)."""
    return int(_lib.fp8vit_attn_workspace_bytes(int(num_segments), int(max_seqlen), int(total_tokens),
                                                int(num_heads), int(head_dim)))


def attn_workspace(num_segments: int, max_seqlen: int, total_tokens: int, num_heads: int, head_dim: int,
                   device="cuda") -> torch.Tensor:
    """A workspace of the size attn_workspace_bytes gives (at least 256 bytes)."""
    n = max(256, attn_workspace_bytes(num_segments, max_seqlen, total_tokens, num_heads, head_dim))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def attn_varlen_ws(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens: torch.Tensor,
                   max_seqlen: int, state: torch.Tensor, workspace: torch.Tensor, softmax_scale: float = 0.0,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """attn_varlen with a caller workspace, which lets the kernel split the keys of a grid too
    small to fill the GPU (a second kernel combines the pieces)."""
    q8, k8, v8, cu_seqlens, state = _attn_inputs(q8, k8, v8, cu_seqlens, max_seqlen, state)
    T, H, d = q8.shape
    workspace = _tensor("workspace", workspace)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if out is not None:
        out = _bhd("out", out, (torch.bfloat16,), shape=q8.shape)
    dev = _same_gpu(q8=q8, k8=k8, v8=v8, cu_seqlens=cu_seqlens, state=state, workspace=workspace, out=out)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen_ws(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                    int(max_seqlen), T, H, d, float(softmax_scale), _ptr(state), _ptr(out), ld_out,
                                    _ptr(workspace), workspace.numel(), _stream(dev))
    _check("fp8vit_attn_varlen_ws", st)
    return out


def attn_varlen_noalloc(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens: torch.Tensor,
                        max_seqlen: int, state: torch.Tensor, softmax_scale: float = 0.0,
                        out: torch.Tensor = None) -> torch.Tensor:
    """attn_varlen_ws with the library's own static workspace: the library allocates nothing
    (pass `out` to allocate nothing here either). Calls that overlap on one GPU race."""
    q8, k8, v8, cu_seqlens, state = _attn_inputs(q8, k8, v8, cu_seqlens, max_seqlen, state)
    T, H, d = q8.shape
    if out is not None:
        out = _bhd("out", out, (torch.bfloat16,), shape=q8.shape)
    dev = _same_gpu(q8=q8, k8=k8, v8=v8, cu_seqlens=cu_seqlens, state=state, out=out)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen_noalloc(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                         int(max_seqlen), T, H, d, float(softmax_scale), _ptr(state), _ptr(out),
                                         ld_out, _stream(dev))
    _check("fp8vit_attn_varlen_noalloc", st)
    return out


def _mx_scales(name, t, shape):
    t = _tensor(name, t)
    if t.dtype != torch.uint8 or tuple(t.shape) != (shape[0], shape[1], 4) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor of shape ({shape[0]}, {shape[1]}, 4)")
    return t


def quantize_qkv_mx(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor, mode="dynamic",
                    out=None):
    """Block-scaled Q and K (e4m3 codes + E8M0 scales [T, H, 4] per 32-element block of
    head_dim), per-tensor V: returns (q8, k8, v8, q_scales, k_scales)."""
    q = _bhd("q", q, (torch.bfloat16,))
    k = _bhd("k", k, (torch.bfloat16,), shape=q.shape)
    v = _bhd("v", v, (torch.bfloat16,), shape=q.shape)
    T, H, d = q.shape
    state = _state_tensor(state)
    if mode not in _MODES and mode not in (FP8VIT_DYNAMIC, FP8VIT_STATIC):
        raise ValueError(f"mode must be 'dynamic' or 'static', got {mode!r}")
    if out is not None:
        if not isinstance(out, (tuple, list)) or len(out) != 5:
            raise ValueError("out must be a tuple (q8, k8, v8, q_scales, k_scales)")
        out = tuple(_bhd(n, o, _CODE_DTYPES, shape=q.shape, contiguous=True)
                    for n, o in zip(("q8", "k8", "v8"), out[:3])) + tuple(
            _mx_scales(n, o, q.shape) for n, o in zip(("q_scales", "k_scales"), out[3:]))
    dev = _same_gpu(q=q, k=k, v=v, state=state,
                    **({} if out is None else dict(zip(("q8", "k8", "v8", "q_scales", "k_scales"), out))))
    if out is None:
        out = tuple(torch.empty((T, H, d), dtype=torch.uint8, device=dev) for _ in range(3)) + tuple(
            torch.empty((T, H, 4), dtype=torch.uint8, device=dev) for _ in range(2))
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    st = _lib.fp8vit_quantize_qkv_mx(_ptr(q), _ptr(k), _ptr(v), _token_stride(q), _token_stride(k), _token_stride(v),
                                     T, H, d, m, *(_ptr(o) for o in out), _ptr(state), _stream(dev))
    _check("fp8vit_quantize_qkv_mx", st)
    return out


def attn_varlen_mx(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scales: torch.Tensor,
                   k_scales: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, state: torch.Tensor,
                   softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention on block-scaled Q and K (from quantize_qkv_mx); bf16 [T, H, d]."""
    q8, k8, v8, cu_seqlens, state = _attn_inputs(q8, k8, v8, cu_seqlens, max_seqlen, state)
    T, H, d = q8.shape
    q_scales = _mx_scales("q_scales", q_scales, q8.shape)
    k_scales = _mx_scales("k_scales", k_scales, q8.shape)
    if out is not None:
        out = _bhd("out", out, (torch.bfloat16,), shape=q8.shape)
    dev = _same_gpu(q8=q8, k8=k8, v8=v8, q_scales=q_scales, k_scales=k_scales, cu_seqlens=cu_seqlens, state=state,
                    out=out)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen_mx(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scales), _ptr(k_scales), _ptr(cu_seqlens),
                                    cu_seqlens.numel() - 1, int(max_seqlen), T, H, d, float(softmax_scale),
                                    _ptr(state), _ptr(out), ld_out, _stream(dev))
    _check("fp8vit_attn_varlen_mx", st)
    return out


def attn_varlen_fp8out(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens: torch.Tensor,
                       max_seqlen: int, state: torch.Tensor, out_descale: torch.Tensor, softmax_scale: float = 0.0,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """As attn_varlen, with e4m3 codes of O / out_descale (device float32[1]) as uint8 [T, H, d]."""
    q8, k8, v8, cu_seqlens, state = _attn_inputs(q8, k8, v8, cu_seqlens, max_seqlen, state)
    T, H, d = q8.shape
    out_descale = _tensor("out_descale", out_descale)
    if out_descale.dtype != torch.float32 or out_descale.numel() != 1:
        raise ValueError("out_descale must be a float32 tensor of one element")
    if out is not None:
        out = _bhd("out", out, _CODE_DTYPES, shape=q8.shape)
    dev = _same_gpu(q8=q8, k8=k8, v8=v8, cu_seqlens=cu_seqlens, state=state, out_descale=out_descale, out=out)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.uint8, device=dev)
    ld_out = out.stride(0) if T > 0 else H * d
    st = _lib.fp8vit_attn_varlen_fp8out(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                        int(max_seqlen), T, H, d, float(softmax_scale), _ptr(state),
                                        _ptr(out_descale), _ptr(out), ld_out, _stream(dev))
    _check("fp8vit_attn_varlen_fp8out", st)
    return out


def state_read(state: torch.Tensor) -> dict:
    state = _state_tensor(state)
    view = _StateView()
    _check("fp8vit_state_read", _lib.fp8vit_state_read(_ptr(state), ctypes.byref(view),
                                                       _stream(_same_gpu(state=state))))
    return {
        "ring": [[view.ring[x][i] for i in range(16)] for x in range(3)],
        "count": int(view.count),
        "static_values": list(view.static_values),
        "descale_used": list(view.descale_used),
        "amax_last": list(view.amax_last),
        "flags": int(view.flags),
        "cu_check": int(view.cu_check),
        "saturated": [int(x) for x in view.saturated],
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
    view.cu_check = int(snapshot.get("cu_check", 0))
    for x, n in enumerate(snapshot.get("saturated", (0, 0, 0))):
        view.saturated[x] = int(n)
    state = _state_tensor(state)
    _check("fp8vit_state_write", _lib.fp8vit_state_write(_ptr(state), ctypes.byref(view),
                                                         _stream(_same_gpu(state=state))))


def state_set_flags(state: torch.Tensor, flags: int) -> None:
    """Set the state's option bits (FP8VIT_FLAG_COUNT_SATURATION) and restart the
    saturation counts; state_read reports them under "saturated"."""
    state = _state_tensor(state)
    _check("fp8vit_state_set_flags",
           _lib.fp8vit_state_set_flags(_ptr(state), int(flags), _stream(_same_gpu(state=state))))


def check_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int, max_seqlen: int, state: torch.Tensor) -> None:
    """Check cu_seqlens on the device; state_read(state)["cu_check"] then holds the
    FP8VIT_CU_* bits of the conditions it violates (0: valid)."""
    cu_seqlens = _cu_seqlens(cu_seqlens, int(total_tokens))
    state = _state_tensor(state)
    dev = _same_gpu(cu_seqlens=cu_seqlens, state=state)
    _check("fp8vit_check_cu_seqlens",
           _lib.fp8vit_check_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, int(total_tokens),
                                        int(max_seqlen), _ptr(state), _stream(dev)))


def calibrated_values(state: torch.Tensor, margin: float = 1.5) -> Tuple[float, float, float]:
    """fp32(margin x ring window max) per tensor, as a calibration saves them."""
    state = _state_tensor(state)
    arr = (_f32 * 3)()
    _check("fp8vit_calibrated_values",
           _lib.fp8vit_calibrated_values(_ptr(state), float(margin), arr, _stream(_same_gpu(state=state))))
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
