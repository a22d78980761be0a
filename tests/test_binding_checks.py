"""The Python binding rejects malformed tensors before any library call:
wrong dtype, shape, strides, sizes or devices raise ValueError (CPU only; the
GPU is never reached because every check comes first)."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp8_quantized_varlen_amd", "libfp8vit.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfp8vit.so not built")

import fp8_quantized_varlen_amd as fv  # noqa: E402

T, H, D = 40, 2, 72


def bf(*shape, dev="cpu"):
    return torch.zeros(shape, dtype=torch.bfloat16, device=dev)


def u8(*shape, dev="cpu"):
    return torch.zeros(shape, dtype=torch.uint8, device=dev)


def state(dev="cpu"):
    return torch.zeros(fv.state_bytes(), dtype=torch.uint8, device=dev)


def cu(dev="cpu"):
    return torch.tensor([0, 17, T], dtype=torch.int32, device=dev)


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_quantize_rejects_bad_inputs():
    q = bf(T, H, D)
    raises("dtype", fv.quantize_qkv, q.float(), q, q, state())
    raises("3-D", fv.quantize_qkv, bf(T, H * D), bf(T, H * D), bf(T, H * D), state())
    raises("shape", fv.quantize_qkv, q, bf(T - 1, H, D), q, state())
    raises("shape", fv.quantize_qkv, q, q, bf(T, H, D + 8), state())
    raises("contiguous", fv.quantize_qkv, bf(T, D, H).transpose(1, 2), q, q, state())
    raises("state", fv.quantize_qkv, q, q, q, state()[:100])
    raises("state", fv.quantize_qkv, q, q, q, state().to(torch.int32))
    raises("mode", fv.quantize_qkv, q, q, q, state(), "sometimes")
    raises("tuple of three", fv.quantize_qkv, q, q, q, state(), out=(u8(T, H, D), u8(T, H, D)))
    raises("shape", fv.quantize_qkv, q, q, q, state(), out=(u8(T, H, D), u8(T, H, D), u8(T - 1, H, D)))
    raises("contiguous", fv.quantize_qkv, q, q, q, state(),
           out=(u8(T, H, D), u8(2 * T, H, D)[::2], u8(T, H, D)))
    raises("dtype", fv.quantize_qkv, q, q, q, state(), out=(u8(T, H, D), u8(T, H, D), bf(T, H, D)))
    # views of a fused [T, 3, H, d] buffer pass the checks (and stop at the device check on the host)
    fused = bf(T, 3, H, D)
    raises("GPU", fv.quantize_qkv, fused[:, 0], fused[:, 1], fused[:, 2], state())
    raises("different devices", fv.quantize_qkv, q, q, bf(T, H, D, dev="meta"), state())


def test_attention_rejects_bad_inputs():
    c = u8(T, H, D)
    raises("dtype", fv.attn_varlen, bf(T, H, D), c, c, cu(), 23, state())
    raises("shape", fv.attn_varlen, c, u8(T, H, D - 8), c, cu(), 23, state())
    raises("shape", fv.attn_varlen, c, c, u8(T + 1, H, D), cu(), 23, state())
    raises("contiguous", fv.attn_varlen, c, u8(2 * T, H, D)[::2], c, cu(), 23, state())
    raises("cu_seqlens", fv.attn_varlen, c, c, c, cu().long(), 23, state())
    raises("cu_seqlens", fv.attn_varlen, c, c, c, torch.zeros((2, 2), dtype=torch.int32), 23, state())
    raises("cu_seqlens", fv.attn_varlen, c, c, c, torch.zeros(6, dtype=torch.int32)[::2], 23, state())
    raises("max_seqlen", fv.attn_varlen, c, c, c, cu(), -1, state())
    raises("state", fv.attn_varlen, c, c, c, cu(), 23, state()[:8])
    raises("shape", fv.attn_varlen, c, c, c, cu(), 23, state(), out=bf(T - 1, H, D))
    raises("dtype", fv.attn_varlen, c, c, c, cu(), 23, state(), out=u8(T, H, D))
    raises("contiguous", fv.attn_varlen, c, c, c, cu(), 23, state(), out=bf(T, D, H).transpose(1, 2))
    # a padded token stride is allowed for the output; a stride below H*d is not
    raises("GPU", fv.attn_varlen, c, c, c, cu(), 23, state(), out=bf(T, H + 1, D)[:, :H])
    raises("different devices", fv.attn_varlen, c, c, c, cu(dev="meta"), 23, state())
    raises("different devices", fv.attn_varlen, c, c, c, cu(), 23, state(), out=bf(T, H, D, dev="meta"))


def test_fp8_output_rejects_bad_inputs():
    c = u8(T, H, D)
    one = torch.ones(1, dtype=torch.float32)
    raises("out_descale", fv.attn_varlen_fp8out, c, c, c, cu(), 23, state(), torch.ones(2))
    raises("out_descale", fv.attn_varlen_fp8out, c, c, c, cu(), 23, state(), one.double())
    raises("dtype", fv.attn_varlen_fp8out, c, c, c, cu(), 23, state(), one, out=bf(T, H, D))
    raises("shape", fv.attn_varlen_fp8out, c, c, c, cu(), 23, state(), one, out=u8(T, H, 2 * D))
    raises("different devices", fv.attn_varlen_fp8out, c, c, c, cu(), 23, state(), one.to("meta"))
    raises("GPU", fv.attn_varlen_fp8out, c, c, c, cu(), 23, state(), one)


def test_state_calls_reject_bad_states():
    raises("state", fv.state_init, state()[:10])
    raises("GPU", fv.state_init, state())
    raises("state", fv.state_set_static, torch.zeros(512, dtype=torch.float32), [1.0, 1.0, 1.0])
    raises("amax_qkv", fv.scales_update, state(), torch.zeros(4, dtype=torch.float32))
    raises("different devices", fv.scales_update, state(), torch.zeros(3, dtype=torch.float32, device="meta"))
    raises("state", fv.state_read, state()[:4])
    raises("state", fv.calibrated_values, "not a tensor")
