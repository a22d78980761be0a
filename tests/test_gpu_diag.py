"""GPU checks of the state's diagnostics against the oracle:

* the saturation count (FP8VIT_FLAG_COUNT_SATURATION): per tensor, the number
  of elements the quantizer's clamp changes equals oracle.quant.saturated_count
  at the descale in use, in static and dynamic mode, contiguous and strided
  inputs, and for the V pass of the block-scaled quantizer; counting leaves
  the codes bit for bit unchanged, counts add up over calls, and setting the
  flags restarts them;
* fp8vit_check_cu_seqlens: the device bits equal oracle.varlen's on valid and
  invalid boundary arrays (only the check kernel sees the invalid ones).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_qkv
from tests.gpu_helpers import codes_np, fv, require_gpu, to_dev
from tests.test_oracle_aux import CU_CASES

pytestmark = pytest.mark.gpu


def _expected(bits3, descales):
    return [oracle.quant.saturated_count(b, d) for b, d in zip(bits3, descales)]


@pytest.mark.parametrize("strided", [False, True])
def test_saturation_count_static(strided):
    dev = require_gpu()
    T, H, d = 1000, 4, 72
    qkv = make_qkv(71, T, H, d, outlier_frac=0.003, outlier_scale=30.0)
    amax = [float(oracle.quant.amax(b)) for b in qkv]
    values = [0.5 * amax[0], 0.25 * amax[1], 1.5 * amax[2]]   # V has headroom: count 0
    if strided:
        fused = to_dev(np.stack(qkv, axis=1), dev)            # [T, 3, H, d]
        x = (fused[:, 0], fused[:, 1], fused[:, 2])
    else:
        x = tuple(to_dev(b, dev) for b in qkv)
    st = fv.new_state(dev)
    fv.state_set_static(st, values)
    plain = fv.quantize_qkv(*x, st, "static")
    fv.state_set_flags(st, fv.FP8VIT_FLAG_COUNT_SATURATION)
    counted = fv.quantize_qkv(*x, st, "static")
    torch.cuda.synchronize()
    for a, b in zip(plain, counted):
        assert torch.equal(a, b)
    view = fv.state_read(st)
    want = _expected(qkv, view["descale_used"])
    assert want[0] > 0 and want[1] > want[0] and want[2] == 0
    assert view["saturated"] == want and view["flags"] == fv.FP8VIT_FLAG_COUNT_SATURATION
    fv.quantize_qkv(*x, st, "static")
    assert fv.state_read(st)["saturated"] == [2 * n for n in want]
    fv.state_set_flags(st, 0)                                  # off: counts restart and stay at zero
    fv.quantize_qkv(*x, st, "static")
    assert fv.state_read(st)["saturated"] == [0, 0, 0]


def test_saturation_count_dynamic_and_mx():
    dev = require_gpu()
    T, H, d = 777, 3, 128
    qkv = make_qkv(72, T, H, d, outlier_frac=0.001)
    x = tuple(to_dev(b, dev) for b in qkv)
    st = fv.new_state(dev)
    fv.state_set_flags(st, fv.FP8VIT_FLAG_COUNT_SATURATION)
    fv.quantize_qkv(*x, st, "dynamic")
    view = fv.state_read(st)
    assert view["saturated"] == _expected(qkv, view["descale_used"])
    # block-scaled Q and K never clamp; the V pass counts at V's per-tensor descale
    st2 = fv.new_state(dev)
    fv.state_set_static(st2, [1.0, 1.0, 0.3 * float(oracle.quant.amax(qkv[2]))])
    fv.state_set_flags(st2, fv.FP8VIT_FLAG_COUNT_SATURATION)
    fv.quantize_qkv_mx(*x, st2, "static")
    view = fv.state_read(st2)
    want_v = oracle.quant.saturated_count(qkv[2], view["descale_used"][2])
    assert want_v > 0 and view["saturated"] == [0, 0, want_v]


def test_state_write_carries_the_diagnostics():
    dev = require_gpu()
    st = fv.new_state(dev)
    snap = fv.state_read(st)
    snap.update(flags=fv.FP8VIT_FLAG_COUNT_SATURATION, cu_check=5, saturated=[3, 2 ** 40, 7])
    fv.state_write(st, snap)
    back = fv.state_read(st)
    assert back["flags"] == 1 and back["cu_check"] == 5 and back["saturated"] == [3, 2 ** 40, 7]


@pytest.mark.parametrize("cu,T,m,bits", CU_CASES + [(list(range(0, 3001, 3)), 3000, 3, 0),
                                                    (list(range(0, 3001, 3))[:-2] + [2990, 3000], 3000, 3, 2 | 8)])
def test_check_cu_seqlens_matches_oracle(cu, T, m, bits):
    dev = require_gpu()
    assert oracle.varlen.cu_seqlens_errors(cu, T, m) == bits
    st = fv.new_state(dev)
    fv.check_cu_seqlens(torch.tensor(cu, dtype=torch.int32, device=dev), T, m, st)
    assert fv.state_read(st)["cu_check"] == bits
