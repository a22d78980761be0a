"""The path through the C ABI alone: `tests/host/abi_gpu_driver` (plain C++,
include/fp8vit.h and the HIP runtime, no PyTorch or Python binding; built by
__graft_entry__.build()) saves and reloads the static scales through the JSON
calls, quantizes Q, K and V and runs the varlen attention with a workspace it
sizes itself. Its outputs must match the oracle as the binding's do: codes and
descales bit for bit, attention within max-abs 1e-2 * max|V|."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth import make_cu_seqlens, make_qkv
from tests.gpu_helpers import ATOL_FRAC_OF_VMAX, require_gpu, vmax_of

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "abi_gpu_driver")

# (segment lengths, heads, head_dim, mode): narrow hd72 static, wide hd72 static with a
# split of the keys (8 heads, one long segment), narrow hd128 dynamic
CASES = [((300, 1, 0, 129), 2, 72, "static"), ((4096,), 8, 72, "static"), ((200, 333), 3, 128, "dynamic")]


@pytest.mark.parametrize("seglens,H,d,mode", CASES)
def test_c_abi_driver_matches_oracle(tmp_path, seglens, H, d, mode):
    require_gpu()
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is missing: run __graft_entry__.build()")
    cu = make_cu_seqlens(seglens)
    T = int(cu[-1])
    qb, kb, vb = make_qkv(4242 + T + H + d, T, H, d)
    static = [float(oracle.quant.amax(x)) * 1.5 for x in (qb, kb, vb)]
    static = [float(np.float32(v)) for v in static]
    prob, res, js = tmp_path / "problem.bin", tmp_path / "result.bin", tmp_path / "scales.json"
    with open(prob, "wb") as f:
        np.array([T, H, d, len(seglens), max(seglens), 1 if mode == "static" else 0], np.int32).tofile(f)
        np.array(static, np.float32).tofile(f)
        np.asarray(cu, np.int32).tofile(f)
        for x in (qb, kb, vb):
            np.ascontiguousarray(x, np.uint16).tofile(f)
    r = subprocess.run([DRIVER, str(prob), str(res), str(js)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    n = T * H * d
    raw = np.fromfile(res, np.uint8)
    codes = [raw[i * n:(i + 1) * n].reshape(T, H, d) for i in range(3)]
    ds = raw[3 * n:3 * n + 12].view(np.float32)
    out = raw[3 * n + 12:].view(np.uint16).reshape(T, H, d)
    ref = oracle.pipeline.forward(qb, kb, vb, cu, mode, ring=oracle.scales.AmaxRing(), static_values=static)
    for g, c in zip(codes, ref.codes):
        assert np.array_equal(g, c)
    assert np.array_equal(ds.view(np.uint32), np.asarray(ref.descales, np.float32).view(np.uint32))
    o = oracle.quant.bf16_to_f32(out).astype(np.float64)
    err = np.abs(o - ref.out).max() / vmax_of(vb)
    assert err <= ATOL_FRAC_OF_VMAX, err
