"""The allocation-free attention entry point (fp8vit_attn_varlen_noalloc)
against the entry point it varies (fp8vit_attn_varlen_ws with a caller
workspace), through the C ABI: two calls in a row, the second with a smaller
input, both on shapes whose plan splits the keys (so the library's static
workspace is used and the second call overwrites the first's partials), then
a problem that does not split. Outputs must be identical bit for bit (same
plan, same kernels) and within the attention tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_cu_seqlens, make_qkv
from tests.gpu_helpers import ATOL_FRAC_OF_VMAX, fv, require_gpu, to_dev, vmax_of

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

# larger split problem first (168 items, three pieces), then a smaller one
# (128 items, two pieces), then one that does not split
CALLS = [((5000, 1, 4000, 0, 300), 4, True), ((2048,), 16, True), ((300, 129), 16, False)]


def test_noalloc_matches_workspace_entry_point():
    dev = require_gpu()
    for i, (seglens, H, splits) in enumerate(CALLS):
        cu = make_cu_seqlens(seglens)
        T, L = int(cu[-1]), max(seglens)
        qb, kb, vb = make_qkv(9100 + i, T, H, 72)
        st = fv.new_state(dev)
        q8, k8, v8 = fv.quantize_qkv(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, "dynamic")
        cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
        assert (fv.attn_workspace_bytes(len(seglens), L, T, H, 72) > 0) == splits
        ws = fv.attn_workspace(len(seglens), L, T, H, 72, device=dev)
        out_na = torch.full((T, H, 72), float("nan"), dtype=torch.bfloat16, device=dev)
        fv.attn_varlen_noalloc(q8, k8, v8, cu_d, L, st, out=out_na)
        ref = fv.attn_varlen_ws(q8, k8, v8, cu_d, L, st, ws)
        torch.cuda.synchronize()
        assert torch.equal(out_na, ref), f"call {i}: differs from fp8vit_attn_varlen_ws"
        o = out_na.float().cpu().numpy().astype(np.float64)
        orc = oracle.pipeline.forward(qb, kb, vb, cu, "dynamic", ring=oracle.scales.AmaxRing())
        err = np.abs(o - orc.out).max() / vmax_of(vb)
        assert err <= ATOL_FRAC_OF_VMAX, (i, err)
