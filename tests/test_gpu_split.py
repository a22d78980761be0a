"""GPU parity of the key-split attention (fp8vit_attn_varlen_ws): grids of
(head, 256-query tile) items too small to fill the GPU cut every item's keys
into pieces whose normalised partials are combined by the last piece.

Checked on shapes whose split plan cuts the keys on an MI355X (256 CUs):
element by element against the quantization-emulating oracle (max-abs <=
1e-2 * max|V|) and against unquantized fp64 (relative RMS <= 5e-2); against
the unsplit kernel; run-to-run determinism; bitwise invariance under segment
permutation; HIP-graph replays.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_cu_seqlens, make_qkv
from tests.gpu_helpers import ATOL_FRAC_OF_VMAX, REL_RMS_VS_FP64, codes_np, fv, rel_rms, require_gpu, to_dev, vmax_of

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

# (segment lengths, heads): one segment of 4096 tokens at 8 heads (128 items
# of 32 key tiles: two pieces each, one round), and a ragged batch with a
# one-token, an empty and a three-tile segment (168 items by the launch's
# upper bound, three pieces each; the short segments' items are not split).
SPLIT_CASES = [((4096,), 8), ((5000, 1, 4000, 0, 300), 4)]


def _setup(seglens, H, seed, dev):
    cu = make_cu_seqlens(seglens)
    T = int(cu[-1])
    qb, kb, vb = make_qkv(seed, T, H, 72)
    st = fv.new_state(dev)
    codes = fv.quantize_qkv(to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev), st, "dynamic")
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
    return cu, (qb, kb, vb), codes, st, cu_d


def _ws(seglens, H, dev):
    nbytes = fv.attn_workspace_bytes(len(seglens), max(seglens), sum(seglens), H, 72)
    assert nbytes > 0, "the split plan should cut the keys of this shape"
    return fv.attn_workspace(len(seglens), max(seglens), sum(seglens), H, 72, device=dev)


@pytest.mark.parametrize("seglens,H", SPLIT_CASES)
def test_split_attention_matches_oracle(seglens, H):
    dev = require_gpu()
    cu, (qb, kb, vb), (q8, k8, v8), st, cu_d = _setup(seglens, H, 7000 + H, dev)
    ws = _ws(seglens, H, dev)
    T = int(cu[-1])
    out = torch.full((T, H, 72), float("nan"), dtype=torch.bfloat16, device=dev)
    fv.attn_varlen_ws(q8, k8, v8, cu_d, max(seglens), st, ws, out=out)
    plain = fv.attn_varlen(q8, k8, v8, cu_d, max(seglens), st)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(o)), "unwritten output elements"
    ref = oracle.pipeline.forward(qb, kb, vb, cu, "dynamic", ring=oracle.scales.AmaxRing())
    for c, r in zip((q8, k8, v8), ref.codes):
        assert np.array_equal(codes_np(c), r)
    vmax = vmax_of(vb)
    err = np.abs(o - ref.out).max() / vmax
    assert err <= ATOL_FRAC_OF_VMAX, err
    unq = oracle.pipeline.reference_unquantized(qb, kb, vb, cu)
    assert rel_rms(o, unq) <= REL_RMS_VS_FP64
    # the partials are rounded to f16 (relative 2^-11): within a bf16 step of the unsplit kernel
    d_plain = np.abs(o - plain.float().cpu().numpy()).max() / vmax
    assert d_plain <= 4e-3, d_plain


def test_split_attention_invariants():
    dev = require_gpu()
    seglens, H = SPLIT_CASES[1]
    cu, (qb, kb, vb), (q8, k8, v8), st, cu_d = _setup(seglens, H, 7100, dev)
    ws = _ws(seglens, H, dev)
    o1 = fv.attn_varlen_ws(q8, k8, v8, cu_d, max(seglens), st, ws).float().cpu().numpy()
    o2 = fv.attn_varlen_ws(q8, k8, v8, cu_d, max(seglens), st, ws).float().cpu().numpy()
    assert np.array_equal(o1, o2), "split attention is not run-to-run deterministic"
    # a workspace too small for any split gives the unsplit kernel exactly
    small = torch.zeros(256, dtype=torch.uint8, device=dev)
    o3 = fv.attn_varlen_ws(q8, k8, v8, cu_d, max(seglens), st, small).float().cpu().numpy()
    o4 = fv.attn_varlen(q8, k8, v8, cu_d, max(seglens), st).float().cpu().numpy()
    assert np.array_equal(o3, o4)
    # permuting segments: each segment's output bitwise unchanged (same amax, same plan)
    order = [2, 4, 0, 3, 1]   # 4000, 300, 5000, 0, 1
    segs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(seglens))]
    idx = np.concatenate([np.arange(*segs[i], dtype=np.int64) for i in order])
    perm = [seglens[i] for i in order]
    cu_dp = torch.from_numpy(np.asarray(make_cu_seqlens(perm), np.int32)).to(dev)
    q8p, k8p, v8p = (torch.from_numpy(codes_np(c)[idx]).to(dev) for c in (q8, k8, v8))
    op = fv.attn_varlen_ws(q8p, k8p, v8p, cu_dp, max(perm), st, ws).float().cpu().numpy()
    assert np.array_equal(op, o1[idx])


def test_split_attention_graph_replays():
    """Captured once (both kernels of the split), replayed with eager work in
    between: every replay equals the eager call."""
    dev = require_gpu()
    seglens, H = SPLIT_CASES[0]
    cu, _, (q8, k8, v8), st, cu_d = _setup(seglens, H, 7200, dev)
    ws = _ws(seglens, H, dev)
    out = torch.empty((sum(seglens), H, 72), dtype=torch.bfloat16, device=dev)
    eager = fv.attn_varlen_ws(q8, k8, v8, cu_d, max(seglens), st, ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fv.attn_varlen_ws(q8, k8, v8, cu_d, max(seglens), st, ws, out=out)
    for r in range(4):
        out.fill_(0)
        fv.attn_varlen(q8, k8, v8, cu_d, max(seglens), st)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
