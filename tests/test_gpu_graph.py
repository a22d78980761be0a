"""HIP-graph capture of the hot path (NEXT row f2): the scale state lives on the
device, so a captured forward keeps working across replays. Each replay is
checked against the eager result of the same input; in dynamic mode the ring
after the replays is checked against the oracle's ring on the same sequence."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_cu_seqlens, make_qkv
from tests.gpu_helpers import codes_np, f32bits, fv, require_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SEGLENS = (130, 0, 257, 64)
# (heads, head_dim): 4 heads run the narrow kernel; 64 heads the wide ones
# (the 32x32-block kernel at head_dim 72, the wide 16x16 shape at 128)
SHAPES = [(4, 72), (64, 72), (64, 128)]


def _inputs(seed, H, D):
    cu = make_cu_seqlens(SEGLENS)
    return make_qkv(seed, int(cu[-1]), H, D), cu


def _forward(bufs, st, mode, cu_d, maxlen):
    q, k, v, q8, k8, v8, out = bufs
    fv.quantize_qkv(q, k, v, st, mode, out=(q8, k8, v8))
    fv.attn_varlen(q8, k8, v8, cu_d, maxlen, st, out=out)


@pytest.mark.parametrize("H,D", SHAPES)
@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_graph_replays_match_eager(mode, H, D):
    dev = require_gpu()
    (qb, kb, vb), cu = _inputs(1, H, D)
    T = int(cu[-1])
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
    maxlen = max(SEGLENS)
    bufs = [to_dev(x, dev) for x in (qb, kb, vb)]
    bufs += [torch.empty((T, H, D), dtype=torch.uint8, device=dev) for _ in range(3)]
    bufs += [torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)]
    st = fv.new_state(dev)
    st_eager = fv.new_state(dev)
    if mode == "static":
        fv.state_set_static(st, [7.0, 6.5, 5.25])
        fv.state_set_static(st_eager, [7.0, 6.5, 5.25])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _forward(bufs, st, mode, cu_d, maxlen)          # warm-up on the capture stream
        torch.cuda.synchronize()
        fv.state_init(st)
        if mode == "static":
            fv.state_set_static(st, [7.0, 6.5, 5.25])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            _forward(bufs, st, mode, cu_d, maxlen)
    torch.cuda.synchronize()
    ring = oracle.scales.AmaxRing()
    n_replays = 40 if mode == "dynamic" else 6
    for r in range(n_replays):
        (q2, k2, v2), _ = _inputs(100 + r, H, D)
        for buf, x in zip(bufs[:3], (q2, k2, v2)):
            buf.copy_(to_dev(x, dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [codes_np(c) for c in bufs[3:6]] + [bufs[6].float().cpu().numpy()]
        # eager forward of the same input on its own state
        ebufs = [to_dev(x, dev) for x in (q2, k2, v2)]
        ebufs += [torch.empty((T, H, D), dtype=torch.uint8, device=dev) for _ in range(3)]
        ebufs += [torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)]
        _forward(ebufs, st_eager, mode, cu_d, maxlen)
        torch.cuda.synchronize()
        want = [codes_np(c) for c in ebufs[3:6]] + [ebufs[6].float().cpu().numpy()]
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {r}"
        if mode == "dynamic":
            ring.push([oracle.quant.amax(x) for x in (q2, k2, v2)])
    state = fv.state_read(st)
    if mode == "dynamic":
        assert state["count"] == n_replays
        assert np.array_equal(f32bits(state["ring"]), f32bits(ring.ring))
        ds = np.float32([oracle.scales.descale_from_amax(a) for a in ring.window_max()])
        assert np.array_equal(f32bits(state["descale_used"]), f32bits(ds))
    else:
        assert state["count"] == 0
    assert state["flags"] == 0
