"""The binding passes the caller's current stream: the raw stream handle it
reads equals torch's current stream on the default stream and inside a
side-stream context, and work launched there is ordered on that stream."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_qkv
from tests.gpu_helpers import codes_np, fv, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def test_stream_handle_is_torch_current_stream():
    dev = require_gpu()
    assert fv._stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        assert fv._stream(dev) == s.cuda_stream == torch.cuda.current_stream(dev).cuda_stream
    assert fv._stream(dev) == torch.cuda.current_stream(dev).cuda_stream


def test_quantize_on_a_side_stream():
    dev = require_gpu()
    T, H, d = 300, 4, 72
    qb, kb, vb = make_qkv(41, T, H, d)
    q, k, v = (to_dev(x, dev) for x in (qb, kb, vb))
    st = fv.new_state(dev)
    fv.state_set_static(st, [5.0, 6.0, 7.0])
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        q8, k8, v8 = fv.quantize_qkv(q, k, v, st, "static")
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    codes, _, _ = oracle.pipeline.quantize_step(qb, kb, vb, "static", static_values=[5.0, 6.0, 7.0])
    for got, want in zip((q8, k8, v8), codes):
        assert np.array_equal(codes_np(got), want)
