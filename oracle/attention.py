"""Non-causal attention over packed variable-length segments, in fp64.

Oracle code: used only by tests, smoke() and the bench's CPU baseline.

What it computes (vLLM page "FP8 ViT Encoder Attention": packed variable-length
image and video batches are attended natively, segment by segment; ViT encoder
attention is non-causal self-attention): for every segment [cu[i], cu[i+1]) and
every head h, with the segment's rows of Q, K, V for that head,

    S = Q K^T * sigma,   P = exp(S - rowmax(S)),   O = (P V) / rowsum(P).

Readings:
  R10 sigma is the fp32 value of 1/sqrt(d) unless the caller passes another
      fp32 softmax scale; it is promoted to fp64 here.
  R11 probabilities are not quantized in the oracle (that is a kernel-internal
      precision choice); the oracle is exact attention on whatever Q/K/V it is
      given (dequantized e4m3 values, or the bf16 values for the unquantized
      reference).
Tokens of different segments never interact. Zero-length segments own no rows.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 512


def default_softmax_scale(head_dim: int) -> np.float32:
    """fp32(1/sqrt(d)), rounded once from the fp64 value."""
    return np.float32(1.0 / np.sqrt(np.float64(head_dim)))


def _segment_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, sigma: float) -> np.ndarray:
    """One (segment, head): q [L, d], k [L, d], v [L, d] in fp64 -> o [L, d]."""
    L = q.shape[0]
    o = np.empty((L, v.shape[1]), dtype=np.float64)
    kt = k.T.copy()
    for r0 in range(0, L, ROW_CHUNK):
        r1 = min(L, r0 + ROW_CHUNK)
        s = (q[r0:r1] @ kt) * sigma
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        o[r0:r1] = (p @ v) / p.sum(axis=1, keepdims=True)
    return o


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens, softmax_scale=None) -> np.ndarray:
    """q, k, v: float arrays [T, H, d]; returns fp64 [T, H, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, d = q.shape
    sigma = np.float64(default_softmax_scale(d) if softmax_scale is None else np.float32(softmax_scale))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros((T, H, v.shape[2]), dtype=np.float64)
    for i in range(len(cu) - 1):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        if s1 <= s0:
            continue
        for h in range(H):
            out[s0:s1, h] = _segment_head(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], sigma)
    return out


def attention_rows(q, k, v, cu_seqlens, rows, softmax_scale=None) -> np.ndarray:
    """Outputs of selected (token, head) rows only: returns fp64 [len(rows), d].

    Used to check full-size runs on a sample of rows. Each row attends over the
    whole segment that contains its token."""
    q = np.asarray(q)
    T, H, d = q.shape
    sigma = np.float64(default_softmax_scale(d) if softmax_scale is None else np.float32(softmax_scale))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    res = np.zeros((len(rows), v.shape[2]), dtype=np.float64)
    for n, (t, h) in enumerate(rows):
        seg = int(np.searchsorted(cu, t, side="right") - 1)
        s0, s1 = int(cu[seg]), int(cu[seg + 1])
        qi = np.asarray(q[t, h], dtype=np.float64)
        ks = np.asarray(k[s0:s1, h], dtype=np.float64)
        vs = np.asarray(v[s0:s1, h], dtype=np.float64)
        s = (ks @ qi) * sigma
        p = np.exp(s - s.max())
        res[n] = (p @ vs) / p.sum()
    return res
