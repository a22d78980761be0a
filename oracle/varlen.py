"""Validity of a packed varlen batch description -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU baseline use this.

Source: vLLM page "FP8 ViT Encoder Attention", the note on ROCm's native
packed variable-length batches: the images and frames of a batch are packed
one after another along the token axis, and cu_seqlens holds the cumulative
segment boundaries (segment i is tokens cu[i] .. cu[i+1]-1). So a valid
cu_seqlens starts at 0, never decreases and ends at the packed token count;
the kernels also take a bound max_seqlen on every segment's length.
"""
from __future__ import annotations

import numpy as np

# Error bits, one per violated condition (0: valid).
CU_FIRST_NOT_ZERO = 1     # cu[0] != 0
CU_DECREASING = 2         # cu[i+1] < cu[i] for some i
CU_LAST_NOT_T = 4         # cu[num_segments] != total_tokens
CU_LONGER_THAN_MAX = 8    # cu[i+1] - cu[i] > max_seqlen for some i


def cu_seqlens_errors(cu, total_tokens: int, max_seqlen: int) -> int:
    """Bitwise or of the conditions above that cu_seqlens violates."""
    cu = [int(x) for x in np.asarray(cu).reshape(-1)]
    bits = 0
    if cu[0] != 0:
        bits |= CU_FIRST_NOT_ZERO
    for a, b in zip(cu[:-1], cu[1:]):
        if b < a:
            bits |= CU_DECREASING
        if b - a > max_seqlen:
            bits |= CU_LONGER_THAN_MAX
    if cu[-1] != total_tokens:
        bits |= CU_LAST_NOT_T
    return bits
