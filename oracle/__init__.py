"""CPU oracle for FP8 ViT-encoder attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the hot path
computes: bf16 Q/K/V -> per-tensor amax -> scale bookkeeping (dynamic 16-entry
amax ring or static calibrated values) -> e4m3 quantization -> non-causal
attention per packed segment, in fp64.

Only the test suite (tests/), ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or run anything in this package. The GPU path
(``fp8_quantized_varlen_amd``) never imports it and shares no code with it; the
two meet only through the seeded input generator in ``synth``.

Sources (web pages, cited by title and section):
  * vLLM documentation page "FP8 ViT Encoder Attention": Usage (dynamic
    scaling with a 16-entry circular buffer of observed Q/K/V amax),
    Calibrate-Once Reuse Workflow (saved scales carry a margin, default 1.5),
    Scale File Format (per-layer q/k/v values and their *_scale aliases).
  * atrex-bench operator #025 "per_token_group_quant_fp8", Reference
    Implementation: scale = clamp(amax / fp8_max, min=1e-10) and
    q = (x_fp32 / scale).clamp(-fp8_max, fp8_max) cast to e4m3fn, with
    fp8_max = 448 for e4m3fn.

Readings where the pages leave a step open are listed in each function's
docstring (R-numbers match the readings table of the design notes).
Every function here is pinned by tests in tests/test_oracle_*.py against
brute force, library routines, closed forms or invariants; the attention
values themselves are never printed on the pages ("parity unpinned" against
page values: pinned instead by brute force and invariants).
"""
from . import e4m3, scales, quant, attention, mx, pipeline, varlen  # noqa: F401
