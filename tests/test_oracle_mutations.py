"""Mutation checks: plant plausible mistakes in the oracle (on the CPU, via
monkeypatch) and confirm that at least one pin fails for each. This shows the
pins above are strong enough to catch a dropped term, a wrong sign or index,
or a transposed operand."""
import numpy as np
import pytest

from oracle import attention, e4m3, quant, scales
from tests import test_oracle_attention as ta
from tests import test_oracle_e4m3 as te
from tests import test_oracle_quant as tq
from tests import test_oracle_scales as ts

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _fails(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except AssertionError:
        return True
    return False


def test_mutation_swapped_k_v(monkeypatch):
    orig = attention._segment_head
    monkeypatch.setattr(attention, "_segment_head", lambda q, k, v, s: orig(q, v, k, s))
    assert _fails(ta.test_attention_brute_force, (5,))


def test_mutation_dropped_softmax_scale(monkeypatch):
    orig = attention._segment_head
    monkeypatch.setattr(attention, "_segment_head", lambda q, k, v, s: orig(q, k, v, 1.0))
    assert _fails(ta.test_attention_brute_force, (2, 6, 3))


def test_mutation_transposed_scores(monkeypatch):
    def bad(q, k, v, sigma):
        s = (k @ q.T) * sigma                     # S^T instead of S
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        return (p @ v) / p.sum(axis=1, keepdims=True)
    monkeypatch.setattr(attention, "_segment_head", bad)
    assert _fails(ta.test_attention_brute_force, (5,))


def test_mutation_normalised_by_column_sums(monkeypatch):
    def bad(q, k, v, sigma):
        s = (q @ k.T) * sigma
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        return (p @ v) / p.sum(axis=0)[:, None]
    monkeypatch.setattr(attention, "_segment_head", bad)
    assert _fails(ta.test_attention_brute_force, (5,))


def test_mutation_segments_ignored(monkeypatch):
    orig = attention.attention
    monkeypatch.setattr(attention, "attention", lambda q, k, v, cu, softmax_scale=None: orig(q, k, v, [0, q.shape[0]], softmax_scale))
    assert _fails(ta.test_attention_brute_force, (3, 0, 4, 1))


def test_mutation_ties_away_from_zero(monkeypatch):
    pos = e4m3.DECODE_TABLE[:0x7F]

    def bad(y):
        y = np.asarray(y, dtype=np.float32)
        a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
        hi = np.minimum(np.searchsorted(pos, a), 0x7E)
        lo = np.maximum(hi - 1, 0)
        code = np.where(a - pos[lo] < pos[hi] - a, lo, hi).astype(np.uint8)
        return code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    monkeypatch.setattr(e4m3, "encode_rne", bad)
    assert _fails(te.test_encode_matches_torch_on_ties_and_random)


def test_mutation_multiply_by_reciprocal(monkeypatch):
    def bad(bits, descale):
        x = quant.bf16_to_f32(bits)
        y = np.clip((x * (np.float32(1) / np.float32(descale))).astype(np.float32), -448, 448).astype(np.float32)
        return e4m3.encode_rne(y)
    monkeypatch.setattr(quant, "quantize", bad)
    assert any(_fails(tq.test_quantize_all_bf16_matches_torch_formula, d) for d in tq.DESCALES)


def test_mutation_delayed_ring(monkeypatch):
    def bad_push(self, a):
        prev = self.window_max()
        self.ring[:, self.count % 16] = np.asarray(a, np.float32)
        self.count += 1
        return prev
    monkeypatch.setattr(scales.AmaxRing, "push", bad_push)
    assert _fails(ts.test_ring_sliding_max, "ramp_up")


def test_mutation_no_floor(monkeypatch):
    monkeypatch.setattr(scales, "DESCALE_FLOOR", np.float32(0.0))
    assert _fails(ts.test_descale_floor)
