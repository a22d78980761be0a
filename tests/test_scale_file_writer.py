"""The library's scale-file writer (fp8vit_save_static_scales), host only.

The file format is the one the vLLM page "FP8 ViT Encoder Attention" gives in
its Scale File Format section: a JSON object from layer names to {"q", "k",
"v"} values that already include the calibration margin. Python's own json
module is the independent reader here: every file the writer produces must
parse with it, hold the same other entries as before, and give back exactly
the float32 values that were saved (the library's loader must agree)."""
import ctypes
import json
import locale
import math
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp8_quantized_varlen_amd", "libfp8vit.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfp8vit.so not built (run __graft_entry__.build())")

LAYER = "visual.blocks.0.attn.attn"


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(LIB)
    f3 = ctypes.POINTER(ctypes.c_float)
    lib.fp8vit_save_static_scales.argtypes = [ctypes.c_char_p, ctypes.c_char_p, f3]
    lib.fp8vit_load_static_scales.argtypes = [ctypes.c_char_p, ctypes.c_char_p, f3]
    return lib


def save(lib, path, layer, vals):
    arr = (ctypes.c_float * 3)(*[float(v) for v in vals])
    return lib.fp8vit_save_static_scales(os.fsencode(str(path)), layer.encode("utf-8"), arr)


def load(lib, path, layer):
    out = (ctypes.c_float * 3)()
    st = lib.fp8vit_load_static_scales(os.fsencode(str(path)), layer.encode("utf-8"), out)
    return st, np.array(out, dtype=np.float32)


def pairs(path):
    return json.loads(open(path, encoding="utf-8").read(), object_pairs_hook=lambda p: p)


def test_round_trip_is_bit_exact_over_the_float_range(lib, tmp_path):
    rng = np.random.default_rng(7)
    vals = (rng.uniform(1, 2, (64, 3)) * np.exp2(rng.integers(-140, 127, (64, 3)))).astype(np.float32)
    edge = np.array([[np.finfo(np.float32).max, np.finfo(np.float32).tiny, np.float32(1e-45)],
                     [0.1, 1.0 / 3.0, 448.0], [1.5, 224.0, np.nextafter(np.float32(1), np.float32(2))]],
                    dtype=np.float32)
    vals = np.concatenate([vals[vals.min(axis=1) > 0], edge])
    p = tmp_path / "scales.json"
    for i, v in enumerate(vals):
        assert save(lib, p, f"layer.{i}", v) == 0
    doc = json.load(open(p))
    assert list(doc) == [f"layer.{i}" for i in range(len(vals))]
    for i, v in enumerate(vals):
        st, got = load(lib, p, f"layer.{i}")
        assert st == 0 and got.tobytes() == v.tobytes(), (i, v, got)
        py = np.array([doc[f"layer.{i}"][k] for k in "qkv"], dtype=np.float64).astype(np.float32)
        assert py.tobytes() == v.tobytes(), (i, v, py)


def test_shortest_text_and_file_layout(lib, tmp_path):
    p = tmp_path / "s.json"
    p.write_text('{"x": 1}')
    assert save(lib, p, "y", [1.5, 224.0, 0.1]) == 0
    assert p.read_text() == '{\n  "x": 1,\n  "y": {"q": 1.5, "k": 224, "v": 0.1}\n}\n'
    assert sorted(os.listdir(tmp_path)) == ["s.json"]          # no sibling file left behind


def test_other_entries_are_kept(lib, tmp_path):
    text = ('{"visual.blocks.1.attn.attn": {"q_scale": 218.0, "k_scale": 195.5, "v_scale": 207},\n'
            ' "meta": {"note": "tab\\there \\"quoted\\" \\\\ caf\\u00e9 \\ud83d\\ude00", "list": [1, 2.5, -0.0, 1e300,'
            ' 0.1, true, false, null, [], {}], "tiny": 5e-324},\n'
            ' "%s": {"q": 1, "k": 2, "v": 3},\n'
            ' "dup": 1, "dup": {"q": 9, "k": 9, "v": 9}}' % LAYER)
    p = tmp_path / "s.json"
    p.write_text(text, encoding="utf-8")
    before = pairs(p)
    assert save(lib, p, LAYER, [2.0, 4.0, 8.0]) == 0
    after = pairs(p)
    assert [k for k, _ in after] == [k for k, _ in before]       # same keys, same order, duplicates kept
    for (kb, vb), (ka, va) in zip(before, after):
        if kb == LAYER:
            assert va == [("q", 2.0), ("k", 4.0), ("v", 8.0)]
        else:
            assert repr(va) == repr(vb), kb                      # repr tells -0.0 from 0.0
    assert load(lib, p, "visual.blocks.1.attn.attn") == (0, pytest.approx(np.float32([218.0, 195.5, 207.0])))
    st, got = load(lib, p, "dup")
    assert st == 0 and got.tolist() == [9.0, 9.0, 9.0]           # last occurrence still wins


def test_layer_replaced_in_place_and_later_duplicates_dropped(lib, tmp_path):
    p = tmp_path / "s.json"
    p.write_text('{"a": {"q": 1, "k": 1, "v": 1}, "b": 2, "a": {"q": 5, "k": 5, "v": 5}}')
    assert save(lib, p, "a", [3.0, 3.0, 3.0]) == 0
    assert pairs(p) == [("a", [("q", 3.0), ("k", 3.0), ("v", 3.0)]), ("b", 2)]
    st, got = load(lib, p, "a")
    assert st == 0 and got.tolist() == [3.0, 3.0, 3.0]


@pytest.mark.parametrize("initial", [None, "", "  \n\t ", "﻿{}", "{}"])
def test_missing_empty_or_bom_file_starts_fresh(lib, tmp_path, initial):
    p = tmp_path / "s.json"
    if initial is not None:
        p.write_text(initial, encoding="utf-8")
    assert save(lib, p, LAYER, [224.0, 198.0, 210.0]) == 0
    assert json.load(open(p)) == {LAYER: {"q": 224.0, "k": 198.0, "v": 210.0}}


def test_awkward_layer_names_round_trip(lib, tmp_path):
    p = tmp_path / "s.json"
    names = ['x"y\\z', "tab\tand\nnewline", "café.blocks.0", "\x01ctl", ""]
    for i, n in enumerate(names):
        assert save(lib, p, n, [i + 1.0, 2.0, 3.0]) == 0
    doc = json.load(open(p, encoding="utf-8"))
    assert list(doc) == names
    for i, n in enumerate(names):
        st, got = load(lib, p, n)
        assert st == 0 and got[0] == i + 1.0


@pytest.mark.parametrize("bad", [[0.0, 1, 1], [1, -1, 1], [1, 1, float("nan")], [float("inf"), 1, 1], [-0.0, 1, 1]])
def test_invalid_values_leave_the_file_untouched(lib, tmp_path, bad):
    p = tmp_path / "s.json"
    p.write_text('{"a": 1}')
    assert save(lib, p, "a", bad) == 1
    assert p.read_text() == '{"a": 1}'


@pytest.mark.parametrize("text", ['{"a": 1', "[1, 2]", '"str"', '{"a": NaN}', "{} x"])
def test_malformed_file_is_not_overwritten(lib, tmp_path, text):
    p = tmp_path / "s.json"
    p.write_text(text)
    assert save(lib, p, "a", [1, 2, 3]) == 5
    assert p.read_text() == text


def test_io_errors(lib, tmp_path):
    assert save(lib, tmp_path / "no_such_dir" / "s.json", "a", [1, 2, 3]) == 4
    assert save(lib, tmp_path, "a", [1, 2, 3]) == 4                 # a directory
    assert lib.fp8vit_save_static_scales(None, b"a", (ctypes.c_float * 3)(1, 2, 3)) == 1
    assert lib.fp8vit_save_static_scales(b"x", None, (ctypes.c_float * 3)(1, 2, 3)) == 1
    assert lib.fp8vit_save_static_scales(b"x", b"a", None) == 1


def test_numbers_ignore_the_callers_locale(lib, tmp_path):
    old = locale.setlocale(locale.LC_NUMERIC)
    for name in ("de_DE.UTF-8", "de_DE.utf8", "fr_FR.UTF-8", "fr_FR.utf8"):
        try:
            locale.setlocale(locale.LC_NUMERIC, name)
            break
        except locale.Error:
            continue
    else:
        pytest.skip("no locale with a decimal comma is installed")
    try:
        assert locale.localeconv()["decimal_point"] == ","
        p = tmp_path / "s.json"
        assert save(lib, p, "a", [1.5, 0.25, 3.75]) == 0
        assert json.load(open(p)) == {"a": {"q": 1.5, "k": 0.25, "v": 3.75}}
        st, got = load(lib, p, "a")
        assert st == 0 and got.tolist() == [1.5, 0.25, 3.75]
    finally:
        locale.setlocale(locale.LC_NUMERIC, old)


def test_binding_round_trip(tmp_path):
    import fp8_quantized_varlen_amd as fv
    p = str(tmp_path / "s.json")
    vals = np.float32([1.0 / 3.0, math.pi, 1e-7])
    fv.save_static_scales(p, LAYER, vals)
    assert np.float32(fv.load_static_scales(p, LAYER)).tobytes() == vals.tobytes()
    with pytest.raises(fv.Fp8VitError):
        fv.save_static_scales(p, LAYER, [1.0, 0.0, 1.0])
