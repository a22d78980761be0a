"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/fp8vit.h declares, rejects bad arguments before any HIP
call, and reads the static scale file format."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8vit.h")
LIB = os.path.join(ROOT, "fp8_quantized_varlen_amd", "libfp8vit.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfp8vit.so not built (run __graft_entry__.build())")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8vit_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), n


PAGES = ('vLLM page "FP8 ViT Encoder Attention"', 'atrex-bench operator #025', 'vLLM issue 29920',
         "FlashInfer PR", "Scale File Format")


def header_declarations():
    """(function name, the comment block right above its declaration)."""
    txt = open(HEADER).read()
    out = []
    for m in re.finditer(r"/\*((?:(?!\*/).)*)\*/\s*\n([^;{]*?\b(fp8vit_[a-z0-9_]+)\s*\([^;]*\);)", txt, re.S):
        out.append((m.group(3), m.group(1)))
    return out


def test_every_declaration_cites_its_passage():
    """Each entry point's comment names the page and section that defines the
    operation (a "Source:" line), or, for an entry point that the pages do not
    define, the callers it is for."""
    decls = header_declarations()
    assert sorted(n for n, _ in decls) == header_functions()
    for name, comment in decls:
        flat = " ".join(comment.replace("*", " ").split())
        m = re.search(r"Source: (.*)", flat)
        assert m, f"{name}: no Source: line"
        assert any(p in m.group(1) for p in PAGES) or "cannot allocate" in m.group(1), f"{name}: {m.group(1)}"


def test_binding_declares_the_same_symbols():
    import fp8_quantized_varlen_amd as fv
    assert sorted(fv.EXPORTED_SYMBOLS) == header_functions()


def test_status_strings(lib):
    lib.fp8vit_status_str.restype = ctypes.c_char_p
    seen = {lib.fp8vit_status_str(i) for i in range(7)}
    assert len(seen) == 7 and lib.fp8vit_status_str(0) == b"ok"
    assert lib.fp8vit_state_bytes() == 512 + 32 * 1024


def test_argument_validation_before_any_hip_call(lib):
    vp, null = ctypes.c_void_p, None
    fake = vp(0x10000)          # aligned but never dereferenced: validation fails first
    lib.fp8vit_quantize_qkv.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        vp, vp, vp, vp, vp]
    q = lib.fp8vit_quantize_qkv
    assert q(null, fake, fake, 1152, 1152, 1152, 10, 16, 72, 0, fake, fake, fake, fake, null) == 1
    assert q(fake, fake, fake, 1152, 1152, 1152, -1, 16, 72, 0, fake, fake, fake, fake, null) == 1
    assert q(fake, fake, fake, 1152, 1152, 1152, 10, 16, 72, 7, fake, fake, fake, fake, null) == 1
    assert q(fake, fake, fake, 1000, 1152, 1152, 10, 16, 72, 0, fake, fake, fake, fake, null) == 1
    assert q(vp(0x10008), fake, fake, 1152, 1152, 1152, 10, 16, 72, 0, fake, fake, fake, fake, null) == 2
    assert q(fake, fake, fake, 1156, 1152, 1152, 10, 16, 72, 0, fake, fake, fake, fake, null) == 2
    assert q(fake, fake, fake, 15, 15, 15, 10, 3, 5, 0, fake, fake, fake, fake, null) == 2
    # 32-bit chunk indices: T * H * d / 8 must stay below 2^31 (14913081 * 144 = 2^31 + 16)
    assert q(fake, fake, fake, 1152, 1152, 1152, 14913081, 16, 72, 0, fake, fake, fake, fake, null) == 2
    a = lib.fp8vit_attn_varlen
    a.argtypes = [vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_float, vp, vp, ctypes.c_int64, vp]
    assert a(fake, fake, fake, fake, 1, 10, 10, 16, 64, 0.0, fake, fake, 1152, null) == 2      # head_dim 64
    assert a(fake, fake, fake, null, 1, 10, 10, 16, 72, 0.0, fake, fake, 1152, null) == 1
    assert a(fake, fake, fake, fake, 1, 10, 10, 16, 72, float("nan"), fake, fake, 1152, null) == 1
    assert a(fake, fake, fake, fake, 1, 10, 10, 16, 72, 0.0, fake, fake, 100, null) == 1
    assert a(fake, fake, fake, fake, 1, 10, 10, 16, 72, 0.0, vp(0x10010), fake, 1152, null) == 2
    # empty problems are a no-op that never touches the device
    assert a(fake, fake, fake, fake, 0, 0, 0, 16, 72, 0.0, fake, fake, 1152, null) == 0
    # size limits, first rejected size (the kernels address each e4m3 tensor with
    # 31-bit offsets, up to three 128-key tiles past a segment's end): T = 1863752
    # tokens of 16 x 72 gives (T + 384) * 1152 = 2^31 + 1024
    assert a(fake, fake, fake, fake, 1, 1863752, 1863752, 16, 72, 0.0, fake, fake, 1152, null) == 2
    assert a(fake, fake, fake, fake, 4, 1000, 1863752, 16, 72, 0.0, fake, fake, 1152, null) == 2
    f8 = lib.fp8vit_attn_varlen_fp8out
    f8.argtypes = [vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_float, vp, vp, vp, ctypes.c_int64, vp]
    assert f8(fake, fake, fake, fake, 1, 10, 10, 16, 72, 0.0, fake, null, fake, 1152, null) == 1   # no descale
    assert f8(fake, fake, fake, fake, 1, 10, 10, 16, 72, 0.0, fake, vp(0x10002), fake, 1152, null) == 2
    assert f8(fake, fake, fake, fake, 1, 10, 10, 16, 72, 0.0, fake, fake, vp(0x10002), 1152, null) == 2
    assert f8(fake, fake, fake, fake, 1, 10, 10, 16, 72, 0.0, fake, fake, fake, 1150, null) == 1
    assert f8(fake, fake, fake, fake, 1, 10, 10, 16, 128, 0.0, fake, fake, fake, 2050, null) == 2
    assert f8(fake, fake, fake, fake, 0, 0, 0, 16, 72, 0.0, fake, fake, fake, 1152, null) == 0
    s = lib.fp8vit_state_set_static
    s.argtypes = [vp, ctypes.POINTER(ctypes.c_float), vp]
    for bad in ([0.0, 1.0, 1.0], [1.0, -2.0, 1.0], [1.0, 1.0, float("inf")], [float("nan"), 1.0, 1.0]):
        assert s(fake, (ctypes.c_float * 3)(*bad), null) == 1
    lib.fp8vit_state_init.argtypes = [vp, vp]
    assert lib.fp8vit_state_init(null, null) == 1
    assert lib.fp8vit_state_init(vp(0x10010), null) == 2
    c = lib.fp8vit_calibrated_values
    c.argtypes = [vp, ctypes.c_float, ctypes.POINTER(ctypes.c_float), vp]
    out = (ctypes.c_float * 3)()
    assert c(null, 1.5, out, null) == 1
    for bad in (0.0, -1.5, float("nan"), float("inf")):
        assert c(fake, bad, out, null) == 1
    assert c(vp(0x10010), 1.5, out, null) == 2
    from fp8_quantized_varlen_amd import _StateView
    w = lib.fp8vit_state_write
    w.argtypes = [vp, vp, vp]
    view = _StateView()
    assert w(fake, null, null) == 1 and w(null, ctypes.addressof(view), null) == 1
    assert w(vp(0x10010), ctypes.addressof(view), null) == 2
    for field, i, bad in (("ring", 0, -1.0), ("ring", 5, float("nan")), ("ring", 15, float("inf")),
                          ("static_values", 0, -0.5), ("descale_used", 1, -2.0), ("amax_last", 2, float("inf"))):
        arr = getattr(view, field) if field != "ring" else view.ring[2]
        arr[i] = bad
        assert w(fake, ctypes.addressof(view), null) == 1, (field, i)
        arr[i] = 0.0
    view.flags = 2                      # not an FP8VIT_FLAG_* bit
    assert w(fake, ctypes.addressof(view), null) == 1
    view.flags = 0
    sf = lib.fp8vit_state_set_flags
    sf.argtypes = [vp, ctypes.c_uint32, vp]
    assert sf(null, 1, null) == 1 and sf(fake, 2, null) == 1 and sf(fake, 0xffffffff, null) == 1
    assert sf(vp(0x10010), 1, null) == 2
    cc = lib.fp8vit_check_cu_seqlens
    cc.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
    assert cc(null, 1, 10, 10, fake, null) == 1 and cc(fake, 1, 10, 10, null, null) == 1
    assert cc(fake, -1, 10, 10, fake, null) == 1 and cc(fake, 1, -1, 10, fake, null) == 1
    assert cc(fake, 1, 10, -1, fake, null) == 1
    assert cc(fake, 1, 10, 10, vp(0x10010), null) == 2 and cc(vp(0x10002), 1, 10, 10, fake, null) == 2


def test_state_view_layout():
    """The binding's view structure has the C layout the header gives (natural
    alignment: the 64-bit counts start at byte 240)."""
    from fp8_quantized_varlen_amd import _StateView
    off = {name: getattr(_StateView, name).offset for name, _ in _StateView._fields_}
    assert off == {"ring": 0, "count": 192, "static_values": 196, "descale_used": 208, "amax_last": 220,
                   "flags": 232, "cu_check": 236, "saturated": 240}
    assert ctypes.sizeof(_StateView) == 264


def load(lib, path, layer):
    f = lib.fp8vit_load_static_scales
    f.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(ctypes.c_float)]
    out = (ctypes.c_float * 3)(-1.0, -1.0, -1.0)
    st = f(os.fsencode(path), layer.encode("utf-8"), out)
    return st, tuple(out)


def test_loader_printed_example_and_aliases(lib, golden_dir):
    for fn in ("scales_example.json", "scales_aliases.json"):
        p = os.path.join(golden_dir, fn)
        assert load(lib, p, "visual.blocks.0.attn.attn") == (0, (224.0, 198.0, 210.0))
        assert load(lib, p, "visual.blocks.1.attn.attn") == (0, (218.0, 195.0, 207.0))
        assert load(lib, p, "visual.blocks.2.attn.attn")[0] == 6


def test_loader_matches_python_json_on_float32_roundtrip(lib, tmp_path):
    rng = np.random.default_rng(0)
    vals = (rng.uniform(1, 2, (40, 3)) * np.exp2(rng.integers(-30, 30, (40, 3)))).astype(np.float32)
    doc = {f"visual.blocks.{i}.attn.attn": {"q": float(v[0]), "k_scale": float(v[1]), "v": float(v[2]), "extra": [1, {}]}
           for i, v in enumerate(vals)}
    p = tmp_path / "s.json"
    p.write_text(json.dumps(doc, indent=1))
    for i, v in enumerate(vals):
        st, got = load(lib, str(p), f"visual.blocks.{i}.attn.attn")
        assert st == 0 and np.array_equal(np.float32(got), v)


@pytest.mark.parametrize("text,layer,status", [
    ('{"a": {"q": 1, "k": 2, "v": 3}}', "a", 0),
    ('{"a": {"q": 1e2, "k": 2.5E-3, "v": 3}}', "a", 0),
    ('  {"a" : {"q":1,"k":2,"v":3} , "b": null}\n', "a", 0),
    ('{"a": {"q": 1, "k": 2}}', "a", 6),
    ('{"a": {"q": 1, "q_scale": 1, "k": 2, "v": 3}}', "a", 1),
    ('{"a": {"q": 0, "k": 2, "v": 3}}', "a", 1),
    ('{"a": {"q": -1, "k": 2, "v": 3}}', "a", 1),
    ('{"a": {"q": "1", "k": 2, "v": 3}}', "a", 1),
    ('{"a": {"q": 1e39, "k": 2, "v": 3}}', "a", 1),
    ('{"a": {"q": 1, "k": 2, "v": 3}', "a", 5),
    ('{"a": {"q": 1, "k": 2, "v": 3}} x', "a", 5),
    ('{"a": [1, 2, 3]}', "a", 5),
    ('[1]', "a", 5),
    ('{"a": {"q": 01, "k": 2, "v": 3}}', "a", 5),
    ('{"a": {"q": NaN, "k": 2, "v": 3}}', "a", 5),
    ('{"a": {"q": 1, "k": 2, "v": 3}, "a": {"q": 4, "k": 5, "v": 6}}', "a", 0),
    ('{"caf\\u00e9.blocks.0": {"q": 1, "k": 2, "v": 3}}', "café.blocks.0", 0),
    ('{"x\\"y\\\\z": {"q": 1, "k": 2, "v": 3}}', 'x"y\\z', 0),
    ('', "a", 5),
])
def test_loader_cases(lib, tmp_path, text, layer, status):
    p = tmp_path / "s.json"
    p.write_text(text, encoding="utf-8")
    st, vals = load(lib, str(p), layer)
    assert st == status, (text, st)
    if status == 0 and text.count('"a"') == 2:
        assert vals == (4.0, 5.0, 6.0)          # last occurrence wins, as in Python's json
    if status == 0:
        ref = json.loads(text)[layer]
        assert vals == tuple(float(np.float32(ref.get(k, ref.get(k + "_scale")))) for k in "qkv")


def test_loader_io_errors(lib, tmp_path):
    assert load(lib, str(tmp_path / "missing.json"), "a")[0] == 4
    assert load(lib, str(tmp_path), "a")[0] in (4, 5)
