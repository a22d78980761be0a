"""The JSON scale-file reader and writer under AddressSanitizer and UBSan.

`fp8_quantized_varlen_amd/csrc/json_scales.cpp` is host code; here it is built
with g++ (no GPU pass) together with `tests/host/json_scales_harness.cpp` and
driven with a corpus of valid, truncated, mutated and adversarial files. The
run must finish without a sanitizer report or a leak, every call must return a
defined status code, and the well-formed files must read back as written.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "fp8_quantized_varlen_amd", "csrc", "json_scales.cpp")
HARNESS = os.path.join(HERE, "host", "json_scales_harness.cpp")
GOLDEN = os.path.join(HERE, "golden", "scales_example.json")
STATUSES = {0, 1, 2, 4, 5, 6}   # OK, INVALID_ARGUMENT, UNSUPPORTED, IO, PARSE, NOT_FOUND


def _adversarial():
    big_digits = "1" + "0" * 5000
    cases = {
        "empty": b"",
        "ws": b" \n\t\r ",
        "bom_only": b"\xef\xbb\xbf",
        "bom_valid": b'\xef\xbb\xbf{"visual.blocks.0.attn.attn": {"q": 1, "k": 2, "v": 3}}',
        "deep_array": b"[" * 100000,
        "deep_object": b'{"a":' * 100000,
        "depth_64": b"[" * 64 + b"]" * 64,
        "depth_65": b"[" * 65 + b"]" * 65,
        "long_string": b'{"' + b"a" * (1 << 20) + b'": 1}',
        "unterminated": b'{"visual.blocks.0.attn.attn": {"q": 1, "k',
        "bad_escape": b'{"a\\x": 1}',
        "short_u": b'{"\\u12": 1}',
        "lone_high": b'{"\\ud800": 1}',
        "lone_low": b'{"\\udc00": 1}',
        "pair": b'{"\\ud83d\\ude00": 1}',
        "high_then_bad": b'{"\\ud800\\u0041": 1}',
        "nul_in_string": b'{"a\x00b": 1}',
        "control_char": b'{"a\x01": 1}',
        "invalid_utf8": b'{"\xff\xfe": 1}',
        "huge_exp": b'{"visual.blocks.0.attn.attn": {"q": 1e999, "k": 2, "v": 3}}',
        "tiny_exp": b'{"visual.blocks.0.attn.attn": {"q": 1e-999, "k": 2, "v": 3}}',
        "neg_zero": b'{"visual.blocks.0.attn.attn": {"q": -0, "k": 2, "v": 3}}',
        "leading_zero": b'{"visual.blocks.0.attn.attn": {"q": 01, "k": 2, "v": 3}}',
        "dot_only": b'{"visual.blocks.0.attn.attn": {"q": 1., "k": .5, "v": 3}}',
        "plus": b'{"visual.blocks.0.attn.attn": {"q": +1, "k": 2, "v": 3}}',
        "nan_inf": b'{"visual.blocks.0.attn.attn": {"q": NaN, "k": Infinity, "v": 3}}',
        "many_digits": ('{"visual.blocks.0.attn.attn": {"q": %s, "k": 2, "v": 3}}' % big_digits).encode(),
        "many_keys": ("{" + ",".join('"k%d": {"q": 1}' % i for i in range(20000)) + "}").encode(),
        "dup_layer": b'{"visual.blocks.0.attn.attn": {"q": 1, "k": 2, "v": 3}, '
                     b'"visual.blocks.0.attn.attn": {"q": 4, "k": 5, "v": 6}}',
        "alias_and_key": b'{"visual.blocks.0.attn.attn": {"q": 1, "q_scale": 1, "k": 2, "v": 3}}',
        "root_array": b"[1, 2, 3]",
        "root_number": b"42",
        "root_string": b'"x"',
        "trailing": b'{"visual.blocks.0.attn.attn": {"q": 1, "k": 2, "v": 3}} x',
        "literals": b'{"visual.blocks.0.attn.attn": {"q": true, "k": false, "v": null}}',
    }
    return cases


def _corpus(tmp_path):
    golden = open(GOLDEN, "rb").read()
    files = {}
    files["golden.json"] = golden
    for n in range(len(golden)):
        files["trunc_%04d.json" % n] = golden[:n]
    rng = np.random.Generator(np.random.PCG64(2024))
    for n in range(400):
        b = bytearray(golden)
        for _ in range(int(rng.integers(1, 6))):
            op = int(rng.integers(0, 3))
            pos = int(rng.integers(0, len(b) + 1))
            if op == 0 and len(b):
                b[min(pos, len(b) - 1)] = int(rng.integers(0, 256))
            elif op == 1:
                b[pos:pos] = bytes([int(x) for x in rng.integers(0, 256, size=int(rng.integers(1, 4)))])
            elif len(b):
                del b[pos:pos + int(rng.integers(1, 4))]
        files["mut_%03d.json" % n] = bytes(b)
    for name, data in _adversarial().items():
        files["adv_%s.json" % name] = data
    paths = []
    for name, data in files.items():
        p = tmp_path / name
        p.write_bytes(data)
        paths.append(str(p))
    return paths


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_json_reader_and_writer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "json_harness")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"), SRC, HARNESS, "-o", exe],
        capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    corpus_dir = tmp_path / "corpus"
    corpus_dir.mkdir()
    paths = _corpus(corpus_dir)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98")
    lines = []
    for i in range(0, len(paths), 200):
        r = subprocess.run([exe] + paths[i:i + 200], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, (r.returncode, r.stderr[-3000:])
        assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
        lines += r.stdout.splitlines()
    assert len(lines) == len(paths)
    status = {}
    for ln in lines:
        parts = ln.split()
        codes = [int(x) for x in parts[1:5]]
        assert len(codes) == 4 and set(codes) <= STATUSES, ln
        status[os.path.basename(parts[0])] = codes
        if codes[2] == 0:   # written: the values read back exactly
            assert codes[3] == 0 and [float(x) for x in parts[5:8]] == [1.5, 2.25, 3.0], ln
    # the printed example (two layers) reads, takes the write and reads it back
    assert status["golden.json"] == [0, 0, 0, 0]
    assert status["adv_bom_valid.json"][0] == 0
    # a file that is not a JSON object is never overwritten; an empty (or
    # whitespace-only) file counts as an empty object and takes the entry
    for name in ("adv_root_array.json", "adv_root_number.json", "adv_deep_array.json", "adv_trailing.json"):
        assert status[name][2] != 0, (name, status[name])
    for name in ("adv_empty.json", "adv_ws.json", "adv_bom_only.json"):
        assert status[name][2:] == [0, 0], (name, status[name])
    for name in ("adv_deep_array.json", "adv_deep_object.json", "adv_depth_65.json", "adv_huge_exp.json",
                 "adv_nan_inf.json", "adv_lone_high.json", "adv_lone_low.json", "adv_bad_escape.json"):
        assert status[name][0] != 0, (name, status[name])
