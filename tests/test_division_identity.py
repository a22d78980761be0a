"""The quantizer forms the fp32 quotient x / descale as RN32(x * RN64(1/descale))
(one fp64 multiply instead of a correctly rounded fp32 division). Check on the
host, with numpy's IEEE arithmetic, that this equals the IEEE fp32 division for
every finite bf16 x and thousands of unrelated fp32 descales."""
import numpy as np

from synth import bf16_bits_to_f32

ALL = bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
FINITE = ALL[np.isfinite(ALL)]


def _descales(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    # random 24-bit mantissas over the whole useful exponent range, including
    # the 1e-10 floor region and values whose quotients overflow
    d = (2.0 ** rng.uniform(-40, 40, n)).astype(np.float32)
    d = np.concatenate([d, np.float32([1e-10, 1.0, 448.0, 0.5, 3.0, 1.0 / 3.0, 2.0 ** -126, 3.0e38])])
    return d[d > 0]


def test_rn64_reciprocal_product_equals_fp32_division():
    x32 = FINITE.astype(np.float32)
    x64 = x32.astype(np.float64)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        for d in _descales(3000, 11):
            want = x32 / np.float32(d)
            r = np.float64(1.0) / np.float64(d)
            got = (x64 * r).astype(np.float32)
            assert np.array_equal(want.view(np.uint32), got.view(np.uint32)), float(d)
