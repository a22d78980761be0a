"""Write descale_examples.txt: fp32 bits of RN_fp32(value / 448) for the printed
example values, using exact rational arithmetic (fractions) -- independent of
both the oracle and the GPU path."""
import os
import struct
from fractions import Fraction


def rn_fp32(x: Fraction) -> int:
    """Round a positive rational to the nearest fp32 (ties to even); return bits."""
    assert x > 0
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    assert -126 <= e <= 127
    m = x / Fraction(2) ** e * (1 << 23)       # in [2^23, 2^24)
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == (1 << 24):
        lo >>= 1
        e += 1
    return ((e + 127) << 23) | (lo - (1 << 23))


if __name__ == "__main__":
    vals = [224.0, 198.0, 210.0, 218.0, 195.0, 207.0]
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "descale_examples.txt"), "w") as f:
        f.write("# value  descale_fp32_bits_hex  descale_value\n")
        for v in vals:
            b = rn_fp32(Fraction(v) / 448)
            f.write(f"{v} 0x{b:08x} {struct.unpack('<f', struct.pack('<I', b))[0]!r}\n")
