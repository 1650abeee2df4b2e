"""Writes dit_tanh_table.hpp: the correctly rounded bf16 tanh of every bf16
magnitude g with code 0x3D80 .. 0x405F (2^-4 <= g < 3.5), the span where the
row kernels look tanh(gate) up instead of returning g or +-1.

tanh(g) = (e^{2g} - 1) / (e^{2g} + 1) is evaluated with Python's decimal
module at 80 significant digits from the exact value of g (a bf16 number is
a short binary fraction, so it converts to decimal exactly).  The quotient by
the bf16 spacing of its binade is then rounded half-to-even to an integer.
tanh of a nonzero rational is irrational, so the exact value is never a
rounding midpoint; the script asserts that the 80-digit value lies farther
than 10^-40 spacings from one, far more than its own error.

    python -m modulation_bf16_row_amd.csrc.gen_tanh_table   (or run the file)
"""
import os
import struct
from decimal import ROUND_HALF_EVEN, Decimal, localcontext

LO, HI = 0x3D80, 0x4060                 # bf16 codes of the table's magnitudes
HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "dit_tanh_table.hpp")


def bf16_value(code):
    return struct.unpack("<f", struct.pack("<I", code << 16))[0]


def tanh_bf16_code(code):
    """bf16 code of the correctly rounded tanh of the bf16 number `code`."""
    g = bf16_value(code)
    with localcontext() as ctx:
        ctx.prec = 80
        e2 = (2 * Decimal(g)).exp()
        t = (e2 - 1) / (e2 + 1)                    # 0 < t < 1
        # binade: 2^k <= t < 2^(k+1), k < 0
        k = -1
        while t < Decimal(2) ** k:
            k -= 1
        spacing = Decimal(2) ** (k - 7)          # 8 significant bits
        q = t / spacing                          # 128 <= q < 256
        frac = q - int(q)
        assert abs(frac - Decimal("0.5")) > Decimal("1e-40"), hex(code)
        n = int(q.to_integral_value(rounding=ROUND_HALF_EVEN))
    value = n * 2.0 ** (k - 7)                   # exact: n <= 256
    bits = struct.unpack("<I", struct.pack("<f", value))[0]
    assert bits & 0xFFFF == 0
    return bits >> 16


def table():
    return [tanh_bf16_code(c) for c in range(LO, HI)]


def header_text(codes):
    rows = []
    for i in range(0, len(codes), 12):
        rows.append("    " + ", ".join("0x%04X" % c for c in codes[i:i + 12]) + ",")
    return (
        "// dit_tanh_table.hpp -- written by gen_tanh_table.py; do not edit.\n"
        "// Correctly rounded bf16 tanh(g) of the bf16 magnitudes g with codes\n"
        "// 0x%04X .. 0x%04X (2^-4 <= g < 3.5), as bf16 codes; entry i is g = code\n"
        "// 0x%04X + i.  The row kernels copy it into LDS.\n"
        "#pragma once\n\n"
        "#include <stdint.h>\n\n"
        "namespace dit {\n\n"
        "constexpr int kTanhTabEntries = %d;\n\n"
        "__device__ __attribute__((aligned(16))) const uint16_t kTanhTabGlobal[%d] = {\n"
        "%s\n"
        "};\n\n"
        "}  // namespace dit\n" % (LO, HI - 1, LO, len(codes), len(codes), "\n".join(rows)))


def main():
    with open(OUT, "w") as f:
        f.write(header_text(table()))
    print(OUT)


if __name__ == "__main__":
    main()
