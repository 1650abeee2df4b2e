"""The row kernels' tanh table (csrc/dit_tanh_table.hpp) is what its generator
writes, and every entry equals the oracle's correctly rounded bf16 tanh.

The two sides compute tanh independently: the generator in 80-digit decimal
arithmetic, the oracle in C from the binary64 tanh rounded once to bf16
(itself pinned against long double on all 65536 inputs).
The device lookup around the table (identity below 2^-4, +-1 from 3.5, NaN)
is checked over all 65536 inputs by the GPU primitive tests."""
import os
import re
import sys

import numpy as np

import oracle

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "modulation_bf16_row_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_tanh_table as gen  # noqa: E402


def _committed_codes():
    with open(os.path.join(CSRC, "dit_tanh_table.hpp")) as f:
        text = f.read()
    body = text[text.index("kTanhTabGlobal"):]
    return [int(h, 16) for h in re.findall(r"0x([0-9A-F]{4})", body[body.index("{"):])]


def test_header_is_the_generator_output():
    with open(os.path.join(CSRC, "dit_tanh_table.hpp")) as f:
        assert f.read() == gen.header_text(gen.table())


def test_table_equals_oracle_tanh():
    codes = np.arange(gen.LO, gen.HI, dtype=np.uint16)
    tab = np.array(_committed_codes(), dtype=np.uint16)
    assert len(tab) == len(codes) == 736
    assert np.array_equal(tab, oracle.tanh_bf16(codes))


def test_table_ends_and_monotonicity():
    tab = np.array(_committed_codes(), dtype=np.int64)
    assert np.all(np.diff(tab) >= 0)                 # tanh is increasing on the span
    assert tab[-1] == 0x3F80                         # tanh(3.48..) rounds to 1
    assert tab[0] == 0x3D80                          # tanh(1/16) rounds back to 1/16
