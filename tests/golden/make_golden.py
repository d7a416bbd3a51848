"""Writes the stored expected values under tests/golden/.

Only closed forms are used here (exact rationals and one IEEE f32 division);
nothing from the HIP library is called. Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def pages_pattern():
    # Activation of the grouped-kernel bit gate, section 25.7.1 of
    # "25 — Writing XPU Kernels": x_j = ((j mod 25) - 12) / 64.
    # amax = 12/64 = 0.1875, so the block scale is the f32 quotient 0.1875/127
    # and the exact code of k = (j mod 25) - 12 is k*127/12 rounded to nearest
    # (k = +-6 is the tie +-63.5; both tie rules give +-64).
    scale = np.float32(0.1875) / np.float32(127.0)
    bits = int(np.array(scale).view(np.uint32))
    codes = [round(Fraction(k * 127, 12)) for k in range(-12, 13)]
    with open(os.path.join(HERE, "pages_pattern_q8k.txt"), "w") as f:
        f.write("# q8_K encoding of x_j = ((j mod 25) - 12)/64 (\"25 — Writing XPU Kernels\",\n")
        f.write("# section 25.7.1, the bit gate's activation). Every 256-block holds all 25\n")
        f.write("# residues, so every block has amax = 12/64 and the same scale.\n")
        f.write("# scale_bits: f32 bits of the block scale 0.1875/127.\n")
        f.write("# codes_k_minus12_to_12: code of an element with k = (j mod 25) - 12,\n")
        f.write("# k = -12..12: round(k*127/12), exact rational, ties to even.\n")
        f.write("# Written by tests/golden/make_golden.py.\n")
        f.write("scale_bits = %08x\n" % bits)
        f.write("codes_k_minus12_to_12 = %s\n" % ",".join(str(c) for c in codes))


def codebook():
    kv = [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]
    with open(os.path.join(HERE, "iq4nl_codebook.txt"), "w") as f:
        f.write("# The 16 signed int8 values of the IQ4_NL codebook, nibble 0..15.\n")
        f.write("# \"25 — Writing XPU Kernels\", section 25.2.1, names the table (the\n")
        f.write("# codebook accessor) without printing it; these are the published IQ4_NL\n")
        f.write("# values that the codebook workload specifies.\n")
        f.write(",".join(str(v) for v in kv) + "\n")


if __name__ == "__main__":
    pages_pattern()
    codebook()
