"""Writes mxfp4_half_lut.txt: the SHA-256 of the oracle's 256 x 16 binary16
table (little-endian uint16, row e, column code) and a few of its entries.
Calls only the oracle.  Run from the repository root:
    python tests/golden/make_mxfp4_half_lut.py
"""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402

lut = oracle.mxfp4_half_lut()
sha = hashlib.sha256(lut.astype("<u2").tobytes()).hexdigest()
lines = [
    "# MXFP4 -> binary16 table: entry [e][c] = E2M1(c) * 2^(e - 127) rounded once to",
    "# nearest-even (ds4.c study notes, glossary page \"quantization\", section",
    "# \"Metal's MXFP4 -> half lookup table\": 256 x 16 exact products, pinned by a",
    "# SHA-256 of the generated table).  Row 255 (infinite scale) holds 0x7E00.",
    "# Written by tests/golden/make_mxfp4_half_lut.py from the oracle.",
    f"sha256 {sha}",
]
for e, c in ((127, 7), (127, 1), (127, 9), (112, 1), (103, 1), (102, 1), (142, 7), (143, 6), (0, 1), (255, 0)):
    lines.append(f"entry {e} {c} 0x{int(lut[e, c]):04x}")
open(os.path.join(HERE, "mxfp4_half_lut.txt"), "w").write("\n".join(lines) + "\n")
print(sha)
