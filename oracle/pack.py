"""Integer-code packing.  TEST INFRASTRUCTURE ONLY.

The ADMM-Q page (experiments, 3. inference) says the quantizer's output keeps the
GPTQ storage format, and the GPTQ tutorial page (section 3, the output of
Algorithm 1) says the output is the codes plus the scale information needed to
decode them; neither gives the bit layout.  Reading used here: each row is one
little-endian bitstream of 32-bit words; code i of the row occupies bits
[i*b, (i+1)*b), least significant bit first, so a code may straddle two words;
each row is padded with zero bits to ceil(cols * b / 32) words.

Written as a plain per-bit loop so that it can be read against the definition.
"""
from __future__ import annotations

import numpy as np


def words_per_row(cols: int, bits: int) -> int:
    return (cols * bits + 31) // 32


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.asarray(codes)
    rows, cols = codes.shape
    assert 1 <= bits <= 8 and int(codes.max(initial=0)) < (1 << bits)
    out = np.zeros((rows, words_per_row(cols, bits)), dtype=np.uint32)
    for r in range(rows):
        acc = [0] * out.shape[1]
        for i in range(cols):
            c = int(codes[r, i])
            for k in range(bits):
                if (c >> k) & 1:
                    pos = i * bits + k
                    acc[pos // 32] |= 1 << (pos % 32)
        out[r] = np.array(acc, dtype=np.uint64).astype(np.uint32)
    return out


def unpack(words: np.ndarray, cols: int, bits: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    rows = words.shape[0]
    out = np.zeros((rows, cols), dtype=np.uint8)
    for r in range(rows):
        w = [int(x) for x in words[r]]
        for i in range(cols):
            c = 0
            for k in range(bits):
                pos = i * bits + k
                c |= ((w[pos // 32] >> (pos % 32)) & 1) << k
            out[r, i] = c
    return out
