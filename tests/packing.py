"""Code-to-byte packer for tests (test helper, not used by either side's arithmetic).

Packs signed integer values into the stored formats so that the same matrix
can be presented as f32, int8, int4 and int2:

  int8: two's-complement byte;
  int4: byte j = (v[2j] + 8) | (v[2j+1] + 8) << 4   (even element in the low nibble);
  int2: byte j = sum_k (v[4j+k] + 2) << 2k          (element 4j+k in bits 2k..2k+1);
  f32 : little-endian IEEE single of the value.

Rows are padded to whole bytes with the pad value given (default 0 bits).
The packing rule is pinned by tests/golden/dequant_table.txt.
"""
from __future__ import annotations

import numpy as np

F32, I8, I4, I2 = 0, 1, 2, 3


def pack(fmt: int, vals: np.ndarray, pad_bits: int = 0) -> np.ndarray:
    vals = np.asarray(vals)
    O, I = vals.shape
    if fmt == F32:
        return vals.astype(np.float32).view(np.uint8).reshape(O, 4 * I).copy()
    v = vals.astype(np.int64)
    if fmt == I8:
        assert v.min() >= -128 and v.max() <= 127
        return (v & 0xFF).astype(np.uint8)
    if fmt == I4:
        assert v.min() >= -8 and v.max() <= 7
        per, off, b = 2, 8, 4
    elif fmt == I2:
        assert v.min() >= -2 and v.max() <= 1
        per, off, b = 4, 2, 2
    else:
        raise ValueError(fmt)
    rb = (I + per - 1) // per
    out = np.zeros((O, rb), dtype=np.int64)
    for i in range(rb * per):
        if i < I:
            c = v[:, i] + off
        else:
            c = np.full(O, pad_bits & ((1 << b) - 1), dtype=np.int64)
        out[:, i // per] |= c << (b * (i % per))
    return out.astype(np.uint8)
