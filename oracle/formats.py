"""Storage-format decoders of the oracle (test infrastructure, not product code).

Both decoders are written from the format definitions, not from a library cast:

* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits; exponent field 0 encodes subnormals m/8 * 2^-6; there are no infinities
  and S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
  The pages name the indexer's precision only as "FP8" (MarkTechPost, "DeepSeek
  V3.2-Exp Cuts Long-Context Costs with DeepSeek Sparse Attention (DSA) While
  Maintaining Benchmark Parity", the two-tier pipeline, whose first tier is an FP8
  indexer); the e4m3fn variant is this library's
  reading (the format gfx950 computes in).
* bfloat16: the top 16 bits of an IEEE-754 binary32.
"""
from __future__ import annotations

import numpy as np


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
