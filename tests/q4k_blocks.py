"""Hand-built Q4_K blocks for the tests, written byte by byte.

Nothing here calls the oracle or the HIP library.  Each helper writes raw
bytes; the expected weights of each case are stated in closed form by the
test that uses it.
"""
from __future__ import annotations

import numpy as np

F16_ONE = 0x3C00      # 1.0
F16_HALF = 0x3800     # 0.5
F16_TWO = 0x4000      # 2.0
F16_NEG_ONE = 0xBC00  # -1.0


def block(d_bits: int = 0, dmin_bits: int = 0, S=None, Q=None) -> np.ndarray:
    """One 144-byte block from raw fp16 bit patterns, 12 scale bytes and 128 quant bytes."""
    b = np.zeros(144, dtype=np.uint8)
    b[0] = d_bits & 0xFF
    b[1] = d_bits >> 8
    b[2] = dmin_bits & 0xFF
    b[3] = dmin_bits >> 8
    if S is not None:
        b[4:16] = np.asarray(S, dtype=np.uint8)
    if Q is not None:
        b[16:144] = np.asarray(Q, dtype=np.uint8)
    return b


# Scale bytes giving sc_j = 1 for all eight sub-blocks and every min 0:
# S[0..3] = 1 (sc_0..3), S[4..7] = 0 (m_0..3), S[8..11] low nibble 1 (sc_4..7),
# high nibble 0 (m_4..7); the high two bits of every field are 0.
S_UNIT_SCALES = [1, 1, 1, 1, 0, 0, 0, 0, 0x01, 0x01, 0x01, 0x01]


def unit_block() -> np.ndarray:
    """d = 1, dmin = 0, every scale 1, every quant 1: all 256 weights are 1.0."""
    return block(F16_ONE, 0, S_UNIT_SCALES, [0x11] * 128)


def unit_matrix(rows: int, cols: int) -> np.ndarray:
    """A Q4_K matrix whose every weight is exactly 1.0."""
    return np.tile(unit_block(), (rows, cols // 256, 1)).reshape(rows, cols // 256, 144)


def scaled_blob(blob: np.ndarray, factor_bits_fn) -> np.ndarray:
    """Copy of ``blob`` with d and dmin replaced through ``factor_bits_fn(uint16 array)``."""
    out = blob.copy()
    for off in (0, 2):
        bits = out[..., off].astype(np.uint16) | (out[..., off + 1].astype(np.uint16) << 8)
        nb = factor_bits_fn(bits)
        out[..., off] = (nb & 0xFF).astype(np.uint8)
        out[..., off + 1] = (nb >> 8).astype(np.uint8)
    return out


def double_fp16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact doubling of normal, finite, non-zero fp16 values: exponent field + 1."""
    bits = bits.astype(np.uint16)
    exp = (bits >> 10) & 0x1F
    assert np.all((exp > 0) & (exp < 30)), "only normal values well below overflow"
    return bits + np.uint16(1 << 10)
