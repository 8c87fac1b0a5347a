"""The compact FP6 operand layout of the int4 codes, written independently of
the library from its description in include/ck4.h, for the tests.

Same blocks and lane images as the FP6 layout (tests/fp6_layout.py) with 16
bytes per lane image instead of 24: every 12-byte run of the FP6 buffer (the
96-bit image W of 16 codes, dwords V0, V1, V2 little-endian) becomes the 8
bytes D0 = V0 | (V1 & Z0), D1 = V2 | (V1 & Z2) with Z0 = 0x18618618 and
Z2 = 0x61861861, and the inverse is V0 = D0 & ~Z0, V2 = D1 & ~Z2,
V1 = (D0 & Z0) | (D1 & Z2). The runs keep their order, so block (r // 16,
k // 128) is 1024 bytes at ((r // 16) * (k // 128) + k // 128) * 1024.
"""
import numpy as np

import fp6_layout

Z0 = np.uint32(0x18618618)
Z2 = np.uint32(0x61861861)


def nbytes(rows: int, k: int) -> int:
    return (rows + 15) // 16 * 16 * k // 2


def compress(fp6_buf: np.ndarray) -> np.ndarray:
    """FP6 layout bytes -> compact layout bytes; raises if an image does not fit (a nonzero exponent bit)."""
    v = np.ascontiguousarray(fp6_buf, np.uint8).reshape(-1, 12).view("<u4")   # [runs, 3]
    v0, v1, v2 = v[:, 0], v[:, 1], v[:, 2]
    if np.any(v0 & Z0) or np.any(v2 & Z2) or np.any(v1 & ~(Z0 | Z2)):
        raise AssertionError("FP6 image with a nonzero exponent bit")
    d = np.stack([v0 | (v1 & Z0), v2 | (v1 & Z2)], axis=1).astype("<u4")
    return d.view(np.uint8).reshape(-1)


def expand(buf: np.ndarray) -> np.ndarray:
    """Compact layout bytes -> FP6 layout bytes."""
    d = np.ascontiguousarray(buf, np.uint8).reshape(-1, 8).view("<u4")       # [runs, 2]
    d0, d1 = d[:, 0], d[:, 1]
    v = np.stack([d0 & ~Z0, (d0 & Z0) | (d1 & Z2), d1 & ~Z2], axis=1).astype("<u4")
    return v.view(np.uint8).reshape(-1)


def encode(q: np.ndarray) -> np.ndarray:
    """int codes [rows, k] (|q| <= 7) -> the compact uint8 buffer, padding rows zero."""
    return compress(fp6_layout.encode(q))


def decode(buf: np.ndarray, rows: int, k: int) -> np.ndarray:
    """compact uint8 buffer -> int codes [rows, k]."""
    b = np.ascontiguousarray(buf, np.uint8).reshape(-1)
    assert b.size >= nbytes(rows, k)
    return fp6_layout.decode(expand(b[: nbytes(rows, k)]), rows, k)
