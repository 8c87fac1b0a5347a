"""The FP6 operand layout of the int4 codes, written independently of the
library from its description in include/ck4.h, for the tests.

rows padded to 16, k a multiple of 128; block (r // 16, k // 128) is 1536
bytes at ((r // 16) * (k_total // 128) + k // 128) * 1536; row i = r % 16 and
k group g = (k % 128) // 32 own the 24 bytes at 24 * (16 g + i), with the
6-bit code of t = k % 32 at bits 6 t (LSB first). The code of q is the FP6
E2M3 value q / 8: sign bit 5, |q| in bits 0-2, bits 3-4 zero.
"""
import numpy as np


def _positions(rows: int, k: int):
    """Bit offset of every (r, kk) code in the buffer, int64 [rows, k]."""
    r = np.arange(rows)[:, None]
    kk = np.arange(k)[None, :]
    block = (r // 16) * (k // 128) + kk // 128
    g = (kk % 128) // 32
    img = block * 1536 + (16 * g + r % 16) * 24
    return img * 8 + 6 * (kk % 32)


def nbytes(rows: int, k: int) -> int:
    return (rows + 15) // 16 * 16 * k * 3 // 4


def decode(buf: np.ndarray, rows: int, k: int) -> np.ndarray:
    """uint8 buffer -> int codes [rows, k]; raises if a code is not q / 8 with |q| <= 7."""
    b = np.ascontiguousarray(buf, np.uint8).reshape(-1)
    assert b.size >= nbytes(rows, k)
    pos = _positions(rows, k)
    byte, sh = pos // 8, pos % 8
    lo = b[byte].astype(np.int64)
    hi = b[np.minimum(byte + 1, b.size - 1)].astype(np.int64)
    code = ((lo | (hi << 8)) >> sh) & 0x3F
    if np.any(code & 0x18):
        raise AssertionError("FP6 code with a nonzero exponent field")
    mag = code & 7
    return np.where(code & 0x20, -mag, mag)


def encode(q: np.ndarray) -> np.ndarray:
    """int codes [rows, k] (|q| <= 7) -> the uint8 buffer, padding rows zero."""
    q = np.asarray(q, np.int64)
    rows, k = q.shape
    code = np.where(q < 0, 0x20 | -q, q)
    bits = np.zeros(nbytes(rows, k) * 8, np.uint8)
    pos = _positions(rows, k)
    for t in range(6):
        bits[(pos + t).ravel()] = ((code >> t) & 1).ravel()
    return np.packbits(bits.reshape(-1, 8), axis=1, bitorder="little").ravel()
