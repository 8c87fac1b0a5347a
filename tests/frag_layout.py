"""MFMA fragment order of a bf16 matrix, as include/ck4.h documents it for the
LoRA operands (test-side implementation, used to pack inputs and unpack
outputs of the LoRA calls).

A matrix Z [rows, cols] (cols a multiple of 32) is stored as 16-row x 32-column
tiles of 512 values with its rows rounded up to a multiple of 16: tile
(r // 16, c // 32) at element offset ((r // 16) * (cols // 32) + c // 32) * 512,
element (i, c) of a tile at (16 * ((c >> 2) & 3) + i) * 8 + 4 * (c >> 4) + (c & 3).
"""
import numpy as np


def rows16(n: int) -> int:
    return (n + 15) // 16 * 16


def offsets(r16: int, cols: int) -> np.ndarray:
    r = np.arange(r16)[:, None]
    c = np.arange(cols)[None, :]
    return (((r >> 4) * (cols // 32) + (c >> 5)) * 512 + (16 * ((c >> 2) & 3) + (r & 15)) * 8
            + 4 * ((c >> 4) & 1) + (c & 3))


def pack(z: np.ndarray) -> np.ndarray:
    """uint16 [rows, cols] -> uint16 [rows16, cols] in fragment order, zero padding rows."""
    rows, cols = z.shape
    r16 = rows16(rows)
    zp = np.zeros((r16, cols), z.dtype)
    zp[:rows] = z
    out = np.empty(r16 * cols, z.dtype)
    out[offsets(r16, cols)] = zp
    return out.reshape(r16, cols)


def unpack(p: np.ndarray, rows: int) -> np.ndarray:
    """Fragment order [rows16, cols] -> the first `rows` rows of the matrix."""
    r16, cols = p.shape
    return np.ascontiguousarray(p.reshape(-1)[offsets(r16, cols)][:rows])
