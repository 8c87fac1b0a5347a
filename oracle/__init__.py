"""CPU oracle for the W4A4 ConvRot linear -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The product library (``int4_w4a4_quantized_amd``) never
does: the two share no code, and the product fails loudly without its HIP
extension instead of falling back here.

Every function is a thin numpy/ctypes shim over ``ck4_oracle.c``, which states
the method step by step with citations to the pages it follows. All inputs
and outputs are host numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ck4_oracle.c")
_LIB = os.path.join(_HERE, "libck4_oracle.so")
CFLAGS = ["-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (in-tree). Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        sig = {
            "ck4o_num_threads": ([], I),
            "ck4o_set_num_threads": ([I], None),
            "ck4o_hadamard_scale_f32": ([I], ctypes.c_float),
            "ck4o_fwht_f32": ([P, I], None),
            "ck4o_fwht_f64": ([P, I], None),
            "ck4o_rotate_rows_f32": ([P, I64, I64, I64, I, P], None),
            "ck4o_rotate_rows_bf16": ([P, I64, I64, I64, I, P], None),
            "ck4o_rotate_rows_f64": ([P, I64, I64, I, P], None),
            "ck4o_quantize_rows": ([P, I64, I64, I, I, P, P], None),
            "ck4o_quantize_rows_sr": ([P, P, I64, I64, I64, I, I, P, P], None),
            "ck4o_e4m3_decode": ([ctypes.c_uint8], ctypes.c_float),
            "ck4o_e4m3_encode": ([ctypes.c_float], ctypes.c_uint8),
            "ck4o_quantize_weight_convrot_e4m3": ([P, I64, I64, I64, I, I, P, P], None),
            "ck4o_quantize_weight_convrot_sr": ([P, I64, I64, I64, I, I, P, I64, P, P], None),
            "ck4o_pack_int4": ([P, I64, P], None),
            "ck4o_unpack_int4": ([P, I64, P], None),
            "ck4o_quantize_weight_convrot": ([P, I64, I64, I64, I, I, P, P], None),
            "ck4o_rotate_quantize_act": ([P, I64, I64, I64, I, I, P, P], None),
            "ck4o_gemm_acc": ([P, P, I64, I64, I64, I, P], None),
            "ck4o_f64_to_bf16": ([ctypes.c_double], ctypes.c_uint16),
            "ck4o_f64_to_bf16_array": ([P, I64, P], None),
            "ck4o_epilogue_bf16": ([P, P, P, P, I64, I64, I64, P], None),
            "ck4o_linear_w4a4": ([P, P, P, P, I64, I64, I64, I, P], None),
            "ck4o_decode_w4a8": ([P, P, I64, I64, I, I64, I64, P, P], None),
            "ck4o_quantize_weight_convrot_codebook": ([P, I64, I64, I64, I, I, P, I, P, P], None),
            "ck4o_decode_w4a8_codebook": ([P, P, P, I64, I64, I, I64, I64, P, P], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().ck4o_num_threads()


def set_num_threads(n: int) -> None:
    lib().ck4o_set_num_threads(int(n))


def hadamard_scale(g: int) -> np.float32:
    return np.float32(lib().ck4o_hadamard_scale_f32(g))


def fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalised FWHT of one block (fp32 or fp64), ascending stages."""
    g = v.shape[-1]
    if v.dtype == np.float64:
        out = _c(v, np.float64).copy()
        for row in out.reshape(-1, g):
            lib().ck4o_fwht_f64(_p(row), g)
        return out
    out = _c(v, np.float32).copy()
    for row in out.reshape(-1, g):
        lib().ck4o_fwht_f32(_p(row), g)
    return out


def rotate_f32(x: np.ndarray, g: int = 128) -> np.ndarray:
    """Block-Hadamard rotation of fp32 rows, fp32 arithmetic."""
    x = _c(x, np.float32)
    m, k = x.shape
    r = np.empty((m, k), np.float32)
    lib().ck4o_rotate_rows_f32(_p(x), m, k, k, g, _p(r))
    return r


def rotate_bf16(x_bits: np.ndarray, g: int = 128) -> np.ndarray:
    """Block-Hadamard rotation of bf16 rows (uint16 bits), fp32 arithmetic."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    r = np.empty((m, k), np.float32)
    lib().ck4o_rotate_rows_bf16(_p(x), m, k, k, g, _p(r))
    return r


def rotate_f64(x: np.ndarray, g: int = 128) -> np.ndarray:
    x = _c(x, np.float64)
    m, k = x.shape
    r = np.empty((m, k), np.float64)
    lib().ck4o_rotate_rows_f64(_p(x), m, k, g, _p(r))
    return r


def quantize_rows(r: np.ndarray, group: int = 0, qmax: int = 7):
    """Absmax quantisation -> (int8 codes [m, k], fp32 scales [m] or [m, k/group])."""
    r = _c(r, np.float32)
    m, k = r.shape
    q = np.empty((m, k), np.int8)
    ng = 1 if group == 0 else k // group
    s = np.empty((m, ng), np.float32)
    lib().ck4o_quantize_rows(_p(r), m, k, group, qmax, _p(q), _p(s))
    return q, (s[:, 0].copy() if group == 0 else s)


def pack_int4(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] // 2,), np.int8)
    lib().ck4o_pack_int4(_p(q), q.size, _p(out))
    return out


def unpack_int4(p: np.ndarray) -> np.ndarray:
    p = _c(p, np.int8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
    lib().ck4o_unpack_int4(_p(p), p.size * 2, _p(out))
    return out


def quantize_weight_convrot(w: np.ndarray, g: int = 128, group: int = 0):
    """Offline weight prep -> (packed int8 [n, k/2], fp32 scales [n] or [n, k/group])."""
    w = _c(w, np.float32)
    n, k = w.shape
    packed = np.empty((n, k // 2), np.int8)
    ng = 1 if group == 0 else k // group
    s = np.empty((n, ng), np.float32)
    lib().ck4o_quantize_weight_convrot(_p(w), n, k, k, g, group, _p(packed), _p(s))
    return packed, (s[:, 0].copy() if group == 0 else s)


def quantize_weight_convrot_int8(w: np.ndarray, g: int = 128):
    """W8A8 weight prep: the fp32 rotation, then rowwise absmax / 127 codes
    -> (int8 [n, k], fp32 [n]). The int8 layout that the int4 one extends
    ([PR63] Description)."""
    return quantize_rows(rotate_f32(w, g), 0, 127)


def linear_w8a8(x_bits: np.ndarray, w8: np.ndarray, w_scales: np.ndarray, bias: np.ndarray | None = None,
                g: int = 128) -> np.ndarray:
    """y bf16 bits [m, n] of the W8A8 ConvRot linear: int8 activations, int32 GEMM, epilogue."""
    xq, sx = rotate_quantize_act(x_bits, g, bits=8)
    acc = gemm_acc(xq, w8, xq.shape[1], bits=8)
    return epilogue_bf16(acc, sx, w_scales, bias)


def quantize_rows_sr(r: np.ndarray, u: np.ndarray, group: int = 0, qmax: int = 7):
    """Stochastic-rounding quantisation with caller-supplied u in [0, 1)."""
    r = _c(r, np.float32)
    u = _c(u, np.float32)
    m, k = r.shape
    q = np.empty((m, k), np.int8)
    ng = 1 if group == 0 else k // group
    s = np.empty((m, ng), np.float32)
    lib().ck4o_quantize_rows_sr(_p(r), _p(u), k, m, k, group, qmax, _p(q), _p(s))
    return q, (s[:, 0].copy() if group == 0 else s)


def quantize_weight_convrot_sr(w: np.ndarray, u: np.ndarray, g: int = 128, group: int = 0):
    """Weight prep with stochastic rounding -> (packed int8 [n, k/2], fp32 scales)."""
    w = _c(w, np.float32)
    u = _c(u, np.float32)
    n, k = w.shape
    packed = np.empty((n, k // 2), np.int8)
    ng = 1 if group == 0 else k // group
    s = np.empty((n, ng), np.float32)
    lib().ck4o_quantize_weight_convrot_sr(_p(w), n, k, k, g, group, _p(u), k, _p(packed), _p(s))
    return packed, (s[:, 0].copy() if group == 0 else s)


def e4m3_decode(b) -> np.ndarray:
    """fp32 values of E4M3 bytes."""
    b = np.asarray(b, np.uint8)
    return np.array([lib().ck4o_e4m3_decode(int(v)) for v in b.ravel()], np.float32).reshape(b.shape)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 bytes of fp32 values (nearest, ties to even, saturating at 448)."""
    x = np.asarray(x, np.float32)
    return np.array([lib().ck4o_e4m3_encode(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def quantize_weight_convrot_e4m3(w: np.ndarray, g: int = 128, group: int = 128):
    """Grouped weight prep with e4m3 group scales -> (packed int8 [n, k/2], uint8 [n, k/group])."""
    w = _c(w, np.float32)
    n, k = w.shape
    packed = np.empty((n, k // 2), np.int8)
    s8 = np.empty((n, k // group), np.uint8)
    lib().ck4o_quantize_weight_convrot_e4m3(_p(w), n, k, k, g, group, _p(packed), _p(s8))
    return packed, s8


def linear_w4a8_grouped_e4m3(x_bits: np.ndarray, w_packed: np.ndarray, scales8: np.ndarray,
                             group: int = 128, g: int = 128) -> np.ndarray:
    """Grouped W4A8 linear with e4m3 group scales: the scales decode exactly to
    fp32, then the same decode, int8 GEMM and epilogue as fp32 scales."""
    return linear_w4a8_grouped(x_bits, w_packed, e4m3_decode(scales8), group, g)


def rotate_quantize_act(x_bits: np.ndarray, g: int = 128, bits: int = 4):
    """Dynamic activation quantisation -> (packed [m, k/2] or int8 [m, k], fp32 [m])."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    out = np.empty((m, k // 2 if bits == 4 else k), np.int8)
    s = np.empty((m,), np.float32)
    lib().ck4o_rotate_quantize_act(_p(x), m, k, k, g, bits, _p(out), _p(s))
    return out, s


def gemm_acc(a: np.ndarray, b: np.ndarray, k: int, bits: int = 4) -> np.ndarray:
    """int32 acc[m, n] = sum_k a[m, k] b[n, k] from packed int4 or int8 codes."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    m, n = a.shape[0], b.shape[0]
    acc = np.empty((m, n), np.int32)
    lib().ck4o_gemm_acc(_p(a), _p(b), m, n, k, bits, _p(acc))
    return acc


def f64_to_bf16(v: float) -> int:
    return int(lib().ck4o_f64_to_bf16(float(v)))


def epilogue_bf16(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    acc = _c(acc, np.int32)
    m, n = acc.shape
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    y = np.empty((m, n), np.uint16)
    b_keep = None if bias is None else _c(bias, np.float32)
    bp = None if b_keep is None else _p(b_keep)
    lib().ck4o_epilogue_bf16(_p(acc), _p(sx), _p(sw), bp, m, n, n, _p(y))
    return y


def linear_w4a4(x_bits: np.ndarray, w_packed: np.ndarray, w_scales: np.ndarray,
                bias: np.ndarray | None = None, g: int = 128) -> np.ndarray:
    """y bf16 bits [m, n] of the full W4A4 ConvRot linear."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    wp = _c(w_packed, np.int8)
    n = wp.shape[0]
    ws = _c(w_scales, np.float32)
    y = np.empty((m, n), np.uint16)
    b_keep = None if bias is None else _c(bias, np.float32)
    lib().ck4o_linear_w4a4(_p(x), _p(wp), _p(ws), None if b_keep is None else _p(b_keep), m, n, k, g, _p(y))
    return y


def decode_w4a8(w_packed: np.ndarray, group_scales: np.ndarray, group: int = 128,
                n0: int = 0, nc: int | None = None):
    """Grouped int4 -> int8 decode of rows [n0, n0+nc) -> (int8 [nc, k], fp32 [nc])."""
    wp = _c(w_packed, np.int8)
    n, k = wp.shape[0], wp.shape[1] * 2
    gs = _c(group_scales, np.float32)
    if nc is None:
        nc = n - n0
    w8 = np.empty((nc, k), np.int8)
    sr = np.empty((nc,), np.float32)
    lib().ck4o_decode_w4a8(_p(wp), _p(gs), n, k, group, n0, nc, _p(w8), _p(sr))
    return w8, sr


def linear_w4a8_grouped(x_bits: np.ndarray, w_packed: np.ndarray, group_scales: np.ndarray,
                        group: int = 128, g: int = 128) -> np.ndarray:
    """Grouped W4A8 linear: decode, int8 activations, int8 GEMM, epilogue."""
    w8, srow = decode_w4a8(w_packed, group_scales, group)
    xq, sx = rotate_quantize_act(x_bits, g, bits=8)
    acc = gemm_acc(xq, w8, xq.shape[1], bits=8)
    return epilogue_bf16(acc, sx, srow)


def quantize_weight_convrot_codebook(w: np.ndarray, codebook, g: int = 128, group: int = 128,
                                     e4m3: bool = False):
    """Grouped weight prep against a 16-entry codebook -> (packed indices int8
    [n, k/2], group scales fp32 [n, k/group] or e4m3 uint8 [n, k/group])."""
    w = _c(w, np.float32)
    cb = _c(codebook, np.float32)
    assert cb.shape == (16,)
    n, k = w.shape
    packed = np.empty((n, k // 2), np.int8)
    scales = np.empty((n, k // group), np.uint8 if e4m3 else np.float32)
    lib().ck4o_quantize_weight_convrot_codebook(_p(w), n, k, k, g, group, _p(cb), int(bool(e4m3)), _p(packed),
                                                _p(scales))
    return packed, scales


def decode_w4a8_codebook(w_packed: np.ndarray, group_scales: np.ndarray, codebook, group: int = 128,
                         n0: int = 0, nc: int | None = None):
    """Codebook decode of rows [n0, n0+nc) -> (int8 [nc, k], fp32 [nc]); e4m3
    scale bytes decode exactly to fp32 first."""
    wp = _c(w_packed, np.int8)
    n, k = wp.shape[0], wp.shape[1] * 2
    gs = np.asarray(group_scales)
    gs = e4m3_decode(gs) if gs.dtype == np.uint8 else _c(gs, np.float32)
    cb = _c(codebook, np.float32)
    if nc is None:
        nc = n - n0
    w8 = np.empty((nc, k), np.int8)
    sr = np.empty((nc,), np.float32)
    lib().ck4o_decode_w4a8_codebook(_p(wp), _p(gs), _p(cb), n, k, group, n0, nc, _p(w8), _p(sr))
    return w8, sr


def linear_w4a8_codebook(x_bits: np.ndarray, w_packed: np.ndarray, group_scales: np.ndarray, codebook,
                         group: int = 128, g: int = 128) -> np.ndarray:
    """Codebook W4A8 linear: codebook decode, int8 activations, int8 GEMM, epilogue."""
    w8, srow = decode_w4a8_codebook(w_packed, group_scales, codebook, group)
    xq, sx = rotate_quantize_act(x_bits, g, bits=8)
    acc = gemm_acc(xq, w8, xq.shape[1], bits=8)
    return epilogue_bf16(acc, sx, srow)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 (or fp32, converted exactly) values once to bf16, nearest even -> uint16 bits."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().ck4o_f64_to_bf16_array(_p(v), v.size, _p(out))
    return out


# ---------------------------------------------------------------------------
# Dynamic LoRA ("Comfy-INT4-HIPtest" README, "LoRA modes": the Dynamic mode
# keeps the LoRA factors apart and adds their product at inference;
# "ComfyUI-INT4-Fast", "Features": the down projection is rotated with the
# same Hadamard blocks so that it matches the rotated activation). With the
# orthonormal block rotation R, x A^T = (x R)(A R)^T: the down projection
# consumes the activation's rotation. Readings (the pages give no arithmetic):
# A R is rounded to bf16 once at preparation; the rotated activation is
# rounded to bf16 before the product; t = alpha * (x R)(A R)^T is rounded to
# bf16; the up projection t B^T is added to the layer's value before its one
# bf16 rounding. Products and sums here are fp64 over those bf16 values.


def lora_prepare_down(a: np.ndarray, g: int = 128) -> np.ndarray:
    """bf16 bits of A R: each fp32 row of the down projection rotated like a weight row."""
    return to_bf16(rotate_f32(a, g))


def lora_down(x_bits: np.ndarray, a_rot_bits: np.ndarray, alpha: float, g: int = 128) -> np.ndarray:
    """t = bf16(alpha * bf16(x R) (A R)^T) -> bf16 bits [m, rank]; x R is the quantiser's fp32 rotation."""
    xr = bf16_bits_to_f64(to_bf16(rotate_bf16(x_bits, g)))
    ar = bf16_bits_to_f64(a_rot_bits)
    return to_bf16(float(alpha) * (xr @ ar.T))


def epilogue_lora(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, t_bits: np.ndarray, b_bits: np.ndarray,
                  bias: np.ndarray | None = None) -> np.ndarray:
    """y = bf16(acc sx sw (+ bias) + t B^T), fp64 -> bf16 bits [m, n]."""
    v = _c(acc, np.int32).astype(np.float64) * _c(sx, np.float32).astype(np.float64)[:, None]
    v = v * _c(sw, np.float32).astype(np.float64)[None, :]
    if bias is not None:
        v = v + _c(bias, np.float32).astype(np.float64)[None, :]
    v = v + bf16_bits_to_f64(t_bits) @ bf16_bits_to_f64(b_bits).T
    return to_bf16(v)


def linear_w4a4_lora(x_bits: np.ndarray, w_packed: np.ndarray, w_scales: np.ndarray, a_rot_bits: np.ndarray,
                     b_bits: np.ndarray, alpha: float, bias: np.ndarray | None = None, g: int = 128) -> np.ndarray:
    """The W4A4 ConvRot layer plus a dynamic LoRA -> bf16 bits [m, n]."""
    xq, sx = rotate_quantize_act(x_bits, g, bits=4)
    acc = gemm_acc(xq, w_packed, xq.shape[1] * 2)
    t = lora_down(x_bits, a_rot_bits, alpha, g)
    return epilogue_lora(acc, sx, w_scales, t, b_bits, bias)
