"""W4A4 ConvRot linear for AMD MI355X (gfx950): Python binding of libck4.so.

Argument marshalling only. Every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/ck4.h``; PyTorch provides device
memory and the current stream. If ``libck4.so`` has not been built, every call
raises: there is no CPU fallback.

The layer ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with fused CUDA
kernels", Description): rotate the activation rows with a block Hadamard
transform, quantise each row to int4 (absmax / 7) and pack it low nibble
first, multiply against int4 weights prepared the same way with an int32
GEMM, apply the row and column scales once in the epilogue, write bf16.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libck4.so")

CK4_OK, CK4_ERR_INVALID, CK4_ERR_UNSUPPORTED, CK4_ERR_DEVICE = 0, 1, 2, 3


class Ck4Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_PF = ctypes.POINTER(ctypes.c_float)  # host float array

SIGNATURES = {
    "ck4_version": ([], ctypes.c_char_p),
    "ck4_status_string": ([_I], ctypes.c_char_p),
    "ck4_last_error": ([], ctypes.c_char_p),
    "ck4_quantize_weight_convrot": ([_P, _I64, _I64, _I64, _I, _I, _P, _P, _P], _I),
    "ck4_quantize_weight_convrot_int8": ([_P, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "ck4_quantize_weight_convrot_sr": ([_P, _I64, _I64, _I64, _I, _I, _P, _I64, _P, _P, _P], _I),
    "ck4_rotate_quantize_act": ([_P, _I64, _I64, _I64, _I, _I, _P, _P, _P], _I),
    "ck4_rotate_act_f32": ([_P, _I64, _I64, _I64, _I, _P, _P], _I),
    "ck4_linear_w4a4": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_linear_w4a4_bf16": ([_P, _I64, _I64, _I64, _I, _P, _P, _P, _I64, _P, _P, _P, _I64, _P], _I),
    "ck4_gemm_w4a4_acc_i32": ([_P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_dequant_w4a8_grouped": ([_P, _P, _I64, _I64, _I, _I64, _I64, _P, _P, _P], _I),
    "ck4_linear_w8a8": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_w4a8_workspace_bytes": ([_I64, _I64, _I64, _I64], ctypes.c_size_t),
    "ck4_linear_w4a8_grouped": ([_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _I64, _P, ctypes.c_size_t, _P], _I),
    "ck4_linear_w4a8_grouped_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _I64, _P], _I),
    "ck4_linear_w4a8_grouped_bf16": ([_P, _I64, _I64, _I64, _I, _P, _P, _I, _I64, _I, _P, _P, _P, _I64, _P,
                                      ctypes.c_size_t, _P], _I),
    "ck4_quantize_weight_convrot_e4m3": ([_P, _I64, _I64, _I64, _I, _I, _P, _P, _P], _I),
    "ck4_dequant_w4a8_grouped_e4m3": ([_P, _P, _I64, _I64, _I, _I64, _I64, _P, _P, _P], _I),
    "ck4_linear_w4a8_grouped_e4m3": ([_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _I64, _P, ctypes.c_size_t,
                                      _P], _I),
    "ck4_quantize_weight_convrot_codebook": ([_P, _I64, _I64, _I64, _I, _I, _PF, _I, _P, _P, _P], _I),
    "ck4_dequant_w4a8_codebook": ([_P, _P, _I, _PF, _I64, _I64, _I, _I64, _I64, _P, _P, _P], _I),
    "ck4_linear_w4a8_codebook": ([_P, _P, _P, _P, _I, _PF, _I64, _I64, _I64, _I, _P, _I64, _I64, _P,
                                  ctypes.c_size_t, _P], _I),
    "ck4_fp6_bytes": ([_I64, _I64], ctypes.c_size_t),
    "ck4_rotate_quantize_act_fp6": ([_P, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "ck4_quantize_weight_convrot_fp6": ([_P, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "ck4_linear_w4a4_fp6": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_gemm_w4a4_fp6_acc_i32": ([_P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_gemm_fp6_tile": ([_I64, _I64, _I64, ctypes.POINTER(_I), ctypes.POINTER(_I)], _I),
    "ck4_fp6c_bytes": ([_I64, _I64], ctypes.c_size_t),
    "ck4_rotate_quantize_act_fp6c": ([_P, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "ck4_quantize_weight_convrot_fp6c": ([_P, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "ck4_linear_w4a4_fp6c": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_gemm_w4a4_fp6c_acc_i32": ([_P, _P, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_linear_w4a4_fp6_lora": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_linear_w4a4_fp6c_lora": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P], _I),
    "ck4_lora_prepare_down": ([_P, _I64, _I64, _I64, _I, _P, _P], _I),
    "ck4_lora_prepare_up": ([_P, _I64, _I64, _I64, _P, _P], _I),
    "ck4_lora_down": ([_P, _I64, _I64, _I64, _I, _P, _I64, ctypes.c_float, _P, _P], _I),
    "ck4_linear_w4a4_lora": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P], _I),
}


def lib():
    """The loaded libck4.so (ctypes). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libck4.so not found at {LIB_PATH}: build it with "
                "`python -m int4_w4a4_quantized_amd._build` (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def version() -> str:
    return lib().ck4_version().decode()


def _check(fn: str, status: int) -> None:
    if status != CK4_OK:
        raise Ck4Error(fn, status, lib().ck4_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# Argument checks. Every wrapper checks types, dtypes, shapes, lengths and
# layouts of all its tensors first and their device last, before it calls the
# library: the kernels derive every buffer extent from m, n and k, so a short or
# mismatched tensor must be refused here rather than read out of bounds.

def _typed(t, dtype, name: str, dims: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")
    if t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dim")


def _dense(t, dtype, name: str, dims: int | None = None) -> None:
    """A contiguous tensor (the kernels take its rows back to back)."""
    _typed(t, dtype, name, dims)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _vec(t, dtype, name: str, count: int) -> None:
    """A contiguous vector holding at least `count` elements."""
    _dense(t, dtype, name)
    if t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {count}")


def _on_gpu(**tensors) -> None:
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _need(t: torch.Tensor, dtype: torch.dtype, name: str, dims: int | None = None) -> None:
    _typed(t, dtype, name, dims)
    _on_gpu(**{name: t})


def _out_checked(out, m: int, n: int, dtype=torch.bfloat16, name: str = "out") -> None:
    _typed(out, dtype, name, 2)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"{name} must have shape {(m, n)}, got {tuple(out.shape)}")


def _fp6_nbytes(rows: int, k: int, compact: bool = False) -> int:
    return (rows + 15) // 16 * 16 * (k // 128) * (64 if compact else 96)


def _fp6_k(q6, name: str, compact: bool = False) -> int:
    """k of an FP6 operand [rows16, 3k/4], or of a compact one [rows16, k/2] (k a multiple of 128)."""
    _dense(q6, torch.uint8, name, 2)
    per = 64 if compact else 96
    if q6.shape[1] % per != 0:
        form = "k/2" if compact else "3k/4"
        raise ValueError(f"{name} has {q6.shape[1]} bytes per row: not {form} for k a multiple of 128")
    return q6.shape[1] * 128 // per


def _out_bf16(m: int, n: int, device) -> torch.Tensor:
    # the kernels store 4 columns per lane: keep the row stride a multiple of 4
    ld = (n + 3) // 4 * 4
    return torch.empty((m, ld), dtype=torch.bfloat16, device=device)[:, :n]


def quantize_weight_convrot(w: torch.Tensor, rot_block: int = 128, group: int = 0):
    """Offline ConvRot weight prep: fp32 [n, k] -> (int8 [n, k/2], fp32 [n] or [n, k/group])."""
    _need(w, torch.float32, "w", 2)
    n, k = w.shape
    wp = torch.empty((n, k // 2), dtype=torch.int8, device=w.device)
    ws = torch.empty((n,) if group == 0 else (n, k // group), dtype=torch.float32, device=w.device)
    _check("ck4_quantize_weight_convrot",
           lib().ck4_quantize_weight_convrot(_ptr(w), n, k, w.stride(0), rot_block, group, _ptr(wp), _ptr(ws),
                                             _stream(w.device)))
    return wp, ws


def quantize_weight_convrot_sr(w: torch.Tensor, u: torch.Tensor, rot_block: int = 128, group: int = 0):
    """Weight prep with stochastic rounding; u fp32 [n, k] holds one draw in [0, 1) per element."""
    _need(w, torch.float32, "w", 2)
    _need(u, torch.float32, "u", 2)
    n, k = w.shape
    wp = torch.empty((n, k // 2), dtype=torch.int8, device=w.device)
    ws = torch.empty((n,) if group == 0 else (n, k // group), dtype=torch.float32, device=w.device)
    _check("ck4_quantize_weight_convrot_sr",
           lib().ck4_quantize_weight_convrot_sr(_ptr(w), n, k, w.stride(0), rot_block, group, _ptr(u), u.stride(0),
                                                _ptr(wp), _ptr(ws), _stream(w.device)))
    return wp, ws


def quantize_weight_convrot_e4m3(w: torch.Tensor, rot_block: int = 128, group: int = 128):
    """Grouped weight prep with E4M3 group scales -> (int8 [n, k/2], uint8 E4M3 bytes [n, k/group])."""
    _need(w, torch.float32, "w", 2)
    n, k = w.shape
    wp = torch.empty((n, k // 2), dtype=torch.int8, device=w.device)
    gs = torch.empty((n, k // group), dtype=torch.uint8, device=w.device)
    _check("ck4_quantize_weight_convrot_e4m3",
           lib().ck4_quantize_weight_convrot_e4m3(_ptr(w), n, k, w.stride(0), rot_block, group, _ptr(wp), _ptr(gs),
                                                  _stream(w.device)))
    return wp, gs


def _codebook(codebook):
    """16 codebook entries (list, numpy array or CPU tensor) -> a host float[16]."""
    if isinstance(codebook, torch.Tensor):
        if codebook.device.type != "cpu":
            raise ValueError("the codebook is a host array of 16 floats")
        codebook = codebook.tolist()
    vals = [float(v) for v in (codebook.tolist() if hasattr(codebook, "tolist") else codebook)]
    if len(vals) != 16:
        raise ValueError(f"the codebook has 16 entries, got {len(vals)}")
    return (ctypes.c_float * 16)(*vals)


def quantize_weight_convrot_codebook(w: torch.Tensor, codebook, rot_block: int = 128, group: int = 128,
                                     scale_e4m3: bool = False):
    """Grouped weight prep against a frozen 16-entry codebook -> (int8 [n, k/2]
    packed indices, group scales fp32 [n, k/group] or uint8 E4M3 bytes)."""
    _need(w, torch.float32, "w", 2)
    n, k = w.shape
    wp = torch.empty((n, k // 2), dtype=torch.int8, device=w.device)
    gs = torch.empty((n, k // group), dtype=torch.uint8 if scale_e4m3 else torch.float32, device=w.device)
    _check("ck4_quantize_weight_convrot_codebook",
           lib().ck4_quantize_weight_convrot_codebook(_ptr(w), n, k, w.stride(0), rot_block, group,
                                                      _codebook(codebook), int(bool(scale_e4m3)), _ptr(wp), _ptr(gs),
                                                      _stream(w.device)))
    return wp, gs


def quantize_weight_convrot_int8(w: torch.Tensor, rot_block: int = 128):
    """Offline W8A8 weight prep: fp32 [n, k] -> (int8 codes [n, k], fp32 row scales [n])."""
    _need(w, torch.float32, "w", 2)
    n, k = w.shape
    wq = torch.empty((n, k), dtype=torch.int8, device=w.device)
    ws = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check("ck4_quantize_weight_convrot_int8",
           lib().ck4_quantize_weight_convrot_int8(_ptr(w), n, k, w.stride(0), rot_block, _ptr(wq), _ptr(ws),
                                                  _stream(w.device)))
    return wq, ws


def rotate_quantize_act(x: torch.Tensor, rot_block: int = 128, bits: int = 4, out=None, scales=None):
    """Dynamic rotate + quantise: bf16 [m, k] -> (int8 [m, k/2] (bits 4) or [m, k] (bits 8), fp32 [m])."""
    _typed(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if out is not None:
        _dense(out, torch.int8, "out", 2)
        if tuple(out.shape) != (m, k // 2 if bits == 4 else k):
            raise ValueError(f"out must have shape {(m, k // 2 if bits == 4 else k)}, got {tuple(out.shape)}")
    if scales is not None:
        _vec(scales, torch.float32, "scales", m)
    _on_gpu(x=x, out=out, scales=scales)
    if out is None:
        out = torch.empty((m, k // 2 if bits == 4 else k), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check("ck4_rotate_quantize_act",
           lib().ck4_rotate_quantize_act(_ptr(x), m, k, x.stride(0), rot_block, bits, _ptr(out), _ptr(scales),
                                         _stream(x.device)))
    return out, scales


def rotate_act_f32(x: torch.Tensor, rot_block: int = 128):
    """fp32 block-Hadamard rotation of bf16 rows: [m, k] -> fp32 [m, k]."""
    _need(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    r = torch.empty((m, k), dtype=torch.float32, device=x.device)
    _check("ck4_rotate_act_f32",
           lib().ck4_rotate_act_f32(_ptr(x), m, k, x.stride(0), rot_block, _ptr(r), _stream(x.device)))
    return r


def _check_gemm(x, w, x_scales, w_scales, bias, out, dtype, what: str):
    """Operands of a GEMM wrapper: x [m, c] and w [n, c] of `dtype`, contiguous,
    with the same row width c; scales and bias long enough; out [m, n] bf16."""
    _dense(x, dtype, "x_" + what, 2)
    _dense(w, dtype, "w_" + what, 2)
    if w.shape[1] != x.shape[1]:
        raise ValueError(f"the weight rows hold {w.shape[1]} bytes, the activation rows {x.shape[1]}: k differs")
    m, n = x.shape[0], w.shape[0]
    if x_scales is not None:
        _vec(x_scales, torch.float32, "x_scales", m)
    if w_scales is not None:
        _vec(w_scales, torch.float32, "w_scales", n)
    if bias is not None:
        _vec(bias, torch.float32, "bias", n)
    if out is not None:
        _out_checked(out, m, n)
    _on_gpu(x=x, w=w, x_scales=x_scales, w_scales=w_scales, bias=bias, out=out)
    return m, n


def linear_w4a4(x_q: torch.Tensor, x_scales: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor,
                bias: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """y bf16 [m, n] from a quantised activation and a prepared weight."""
    m, n = _check_gemm(x_q, w_packed, x_scales, w_scales, bias, out, torch.int8, "q")
    k = x_q.shape[1] * 2
    if out is None:
        out = _out_bf16(m, n, x_q.device)
    _check("ck4_linear_w4a4",
           lib().ck4_linear_w4a4(_ptr(x_q), _ptr(x_scales), _ptr(w_packed), _ptr(w_scales), _ptr(bias), m, n, k,
                                 _ptr(out), out.stride(0), _stream(x_q.device)))
    return out


def gemm_w4a4_acc_i32(x_q: torch.Tensor, w_packed: torch.Tensor):
    """Exact int32 accumulators [m, n] of the W4A4 GEMM (same kernel, int32 store)."""
    m, n = _check_gemm(x_q, w_packed, None, None, None, None, torch.int8, "q")
    k = x_q.shape[1] * 2
    ldacc = (n + 3) // 4 * 4
    acc = torch.empty((m, ldacc), dtype=torch.int32, device=x_q.device)
    _check("ck4_gemm_w4a4_acc_i32",
           lib().ck4_gemm_w4a4_acc_i32(_ptr(x_q), _ptr(w_packed), m, n, k, _ptr(acc), ldacc, _stream(x_q.device)))
    return acc[:, :n]


def linear_w4a4_bf16(x: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor, bias=None,
                     rot_block: int = 128, x_q=None, x_scales=None, out=None):
    """The whole layer in one library call: bf16 x [m, k] -> (y bf16 [m, n], x_q int8 [m, k/2], x_scales fp32 [m]).

    Bitwise rotate_quantize_act(x, rot_block, 4) followed by linear_w4a4; for
    m <= 2 (rot_block 128) one kernel does both."""
    _typed(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    _dense(w_packed, torch.int8, "w_packed", 2)
    if w_packed.shape[1] * 2 != k:
        raise ValueError(f"the weight rows hold {w_packed.shape[1]} bytes, not k/2 = {k // 2}")
    n = w_packed.shape[0]
    _vec(w_scales, torch.float32, "w_scales", n)
    if bias is not None:
        _vec(bias, torch.float32, "bias", n)
    if x_q is not None:
        _dense(x_q, torch.int8, "x_q", 2)
        if tuple(x_q.shape) != (m, k // 2):
            raise ValueError(f"x_q must have shape {(m, k // 2)}, got {tuple(x_q.shape)}")
    if x_scales is not None:
        _vec(x_scales, torch.float32, "x_scales", m)
    if out is not None:
        _out_checked(out, m, n)
    _on_gpu(x=x, w_packed=w_packed, w_scales=w_scales, bias=bias, x_q=x_q, x_scales=x_scales, out=out)
    if x_q is None:
        x_q = torch.empty((m, k // 2), dtype=torch.int8, device=x.device)
    if x_scales is None:
        x_scales = torch.empty((m,), dtype=torch.float32, device=x.device)
    if out is None:
        out = _out_bf16(m, n, x.device)
    _check("ck4_linear_w4a4_bf16",
           lib().ck4_linear_w4a4_bf16(_ptr(x), m, k, x.stride(0), rot_block, _ptr(w_packed), _ptr(w_scales),
                                      _ptr(bias), n, _ptr(x_q), _ptr(x_scales), _ptr(out), out.stride(0),
                                      _stream(x.device)))
    return out, x_q, x_scales


def w4a4_linear(x: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor, bias=None, rot_block: int = 128):
    """The whole layer: rotate + quantise x, then the W4A4 GEMM + epilogue (one library call)."""
    return linear_w4a4_bf16(x, w_packed, w_scales, bias, rot_block)[0]


def dequant_w4a8_grouped(w_packed: torch.Tensor, group_scales: torch.Tensor, group: int = 128, n0: int = 0,
                         nc: int | None = None, codebook=None):
    """Grouped int4 -> int8 decode of weight rows [n0, n0+nc) -> (int8 [nc, k], fp32 [nc]).

    group_scales: fp32, or uint8 holding E4M3 bytes. codebook: the 16 host
    entries the weight was prepared with, or None for plain int4 codes.
    """
    _dense(w_packed, torch.int8, "w_packed", 2)
    n, k = w_packed.shape[0], w_packed.shape[1] * 2
    if nc is None:
        nc = n - n0
    if group <= 0 or k % group != 0:
        raise ValueError(f"group={group} must divide k={k}")
    _vec(group_scales, (torch.float32, torch.uint8), "group_scales", n * (k // group))
    if not (0 <= n0 and 0 < nc and n0 + nc <= n):
        raise ValueError(f"rows [{n0}, {n0 + nc}) are not inside [0, {n})")
    _on_gpu(w_packed=w_packed, group_scales=group_scales)
    w8 = torch.empty((nc, k), dtype=torch.int8, device=w_packed.device)
    sr = torch.empty((nc,), dtype=torch.float32, device=w_packed.device)
    e4m3 = group_scales.dtype == torch.uint8
    if codebook is not None:
        _check("ck4_dequant_w4a8_codebook",
               lib().ck4_dequant_w4a8_codebook(_ptr(w_packed), _ptr(group_scales), int(e4m3), _codebook(codebook), n,
                                               k, group, n0, nc, _ptr(w8), _ptr(sr), _stream(w_packed.device)))
        return w8, sr
    name = "ck4_dequant_w4a8_grouped_e4m3" if e4m3 else "ck4_dequant_w4a8_grouped"
    _check(name, getattr(lib(), name)(_ptr(w_packed), _ptr(group_scales), n, k, group, n0, nc, _ptr(w8), _ptr(sr),
                                      _stream(w_packed.device)))
    return w8, sr


def linear_w8a8(x_q8, x_scales, w8, w_scales, bias=None, out=None):
    """Rowwise int8 linear from int8 activations and int8 weights -> bf16 [m, n]."""
    m, n = _check_gemm(x_q8, w8, x_scales, w_scales, bias, out, torch.int8, "q8")
    k = x_q8.shape[1]
    if out is None:
        out = _out_bf16(m, n, x_q8.device)
    _check("ck4_linear_w8a8",
           lib().ck4_linear_w8a8(_ptr(x_q8), _ptr(x_scales), _ptr(w8), _ptr(w_scales), _ptr(bias), m, n, k,
                                 _ptr(out), out.stride(0), _stream(x_q8.device)))
    return out


def w8a8_linear(x: torch.Tensor, w8: torch.Tensor, w_scales: torch.Tensor, bias=None, rot_block: int = 128):
    """The whole W8A8 ConvRot layer: rotate + int8-quantise x, then the int8 GEMM + epilogue."""
    x_q8, sx = rotate_quantize_act(x, rot_block, 8)
    return linear_w8a8(x_q8, sx, w8, w_scales, bias)


def w4a8_workspace_bytes(m: int, n: int, k: int, chunk_cols: int = 0) -> int:
    return int(lib().ck4_w4a8_workspace_bytes(m, n, k, chunk_cols))


def linear_w4a8_grouped(x_q8, x_scales, w_packed, group_scales, group: int = 128, chunk_cols: int = 0,
                        out=None, workspace=None, codebook=None):
    """Grouped W4A8 linear -> bf16 [m, n].

    chunk_cols > 0: decode per column chunk + int8 GEMM; < 0: one decode pass
    + one GEMM; 0: the library's policy (the fused kernel for m <= 64).
    group_scales: fp32, or uint8 holding E4M3 bytes. codebook: the 16 host
    entries the weight was prepared with, or None.
    """
    _dense(x_q8, torch.int8, "x_q8", 2)
    _dense(w_packed, torch.int8, "w_packed", 2)
    m, k = x_q8.shape
    n = w_packed.shape[0]
    if w_packed.shape[1] * 2 != k:
        raise ValueError(f"w_packed rows hold {w_packed.shape[1]} bytes, the int8 activation has k={k}")
    if group <= 0 or k % group != 0:
        raise ValueError(f"group={group} must divide k={k}")
    _vec(x_scales, torch.float32, "x_scales", m)
    _vec(group_scales, (torch.float32, torch.uint8), "group_scales", n * (k // group))
    if out is not None:
        _out_checked(out, m, n)
    if workspace is not None:
        _dense(workspace, torch.uint8, "workspace")
    _on_gpu(x_q8=x_q8, x_scales=x_scales, w_packed=w_packed, group_scales=group_scales, out=out,
            workspace=workspace)
    if out is None:
        out = _out_bf16(m, n, x_q8.device)
    need = w4a8_workspace_bytes(m, n, k, chunk_cols)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x_q8.device)
    e4m3 = group_scales.dtype == torch.uint8
    if codebook is not None:
        _check("ck4_linear_w4a8_codebook",
               lib().ck4_linear_w4a8_codebook(_ptr(x_q8), _ptr(x_scales), _ptr(w_packed), _ptr(group_scales),
                                              int(e4m3), _codebook(codebook), m, n, k, group, _ptr(out),
                                              out.stride(0), chunk_cols, _ptr(workspace),
                                              0 if workspace is None else workspace.numel(), _stream(x_q8.device)))
        return out
    name = "ck4_linear_w4a8_grouped_e4m3" if e4m3 else "ck4_linear_w4a8_grouped"
    _check(name, getattr(lib(), name)(_ptr(x_q8), _ptr(x_scales), _ptr(w_packed), _ptr(group_scales), m, n, k,
                                      group, _ptr(out), out.stride(0), chunk_cols, _ptr(workspace),
                                      0 if workspace is None else workspace.numel(), _stream(x_q8.device)))
    return out


def linear_w4a8_grouped_bf16(x: torch.Tensor, w_packed: torch.Tensor, group_scales: torch.Tensor, group: int = 128,
                             rot_block: int = 128, x_q8=None, x_scales=None, out=None, workspace=None):
    """The whole grouped W4A8 layer in one library call: bf16 x [m, k] -> (y bf16 [m, n], x_q8 int8 [m, k],
    x_scales fp32 [m]).

    Bitwise rotate_quantize_act(x, rot_block, 8) followed by linear_w4a8_grouped(..., chunk_cols=0);
    for m = 1 (n <= 8192, rot_block 128, k <= 8192, groups of 32 or more) one kernel does both. group_scales:
    fp32, or uint8 holding E4M3 bytes."""
    _typed(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    _dense(w_packed, torch.int8, "w_packed", 2)
    if w_packed.shape[1] * 2 != k:
        raise ValueError(f"the weight rows hold {w_packed.shape[1]} bytes, not k/2 = {k // 2}")
    n = w_packed.shape[0]
    if group <= 0 or k % group != 0:
        raise ValueError(f"group={group} must divide k={k}")
    _vec(group_scales, (torch.float32, torch.uint8), "group_scales", n * (k // group))
    if x_q8 is not None:
        _dense(x_q8, torch.int8, "x_q8", 2)
        if tuple(x_q8.shape) != (m, k):
            raise ValueError(f"x_q8 must have shape {(m, k)}, got {tuple(x_q8.shape)}")
    if x_scales is not None:
        _vec(x_scales, torch.float32, "x_scales", m)
    if out is not None:
        _out_checked(out, m, n)
    if workspace is not None:
        _dense(workspace, torch.uint8, "workspace")
    _on_gpu(x=x, w_packed=w_packed, group_scales=group_scales, x_q8=x_q8, x_scales=x_scales, out=out,
            workspace=workspace)
    if x_q8 is None:
        x_q8 = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scales is None:
        x_scales = torch.empty((m,), dtype=torch.float32, device=x.device)
    if out is None:
        out = _out_bf16(m, n, x.device)
    need = w4a8_workspace_bytes(m, n, k, 0)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    e4m3 = group_scales.dtype == torch.uint8
    _check("ck4_linear_w4a8_grouped_bf16",
           lib().ck4_linear_w4a8_grouped_bf16(_ptr(x), m, k, x.stride(0), rot_block, _ptr(w_packed),
                                              _ptr(group_scales), int(e4m3), n, group, _ptr(x_q8), _ptr(x_scales),
                                              _ptr(out), out.stride(0), _ptr(workspace),
                                              0 if workspace is None else workspace.numel(), _stream(x.device)))
    return out, x_q8, x_scales


def linear_w4a8_grouped_noalloc(x_q8, x_scales, w_packed, group_scales, group: int = 128, chunk_cols: int = 0,
                                out=None):
    """linear_w4a8_grouped (fp32 group scales) without a workspace: the decode paths use the library's fixed
    device buffer (ck4.h: CK4_NOALLOC_SCRATCH_BYTES per GPU), so the call allocates nothing beyond `out` when
    one is given. Calls that overlap on one GPU race on that buffer."""
    _dense(x_q8, torch.int8, "x_q8", 2)
    _dense(w_packed, torch.int8, "w_packed", 2)
    m, k = x_q8.shape
    n = w_packed.shape[0]
    if w_packed.shape[1] * 2 != k:
        raise ValueError(f"w_packed rows hold {w_packed.shape[1]} bytes, the int8 activation has k={k}")
    if group <= 0 or k % group != 0:
        raise ValueError(f"group={group} must divide k={k}")
    _vec(x_scales, torch.float32, "x_scales", m)
    _vec(group_scales, torch.float32, "group_scales", n * (k // group))
    if out is not None:
        _out_checked(out, m, n)
    _on_gpu(x_q8=x_q8, x_scales=x_scales, w_packed=w_packed, group_scales=group_scales, out=out)
    if out is None:
        out = _out_bf16(m, n, x_q8.device)
    _check("ck4_linear_w4a8_grouped_noalloc",
           lib().ck4_linear_w4a8_grouped_noalloc(_ptr(x_q8), _ptr(x_scales), _ptr(w_packed), _ptr(group_scales), m,
                                                 n, k, group, _ptr(out), out.stride(0), chunk_cols,
                                                 _stream(x_q8.device)))
    return out


def _rows16(n: int) -> int:
    return (n + 15) // 16 * 16


# FP6 operand path (large m): int4 codes held as FP6 E2M3 q / 8 in the MFMA
# operand layout, uint8 [rows16, k * 3 / 4]; bit-identical results to the
# int4 path at twice the matrix rate.

def fp6_bytes(rows: int, k: int) -> int:
    return int(lib().ck4_fp6_bytes(rows, k))


def gemm_fp6_tile(m: int, n: int, k: int):
    """(tile_m, tile_n): the output tile the FP6 GEMM launches for an m x n x k product."""
    tm, tn = ctypes.c_int(0), ctypes.c_int(0)
    _check("ck4_gemm_fp6_tile", lib().ck4_gemm_fp6_tile(m, n, k, ctypes.byref(tm), ctypes.byref(tn)))
    return tm.value, tn.value


def rotate_quantize_act_fp6(x: torch.Tensor, rot_block: int = 128, out=None, scales=None):
    """bf16 [m, k] -> (uint8 [rows16(m), 3k/4] FP6 codes, fp32 [m] scales)."""
    _typed(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if out is not None:
        _vec(out, torch.uint8, "out", _fp6_nbytes(m, k))
    if scales is not None:
        _vec(scales, torch.float32, "scales", m)
    _on_gpu(x=x, out=out, scales=scales)
    if out is None:
        out = torch.empty((_rows16(m), k * 3 // 4), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check("ck4_rotate_quantize_act_fp6",
           lib().ck4_rotate_quantize_act_fp6(_ptr(x), m, k, x.stride(0), rot_block, _ptr(out), _ptr(scales),
                                             _stream(x.device)))
    return out, scales


def quantize_weight_convrot_fp6(w: torch.Tensor, rot_block: int = 128):
    """fp32 [n, k] -> (uint8 [rows16(n), 3k/4] FP6 codes, fp32 [n] row scales)."""
    _need(w, torch.float32, "w", 2)
    n, k = w.shape
    wq = torch.empty((_rows16(n), k * 3 // 4), dtype=torch.uint8, device=w.device)
    ws = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check("ck4_quantize_weight_convrot_fp6",
           lib().ck4_quantize_weight_convrot_fp6(_ptr(w), n, k, w.stride(0), rot_block, _ptr(wq), _ptr(ws),
                                                 _stream(w.device)))
    return wq, ws


def linear_w4a4_fp6(x_q6, x_scales, w_q6, w_scales, bias=None, out=None, m: int | None = None,
                    n: int | None = None):
    """W4A4 GEMM + epilogue from FP6 operands -> bf16 [m, n] (m, n default to the scale lengths)."""
    _typed(x_scales, torch.float32, "x_scales")
    _typed(w_scales, torch.float32, "w_scales")
    m = x_scales.numel() if m is None else m
    n = w_scales.numel() if n is None else n
    k = _check_fp6_gemm(x_q6, w_q6, m, n, x_scales, w_scales, bias, out)
    if out is None:
        out = _out_bf16(m, n, x_q6.device)
    _check("ck4_linear_w4a4_fp6",
           lib().ck4_linear_w4a4_fp6(_ptr(x_q6), _ptr(x_scales), _ptr(w_q6), _ptr(w_scales), _ptr(bias), m, n, k,
                                     _ptr(out), out.stride(0), _stream(x_q6.device)))
    return out


def _check_fp6_gemm(x_q6, w_q6, m: int, n: int, x_scales, w_scales, bias, out, compact: bool = False) -> int:
    """Operands of an FP6 (or compact FP6) GEMM wrapper; returns k."""
    k = _fp6_k(x_q6, "x_q6", compact)
    if _fp6_k(w_q6, "w_q6", compact) != k:
        raise ValueError(f"w_q6 rows hold {w_q6.shape[1]} bytes, x_q6 rows {x_q6.shape[1]}: k differs")
    if m <= 0 or n <= 0:
        raise ValueError("m and n must be positive")
    if x_q6.numel() < _fp6_nbytes(m, k, compact):
        raise ValueError(f"x_q6 holds {x_q6.numel()} bytes, {m} rows need {_fp6_nbytes(m, k, compact)}")
    if w_q6.numel() < _fp6_nbytes(n, k, compact):
        raise ValueError(f"w_q6 holds {w_q6.numel()} bytes, {n} rows need {_fp6_nbytes(n, k, compact)}")
    if x_scales is not None:
        _vec(x_scales, torch.float32, "x_scales", m)
    if w_scales is not None:
        _vec(w_scales, torch.float32, "w_scales", n)
    if bias is not None:
        _vec(bias, torch.float32, "bias", n)
    if out is not None:
        _out_checked(out, m, n)
    _on_gpu(x_q6=x_q6, w_q6=w_q6, x_scales=x_scales, w_scales=w_scales, bias=bias, out=out)
    return k


def gemm_w4a4_fp6_acc_i32(x_q6, w_q6, m: int, n: int):
    """Integer accumulators of the FP6 GEMM -> int32 [m, n]."""
    k = _check_fp6_gemm(x_q6, w_q6, m, n, None, None, None, None)
    acc = torch.empty((m, (n + 3) // 4 * 4), dtype=torch.int32, device=x_q6.device)
    _check("ck4_gemm_w4a4_fp6_acc_i32",
           lib().ck4_gemm_w4a4_fp6_acc_i32(_ptr(x_q6), _ptr(w_q6), m, n, k, _ptr(acc), acc.stride(0),
                                           _stream(x_q6.device)))
    return acc[:, :n]


def w4a4_linear_fp6(x: torch.Tensor, w_q6: torch.Tensor, w_scales: torch.Tensor, bias=None, rot_block: int = 128):
    """The whole layer on the FP6 path: rotate + quantise x to FP6 codes, then the GEMM + epilogue."""
    x_q6, sx = rotate_quantize_act_fp6(x, rot_block)
    return linear_w4a4_fp6(x_q6, sx, w_q6, w_scales, bias)


# Compact FP6 operands: the same images without the two zero exponent bits
# of each code, uint8 [rows16, k / 2] (ck4_fp6c_bytes); expanded in registers
# before the MFMAs, with the FP6 path's results bit for bit.

def fp6c_bytes(rows: int, k: int) -> int:
    return int(lib().ck4_fp6c_bytes(rows, k))


def rotate_quantize_act_fp6c(x: torch.Tensor, rot_block: int = 128, out=None, scales=None):
    """bf16 [m, k] -> (uint8 [rows16(m), k/2] compact FP6 codes, fp32 [m] scales)."""
    _typed(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if out is not None:
        _vec(out, torch.uint8, "out", _fp6_nbytes(m, k, True))
    if scales is not None:
        _vec(scales, torch.float32, "scales", m)
    _on_gpu(x=x, out=out, scales=scales)
    if out is None:
        out = torch.empty((_rows16(m), k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check("ck4_rotate_quantize_act_fp6c",
           lib().ck4_rotate_quantize_act_fp6c(_ptr(x), m, k, x.stride(0), rot_block, _ptr(out), _ptr(scales),
                                              _stream(x.device)))
    return out, scales


def quantize_weight_convrot_fp6c(w: torch.Tensor, rot_block: int = 128):
    """fp32 [n, k] -> (uint8 [rows16(n), k/2] compact FP6 codes, fp32 [n] row scales)."""
    _need(w, torch.float32, "w", 2)
    n, k = w.shape
    wq = torch.empty((_rows16(n), k // 2), dtype=torch.uint8, device=w.device)
    ws = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check("ck4_quantize_weight_convrot_fp6c",
           lib().ck4_quantize_weight_convrot_fp6c(_ptr(w), n, k, w.stride(0), rot_block, _ptr(wq), _ptr(ws),
                                                  _stream(w.device)))
    return wq, ws


def linear_w4a4_fp6c(x_q6c, x_scales, w_q6c, w_scales, bias=None, out=None, m: int | None = None,
                     n: int | None = None):
    """W4A4 GEMM + epilogue from compact FP6 operands -> bf16 [m, n]."""
    _typed(x_scales, torch.float32, "x_scales")
    _typed(w_scales, torch.float32, "w_scales")
    m = x_scales.numel() if m is None else m
    n = w_scales.numel() if n is None else n
    k = _check_fp6_gemm(x_q6c, w_q6c, m, n, x_scales, w_scales, bias, out, compact=True)
    if out is None:
        out = _out_bf16(m, n, x_q6c.device)
    _check("ck4_linear_w4a4_fp6c",
           lib().ck4_linear_w4a4_fp6c(_ptr(x_q6c), _ptr(x_scales), _ptr(w_q6c), _ptr(w_scales), _ptr(bias), m, n, k,
                                      _ptr(out), out.stride(0), _stream(x_q6c.device)))
    return out


def gemm_w4a4_fp6c_acc_i32(x_q6c, w_q6c, m: int, n: int):
    """Integer accumulators of the compact FP6 GEMM -> int32 [m, n]."""
    k = _check_fp6_gemm(x_q6c, w_q6c, m, n, None, None, None, None, compact=True)
    acc = torch.empty((m, (n + 3) // 4 * 4), dtype=torch.int32, device=x_q6c.device)
    _check("ck4_gemm_w4a4_fp6c_acc_i32",
           lib().ck4_gemm_w4a4_fp6c_acc_i32(_ptr(x_q6c), _ptr(w_q6c), m, n, k, _ptr(acc), acc.stride(0),
                                            _stream(x_q6c.device)))
    return acc[:, :n]


def w4a4_linear_fp6c(x: torch.Tensor, w_q6c: torch.Tensor, w_scales: torch.Tensor, bias=None, rot_block: int = 128):
    """The whole layer on compact FP6 operands: rotate + quantise, then the GEMM + epilogue."""
    x_q6c, sx = rotate_quantize_act_fp6c(x, rot_block)
    return linear_w4a4_fp6c(x_q6c, sx, w_q6c, w_scales, bias)


def lora_prepare_down(a: torch.Tensor, rot_block: int = 128):
    """Rotated LoRA down projection: fp32 A [rank, k] -> bf16 A R [rank, k] in MFMA fragment order."""
    _need(a, torch.float32, "a", 2)
    rank, k = a.shape
    a_pack = torch.empty((rank, k), dtype=torch.bfloat16, device=a.device)
    _check("ck4_lora_prepare_down",
           lib().ck4_lora_prepare_down(_ptr(a), rank, k, a.stride(0), rot_block, _ptr(a_pack), _stream(a.device)))
    return a_pack


def lora_prepare_up(b: torch.Tensor):
    """LoRA up projection: bf16 B [n, rank] -> fragment order [16 * ceil(n / 16), rank] (zero padding rows)."""
    _need(b, torch.bfloat16, "b", 2)
    n, rank = b.shape
    b_pack = torch.empty((_rows16(n), rank), dtype=torch.bfloat16, device=b.device)
    _check("ck4_lora_prepare_up",
           lib().ck4_lora_prepare_up(_ptr(b), n, rank, b.stride(0), _ptr(b_pack), _stream(b.device)))
    return b_pack


def lora_down(x: torch.Tensor, a_pack: torch.Tensor, alpha: float = 1.0, rot_block: int = 128, out=None):
    """t = bf16(alpha * bf16(x R) (A R)^T) in fragment order [16 * ceil(m / 16), rank], from bf16 x [m, k]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(a_pack, torch.bfloat16, "a_pack", 2)
    m, k = x.shape
    rank = a_pack.shape[0]
    if a_pack.shape[1] != k or not a_pack.is_contiguous():
        raise ValueError("a_pack must be a contiguous [rank, k] tensor")
    if out is None:
        out = torch.empty((_rows16(m), rank), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (_rows16(m), rank) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [16 * ceil(m / 16), rank] tensor")
    _check("ck4_lora_down",
           lib().ck4_lora_down(_ptr(x), m, k, x.stride(0), rot_block, _ptr(a_pack), rank, float(alpha), _ptr(out),
                               _stream(x.device)))
    return out


def linear_w4a4_lora(x_q: torch.Tensor, x_scales: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor,
                     t_pack: torch.Tensor, b_pack: torch.Tensor, bias: torch.Tensor | None = None,
                     out: torch.Tensor | None = None):
    """W4A4 linear with the LoRA up projection in its epilogue: y = base + t B^T, bf16 [m, n].

    t_pack from lora_down, b_pack from lora_prepare_up (both in fragment order)."""
    m, n = _check_gemm(x_q, w_packed, x_scales, w_scales, bias, out, torch.int8, "q")
    k = x_q.shape[1] * 2
    _need(t_pack, torch.bfloat16, "t_pack", 2)
    _need(b_pack, torch.bfloat16, "b_pack", 2)
    rank = t_pack.shape[1]
    if tuple(t_pack.shape) != (_rows16(m), rank) or not t_pack.is_contiguous():
        raise ValueError("t_pack must be a contiguous [16 * ceil(m / 16), rank] tensor")
    if tuple(b_pack.shape) != (_rows16(n), rank) or not b_pack.is_contiguous():
        raise ValueError("b_pack must be a contiguous [16 * ceil(n / 16), rank] tensor")
    if out is None:
        out = _out_bf16(m, n, x_q.device)
    _need(out, torch.bfloat16, "out", 2)
    _check("ck4_linear_w4a4_lora",
           lib().ck4_linear_w4a4_lora(_ptr(x_q), _ptr(x_scales), _ptr(w_packed), _ptr(w_scales), _ptr(bias),
                                      _ptr(t_pack), _ptr(b_pack), rank, m, n, k, _ptr(out), out.stride(0),
                                      _stream(x_q.device)))
    return out


def linear_w4a4_fp6_lora(x_q6: torch.Tensor, x_scales: torch.Tensor, w_q6: torch.Tensor, w_scales: torch.Tensor,
                         t_pack: torch.Tensor, b_pack: torch.Tensor, bias: torch.Tensor | None = None,
                         out: torch.Tensor | None = None):
    """linear_w4a4_lora on the FP6 operand path (same bits): y = base + t B^T, bf16 [m, n]."""
    return _fp6_lora(x_q6, x_scales, w_q6, w_scales, t_pack, b_pack, bias, out, False)


def linear_w4a4_fp6c_lora(x_q6c: torch.Tensor, x_scales: torch.Tensor, w_q6c: torch.Tensor,
                          w_scales: torch.Tensor, t_pack: torch.Tensor, b_pack: torch.Tensor,
                          bias: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """linear_w4a4_lora on compact FP6 operands (same bits): y = base + t B^T, bf16 [m, n]."""
    return _fp6_lora(x_q6c, x_scales, w_q6c, w_scales, t_pack, b_pack, bias, out, True)


def _fp6_lora(x_q6, x_scales, w_q6, w_scales, t_pack, b_pack, bias, out, compact: bool):
    _typed(x_scales, torch.float32, "x_scales")
    _typed(w_scales, torch.float32, "w_scales")
    m, n = x_scales.numel(), w_scales.numel()
    k = _check_fp6_gemm(x_q6, w_q6, m, n, x_scales, w_scales, bias, out, compact=compact)
    _need(t_pack, torch.bfloat16, "t_pack", 2)
    _need(b_pack, torch.bfloat16, "b_pack", 2)
    rank = t_pack.shape[1]
    if tuple(t_pack.shape) != (_rows16(m), rank) or not t_pack.is_contiguous():
        raise ValueError("t_pack must be a contiguous [16 * ceil(m / 16), rank] tensor")
    if tuple(b_pack.shape) != (_rows16(n), rank) or not b_pack.is_contiguous():
        raise ValueError("b_pack must be a contiguous [16 * ceil(n / 16), rank] tensor")
    if out is None:
        out = _out_bf16(m, n, x_q6.device)
    _need(out, torch.bfloat16, "out", 2)
    name = "ck4_linear_w4a4_fp6c_lora" if compact else "ck4_linear_w4a4_fp6_lora"
    _check(name, getattr(lib(), name)(_ptr(x_q6), _ptr(x_scales), _ptr(w_q6), _ptr(w_scales), _ptr(bias),
                                      _ptr(t_pack), _ptr(b_pack), rank, m, n, k, _ptr(out), out.stride(0),
                                      _stream(x_q6.device)))
    return out


def w4a4_lora_linear(x: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor, a_pack: torch.Tensor,
                     b_pack: torch.Tensor, alpha: float = 1.0, bias=None, rot_block: int = 128):
    """The whole layer with a dynamic LoRA: quantise x, down-project its rotation, GEMM + fused up projection."""
    x_q, sx = rotate_quantize_act(x, rot_block, 4)
    t = lora_down(x, a_pack, alpha, rot_block)
    return linear_w4a4_lora(x_q, sx, w_packed, w_scales, t, b_pack, bias)


def w4a4_lora_linear_fp6(x: torch.Tensor, w_q6: torch.Tensor, w_scales: torch.Tensor, a_pack: torch.Tensor,
                         b_pack: torch.Tensor, alpha: float = 1.0, bias=None, rot_block: int = 128):
    """w4a4_lora_linear on the FP6 operand path (same bits): FP6 codes of x, LoRA down projection, FP6 GEMM with
    the fused up projection."""
    x_q6, sx = rotate_quantize_act_fp6(x, rot_block)
    t = lora_down(x, a_pack, alpha, rot_block)
    return linear_w4a4_fp6_lora(x_q6, sx, w_q6, w_scales, t, b_pack, bias)


def w4a4_lora_linear_fp6c(x: torch.Tensor, w_q6c: torch.Tensor, w_scales: torch.Tensor, a_pack: torch.Tensor,
                          b_pack: torch.Tensor, alpha: float = 1.0, bias=None, rot_block: int = 128):
    """w4a4_lora_linear on compact FP6 operands (same bits): compact codes of x, LoRA down projection, GEMM with
    the fused up projection."""
    x_q6c, sx = rotate_quantize_act_fp6c(x, rot_block)
    t = lora_down(x, a_pack, alpha, rot_block)
    return linear_w4a4_fp6c_lora(x_q6c, sx, w_q6c, w_scales, t, b_pack, bias)
