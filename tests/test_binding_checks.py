"""Host-side checks of the Python binding's argument validation (no GPU needed).

The kernels take every buffer extent from m, n and k, so the binding must
refuse a tensor of the wrong dtype, width or length before anything reaches
the library. These tests replace the library handle with one that fails the
test if it is touched, pass CPU tensors, and expect ValueError: first for each
planted mismatch, then (everything else right) for the host placement itself.
"""
import pytest
import torch

import int4_w4a4_quantized_amd as ck


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def touched():
        raise AssertionError("the library was called before the arguments were validated")
    monkeypatch.setattr(ck, "lib", touched)


def i8(*shape):
    return torch.zeros(shape, dtype=torch.int8)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def refused(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


M, N, K = 8, 12, 256


def test_linear_w4a4_checks():
    ok = dict(x_q=i8(M, K // 2), x_scales=f32(M), w_packed=i8(N, K // 2), w_scales=f32(N))
    refused("k differs", ck.linear_w4a4, **{**ok, "w_packed": i8(N, K // 2 + 64)})
    refused("int8", ck.linear_w4a4, **{**ok, "x_q": u8(M, K // 2)})
    refused("x_scales holds 7", ck.linear_w4a4, **{**ok, "x_scales": f32(M - 1)})
    refused("w_scales holds", ck.linear_w4a4, **{**ok, "w_scales": f32(N - 1)})
    refused("w_scales must be torch.float32", ck.linear_w4a4, **{**ok, "w_scales": bf16(N)})
    refused("bias must be torch.float32", ck.linear_w4a4, **ok, bias=bf16(N))
    refused("bias holds", ck.linear_w4a4, **ok, bias=f32(N - 2))
    refused("contiguous", ck.linear_w4a4, **{**ok, "x_q": i8(M, K)[:, :K // 2]})
    refused("unit stride", ck.linear_w4a4, **{**ok, "x_q": i8(K // 2, M).t()})
    refused("out must have shape", ck.linear_w4a4, **ok, out=bf16(M, N + 1))
    refused("out must be torch.bfloat16", ck.linear_w4a4, **ok, out=f32(M, N))
    refused("CUDA", ck.linear_w4a4, **ok)
    refused("k differs", ck.gemm_w4a4_acc_i32, i8(M, K // 2), i8(N, K))
    refused("CUDA", ck.gemm_w4a4_acc_i32, i8(M, K // 2), i8(N, K // 2))


def test_linear_w4a4_bf16_checks():
    ok = dict(x=bf16(M, K), w_packed=i8(N, K // 2), w_scales=f32(N))
    refused("not k/2", ck.linear_w4a4_bf16, **{**ok, "w_packed": i8(N, K)})
    refused("x must be torch.bfloat16", ck.linear_w4a4_bf16, **{**ok, "x": f32(M, K)})
    refused("w_scales holds", ck.linear_w4a4_bf16, **{**ok, "w_scales": f32(N - 1)})
    refused("bias holds", ck.linear_w4a4_bf16, **ok, bias=f32(N - 1))
    refused("x_q must have shape", ck.linear_w4a4_bf16, **ok, x_q=i8(M, K))
    refused("x_scales holds", ck.linear_w4a4_bf16, **ok, x_scales=f32(M - 1))
    refused("out must have shape", ck.linear_w4a4_bf16, **ok, out=bf16(M + 1, N))
    refused("CUDA", ck.linear_w4a4_bf16, **ok)


def test_linear_w4a8_bf16_checks():
    g = 128
    ok = dict(x=bf16(M, K), w_packed=i8(N, K // 2), group_scales=f32(N, K // g))
    refused("not k/2", ck.linear_w4a8_grouped_bf16, **{**ok, "w_packed": i8(N, K)})
    refused("x must be torch.bfloat16", ck.linear_w4a8_grouped_bf16, **{**ok, "x": f32(M, K)})
    refused("group_scales holds", ck.linear_w4a8_grouped_bf16, **{**ok, "group_scales": f32(N, K // g - 1)})
    refused("group_scales must be", ck.linear_w4a8_grouped_bf16, **{**ok, "group_scales": bf16(N, K // g)})
    refused("must divide", ck.linear_w4a8_grouped_bf16, **ok, group=96)
    refused("x_q8 must have shape", ck.linear_w4a8_grouped_bf16, **ok, x_q8=i8(M, K // 2))
    refused("x_scales holds", ck.linear_w4a8_grouped_bf16, **ok, x_scales=f32(M - 1))
    refused("out must have shape", ck.linear_w4a8_grouped_bf16, **ok, out=bf16(M + 1, N))
    refused("workspace must be", ck.linear_w4a8_grouped_bf16, **ok, workspace=f32(64))
    refused("CUDA", ck.linear_w4a8_grouped_bf16, **ok)
    refused("CUDA", ck.linear_w4a8_grouped_bf16, **{**ok, "group_scales": u8(N, K // g)})


def test_linear_w8a8_checks():
    refused("k differs", ck.linear_w8a8, i8(M, K), f32(M), i8(N, K // 2), f32(N))
    refused("w_scales holds", ck.linear_w8a8, i8(M, K), f32(M), i8(N, K), f32(3))
    refused("CUDA", ck.linear_w8a8, i8(M, K), f32(M), i8(N, K), f32(N))


def test_linear_w4a8_checks():
    g = 128
    ok = dict(x_q8=i8(M, K), x_scales=f32(M), w_packed=i8(N, K // 2), group_scales=f32(N, K // g))
    refused("k=256", ck.linear_w4a8_grouped, **{**ok, "w_packed": i8(N, K)})
    refused("group_scales holds", ck.linear_w4a8_grouped, **{**ok, "group_scales": f32(N, K // g - 1)})
    refused("group_scales must be", ck.linear_w4a8_grouped, **{**ok, "group_scales": bf16(N, K // g)})
    refused("must divide", ck.linear_w4a8_grouped, **ok, group=96)
    refused("x_scales holds", ck.linear_w4a8_grouped, **{**ok, "x_scales": f32(1)})
    refused("workspace must be", ck.linear_w4a8_grouped, **ok, workspace=f32(64))
    refused("CUDA", ck.linear_w4a8_grouped, **ok)
    refused("CUDA", ck.linear_w4a8_grouped, **{**ok, "group_scales": u8(N, K // g)})
    refused("group_scales holds", ck.dequant_w4a8_grouped, i8(N, K // 2), f32(N), 128)
    refused("not inside", ck.dequant_w4a8_grouped, i8(N, K // 2), f32(N, 2), 128, 8, 8)
    refused("CUDA", ck.dequant_w4a8_grouped, i8(N, K // 2), f32(N, 2), 128)


def test_fp6_checks():
    k = 384
    b = lambda rows: (rows + 15) // 16 * 16  # noqa: E731
    ok = dict(x_q6=u8(b(M), k * 3 // 4), x_scales=f32(M), w_q6=u8(b(N), k * 3 // 4), w_scales=f32(N))
    refused("k differs", ck.linear_w4a4_fp6, **{**ok, "w_q6": u8(b(N), 96)})
    refused("not 3k/4", ck.linear_w4a4_fp6, **{**ok, "x_q6": u8(b(M), 100)})
    refused("uint8", ck.linear_w4a4_fp6, **{**ok, "x_q6": i8(b(M), k * 3 // 4)})
    refused("x_q6 holds", ck.linear_w4a4_fp6, **ok, m=40)
    refused("w_q6 holds", ck.linear_w4a4_fp6, **ok, n=40)
    refused("x_scales holds", ck.linear_w4a4_fp6, **ok, m=9)
    refused("bias holds", ck.linear_w4a4_fp6, **ok, bias=f32(1))
    refused("CUDA", ck.linear_w4a4_fp6, **ok)
    refused("x_q6 holds", ck.gemm_w4a4_fp6_acc_i32, ok["x_q6"], ok["w_q6"], 17, N)
    refused("CUDA", ck.gemm_w4a4_fp6_acc_i32, ok["x_q6"], ok["w_q6"], M, N)


def test_fp6c_checks():
    k = 384
    b = lambda rows: (rows + 15) // 16 * 16  # noqa: E731
    ok = dict(x_q6c=u8(b(M), k // 2), x_scales=f32(M), w_q6c=u8(b(N), k // 2), w_scales=f32(N))
    refused("k differs", ck.linear_w4a4_fp6c, **{**ok, "w_q6c": u8(b(N), 64)})
    refused("not k/2", ck.linear_w4a4_fp6c, **{**ok, "x_q6c": u8(b(M), 100)})
    refused("not k/2", ck.linear_w4a4_fp6c, **{**ok, "x_q6c": u8(b(M), k * 3 // 4)})  # an FP6-image operand
    refused("uint8", ck.linear_w4a4_fp6c, **{**ok, "x_q6c": i8(b(M), k // 2)})
    refused("x_q6 holds", ck.linear_w4a4_fp6c, **ok, m=40)
    refused("w_q6 holds", ck.linear_w4a4_fp6c, **ok, n=40)
    refused("x_scales holds", ck.linear_w4a4_fp6c, **ok, m=9)
    refused("bias holds", ck.linear_w4a4_fp6c, **ok, bias=f32(1))
    refused("CUDA", ck.linear_w4a4_fp6c, **ok)
    refused("x_q6 holds", ck.gemm_w4a4_fp6c_acc_i32, ok["x_q6c"], ok["w_q6c"], 17, N)
    refused("CUDA", ck.gemm_w4a4_fp6c_acc_i32, ok["x_q6c"], ok["w_q6c"], M, N)
    refused("out holds", ck.rotate_quantize_act_fp6c, bf16(M, K), 128, out=u8(4, 64))
    refused("CUDA", ck.rotate_quantize_act_fp6c, bf16(M, K), 128)
    t, bp = bf16(b(M), 32), bf16(b(N), 32)
    refused("CUDA", ck.linear_w4a4_fp6c_lora, ok["x_q6c"], ok["x_scales"], ok["w_q6c"], ok["w_scales"], t, bp)


def test_quantiser_output_checks():
    refused("out must have shape", ck.rotate_quantize_act, bf16(M, K), 128, 4, out=i8(M, K))
    refused("scales holds", ck.rotate_quantize_act, bf16(M, K), 128, 8, out=i8(M, K), scales=f32(2))
    refused("CUDA", ck.rotate_quantize_act, bf16(M, K), 128, 4)
    refused("out holds", ck.rotate_quantize_act_fp6, bf16(M, K), 128, out=u8(4, 96))
    refused("CUDA", ck.rotate_quantize_act_fp6, bf16(M, K), 128)


def test_lora_gemm_checks():
    t = bf16(16, 32)
    bp = bf16(16, 32)
    refused("k differs", ck.linear_w4a4_lora, i8(M, K // 2), f32(M), i8(N, 64), f32(N), t, bp)
    refused("CUDA", ck.linear_w4a4_lora, i8(M, K // 2), f32(M), i8(N, K // 2), f32(N), t, bp)
