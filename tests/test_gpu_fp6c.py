"""GPU parity of the compact FP6 operand path (ck4_*_fp6c) through the C ABI.

The quantisers' compact codes are checked byte for byte against the layout of
tests/fp6c_layout.py applied to the oracle's codes, and decoded against the
oracle; the GEMM's int32 accumulators bit-exact against the oracle; the bf16
outputs bit-identical to the FP6 path (itself pinned to the oracle) and
within 1e-2 of the oracle.
"""
import numpy as np
import pytest
import torch

import fp6c_layout
import oracle
import workloads
from test_gpu_parity import (FP6_CASES, _rows_per_tile_row, act, assert_bf16_close, bf16_host_bits, dev_bf16,
                             host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ck():
    import int4_w4a4_quantized_amd as ck
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    return ck


@pytest.mark.parametrize("m,k,rb", [(64, 256, 128), (17, 384, 128), (5, 3072, 128), (3, 12288, 128),
                                    (9, 1024, 16), (9, 2048, 256), (2, 16384, 128), (20, 384, 128),
                                    (36, 4096, 128), (132, 3072, 128), (4, 128, 16)])
def test_fp6c_activation_codes_bitexact(ck, m, k, rb):
    xb = act(m, k, 5000 + m + k)
    xb[0] = 0                          # an all-zero row: scale 0, codes 0
    x = dev_bf16(xb)
    q, sx = ck.rotate_quantize_act_fp6c(x, rb)
    q_ref, s_ref = oracle.rotate_quantize_act(xb, rb, 4)
    codes = oracle.unpack_int4(q_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
    got = host(q).reshape(-1)[: fp6c_layout.nbytes(m, k)]
    assert np.array_equal(fp6c_layout.decode(got, m, k), codes)
    # the written rows, byte for byte (padding rows are not written)
    want = fp6c_layout.encode(codes).reshape(-1, 1024)
    for blk in range(want.shape[0]):
        rows = min(16, m - (blk // (k // 128)) * 16)
        img = np.arange(1024).reshape(4, 16, 16)[:, :rows].ravel()
        assert np.array_equal(got.reshape(-1, 1024)[blk, img], want[blk, img])


@pytest.mark.parametrize("n,k,rb", [(64, 256, 128), (300, 3072, 128), (5, 12288, 128), (33, 1024, 64)])
def test_fp6c_weight_codes_bitexact(ck, n, k, rb):
    rng = np.random.default_rng(5100 + n)
    w = workloads.make_weight(rng, n, k)
    w[1] = 0
    w[2, 5] = 3.0
    q, ws = ck.quantize_weight_convrot_fp6c(torch.from_numpy(w).cuda(), rb)
    wp_ref, ws_ref = oracle.quantize_weight_convrot(w, rb, 0)
    assert np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(fp6c_layout.decode(host(q), n, k), oracle.unpack_int4(wp_ref))


def _operands(m, n, k, seed):
    """Oracle codes and scales, and the same codes uploaded in the compact layout."""
    rng = np.random.default_rng(seed)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    xq, sx = oracle.rotate_quantize_act(xb, 128, 4)
    wp, ws = oracle.quantize_weight_convrot(w, 128, 0)
    xc = torch.from_numpy(fp6c_layout.encode(oracle.unpack_int4(xq)).reshape(-1, k // 2)).cuda()
    wc = torch.from_numpy(fp6c_layout.encode(oracle.unpack_int4(wp)).reshape(-1, k // 2)).cuda()
    return xb, xq, sx, wp, ws, xc, wc


@pytest.mark.parametrize("m,n,k", FP6_CASES)
def test_fp6c_gemm_acc_i32_bitexact(ck, m, n, k):
    _, xq, _, wp, _, xc, wc = _operands(m, n, k, 5200 + m + n)
    acc = host(ck.gemm_w4a4_fp6c_acc_i32(xc, wc, m, n))
    assert np.array_equal(acc, oracle.gemm_acc(xq, wp, k, bits=4))


@pytest.mark.parametrize("m,n,k", FP6_CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_fp6c_linear_matches_oracle(ck, m, n, k, with_bias):
    xb, xq, sx, wp, ws, xc, wc = _operands(m, n, k, 5300 + m + n)
    bias = np.random.default_rng(5301).normal(0, 0.1, n).astype(np.float32) if with_bias else None
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    sxd, wsd = torch.from_numpy(sx).cuda(), torch.from_numpy(ws).cuda()
    y = bf16_host_bits(ck.linear_w4a4_fp6c(xc, sxd, wc, wsd, bd))
    acc = oracle.gemm_acc(xq, wp, k, bits=4)
    ref = oracle.epilogue_bf16(acc, sx, ws, bias)
    atol = None
    if bias is not None:
        terms = np.abs(acc * sx.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]) + np.abs(bias)
        atol = 2.0 ** -21 * terms
    assert_bf16_close(y, ref, atol=atol)


@pytest.mark.parametrize("m,n,k", [(4600, 3000, 1024), (4100, 2900, 512), (2000, 1500, 1536), (1000, 700, 768),
                                   (2000, 3500, 384)])
def test_fp6c_ragged_large_equals_fp6_path(ck, m, n, k):
    """Ragged edges on both tile sizes, quantisers included: the compact path gives the FP6 path's bits."""
    rng = np.random.default_rng(5400 + m)
    xb = workloads.make_activations(rng, m, k)
    w = torch.from_numpy(workloads.make_weight(rng, n, k)).cuda()
    bias = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    x = dev_bf16(xb)
    wq6, ws6 = ck.quantize_weight_convrot_fp6(w, 128)
    wqc, wsc = ck.quantize_weight_convrot_fp6c(w, 128)
    xq6, sx6 = ck.rotate_quantize_act_fp6(x, 128)
    xqc, sxc = ck.rotate_quantize_act_fp6c(x, 128)
    assert torch.equal(ws6, wsc) and torch.equal(sx6, sxc)
    ldy = (n + 7) // 8 * 8 + 4          # rows 8-byte but not 16-byte aligned
    y6 = torch.full((m, ldy), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    yc = y6.clone()
    ck.linear_w4a4_fp6(xq6, sx6, wq6, ws6, bias, out=y6[:, :n])
    ck.linear_w4a4_fp6c(xqc, sxc, wqc, wsc, bias, out=yc[:, :n])
    assert np.array_equal(bf16_host_bits(y6), bf16_host_bits(yc))
    assert (bf16_host_bits(yc)[:, n:] == 0xFFFF).all()   # nothing written past n
    assert torch.equal(ck.gemm_w4a4_fp6_acc_i32(xq6, wq6, m, n), ck.gemm_w4a4_fp6c_acc_i32(xqc, wqc, m, n))


@pytest.mark.parametrize("k", [128, 3072, 12288, 131072])
@pytest.mark.parametrize("m,n,tile", [(16, 8, (96, 128)), (2304, 3072, (288, 192))])
def test_fp6c_accumulator_bound_is_reached_exactly(ck, m, n, tile, k):
    """Codes +7 everywhere against rows of +7 and -7 give acc = +-49 K exactly on both tiles of the compact
    GEMM, up to the largest k it accepts ([PR #63] Description: |acc| <= 49 K)."""
    assert ck.gemm_fp6_tile(m, n, k) == tile
    blocks = k // 128

    def block(row_codes):
        return fp6c_layout.encode(np.repeat(np.asarray(row_codes, np.int64)[:, None], 128, axis=1))

    a = torch.from_numpy(block([7] * 16)).cuda().repeat(m // 16 * blocks)
    b = torch.from_numpy(block([7, -7] * 8)).cuda().repeat((n + 15) // 16 * blocks)
    acc = host(ck.gemm_w4a4_fp6c_acc_i32(a.view(-1, k // 2), b.view(-1, k // 2), m, n))
    expect = np.where(np.arange(n) % 2 == 0, 49 * k, -49 * k).astype(np.int32)
    assert np.array_equal(acc, np.broadcast_to(expect, (m, n)))


@pytest.mark.parametrize("name", ["square_3072", "up_3072_12288", "down_12288_3072"])
def test_fp6c_full_size_layer_against_oracle(ck, name):
    """The layer at full size, seed 0 (the benchmark's inputs), on compact operands, against the oracle: the
    quantisers' codes (all rows) and scales bit-exact, the int32 accumulators of the 288 x 192-tile GEMM
    bit-exact on two sampled rows of every 288-row band of tiles (all columns), and the bf16 outputs of those
    rows within 1e-2."""
    cfg = workloads.WORKLOADS[name]
    lay = workloads.make_layer(seed=0, **cfg)
    m, k, n = lay.m, lay.k, lay.n
    assert ck.gemm_fp6_tile(m, n, k) == (288, 192)
    xqc, sxc = ck.rotate_quantize_act_fp6c(dev_bf16(lay.x_bf16), 128)
    xq_ref, sx_ref = oracle.rotate_quantize_act(lay.x_bf16)
    assert np.array_equal(host(sxc).view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(fp6c_layout.decode(host(xqc), m, k), oracle.unpack_int4(xq_ref))
    wqc, wsc = ck.quantize_weight_convrot_fp6c(torch.from_numpy(lay.weights[0]).cuda(), 128)
    wp_ref, ws_ref = oracle.quantize_weight_convrot(lay.weights[0])
    assert np.array_equal(host(wsc).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(fp6c_layout.decode(host(wqc), n, k), oracle.unpack_int4(wp_ref))
    rows = _rows_per_tile_row(m, 288, 2, 13)
    acc = host(ck.gemm_w4a4_fp6c_acc_i32(xqc, wqc, m, n))
    acc_ref = oracle.gemm_acc(np.ascontiguousarray(xq_ref[rows]), wp_ref, k)
    assert np.array_equal(acc[rows], acc_ref)
    assert np.abs(acc).max() <= 49 * k
    y = bf16_host_bits(ck.w4a4_linear_fp6c(dev_bf16(lay.x_bf16), wqc, wsc))
    assert_bf16_close(y[rows], oracle.epilogue_bf16(acc_ref, sx_ref[rows], ws_ref))


# --------------------------------------------------------------------------
# Dynamic LoRA on compact operands: the up projection fused into the epilogue


@pytest.mark.parametrize("m,n,k,rank", [(1, 77, 256, 32), (33, 130, 1024, 128), (300, 200, 768, 256),
                                         (2304, 3072, 384, 64)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_fp6c_lora_epilogue_matches_int4_path_and_oracle(ck, m, n, k, rank, with_bias):
    from test_gpu_parity import _lora_atol
    import frag_layout
    xb, xq, sx, wp, ws, xc, wc = _operands(m, n, k, 5500 + m + rank)
    rng = np.random.default_rng(5510 + rank)
    t = workloads.f32_to_bf16_bits(rng.normal(0.0, 2.0, (m, rank)).astype(np.float32))
    _, b = workloads.make_lora(rng, rank, k, n)
    bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    td, bpd = dev_bf16(frag_layout.pack(t)), dev_bf16(frag_layout.pack(b))
    sxd, wsd = torch.from_numpy(sx).cuda(), torch.from_numpy(ws).cuda()
    yc = bf16_host_bits(ck.linear_w4a4_fp6c_lora(xc, sxd, wc, wsd, td, bpd, bd))
    y4 = bf16_host_bits(ck.linear_w4a4_lora(torch.from_numpy(xq).cuda(), sxd, torch.from_numpy(wp).cuda(), wsd,
                                            td, bpd, bd))
    assert np.array_equal(yc, y4)
    acc = oracle.gemm_acc(xq, wp, k)
    assert_bf16_close(yc, oracle.epilogue_lora(acc, sx, ws, t, b, bias),
                      atol=_lora_atol(acc, sx, ws, bias, t, b, rank))


def test_fp6c_lora_layer_full_size_equals_int4_path(ck):
    lay = workloads.make_layer(4608, 3072, 3072, seed=975)
    rank = 128
    a, b = workloads.make_lora(np.random.default_rng(976), rank, 3072, 3072)
    w = torch.from_numpy(lay.weights[0]).cuda()
    wp, ws = ck.quantize_weight_convrot(w, 128, 0)
    wqc, wsc = ck.quantize_weight_convrot_fp6c(w, 128)
    a_pack = ck.lora_prepare_down(torch.from_numpy(a).cuda(), 128)
    b_pack = ck.lora_prepare_up(dev_bf16(b))
    bias = torch.from_numpy(np.random.default_rng(977).standard_normal(3072).astype(np.float32)).cuda()
    x = dev_bf16(lay.x_bf16)
    y4 = bf16_host_bits(ck.w4a4_lora_linear(x, wp, ws, a_pack, b_pack, 0.5, bias, 128))
    yc = bf16_host_bits(ck.w4a4_lora_linear_fp6c(x, wqc, wsc, a_pack, b_pack, 0.5, bias, 128))
    assert np.array_equal(y4, yc)
