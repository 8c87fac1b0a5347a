"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed int4 bytes, int8 codes, fp32 scales and int32 accumulators are
bit-exact; the fp32 rotation is within 1e-6 relative (bitwise equal in
practice: both sides take the same fp32 butterflies in the same order); bf16
outputs are within 1e-2 relative of the oracle's single-rounded fp64 value and
exactly 0 where the oracle's is 0.
"""
import numpy as np
import pytest
import torch

import fp6_layout
import frag_layout
import oracle
import workloads

pytestmark = pytest.mark.gpu

ROT_CASES = [
    (64, 256, 128), (17, 384, 128), (5, 3072, 128), (3, 12288, 128), (7, 5120, 128),
    (9, 1024, 16), (9, 1024, 32), (9, 1024, 64), (9, 2048, 256), (4, 4096, 1024), (2, 16384, 128),
]
GEMM_CASES = [
    (64, 256, 256), (1, 1, 256), (3, 17, 256), (17, 3, 512), (130, 200, 768), (16, 64, 3072),
    (64, 130, 1024), (257, 129, 512), (33, 77, 256), (8, 1000, 512), (200, 8, 1280),
    # k = 128 (mod 256): the last 256-k step is a half step (skinny direct and
    # staged kernels, large kernel)
    (3, 17, 384), (64, 130, 640), (130, 200, 1152), (257, 129, 384), (20, 1000, 1152),
]


@pytest.fixture(scope="module")
def ck():
    import int4_w4a4_quantized_amd as ck
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    return ck


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_close(got_bits: np.ndarray, ref_bits: np.ndarray, rtol: float = 1e-2, atol=None) -> None:
    """|gpu - oracle| <= rtol |oracle| (+ atol where a bias add can cancel), exact zeros."""
    g = workloads.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = workloads.bf16_bits_to_f32(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(g))
    if atol is None:
        assert np.all(g[r == 0] == 0)
        atol = 0.0
    bad = np.abs(g - r) > rtol * np.abs(r) + atol
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside {rtol} rel; first at {np.argwhere(bad)[0]}"


def act(m, k, seed):
    rng = np.random.default_rng(seed)
    return workloads.make_activations(rng, m, k)


# --------------------------------------------------------------------------


def test_library_identity(ck):
    assert ck.version().startswith("ck4")


@pytest.mark.parametrize("m,k,rb", ROT_CASES)
def test_rotation_f32(ck, m, k, rb):
    xb = act(m, k, 100 + m)
    r = host(ck.rotate_act_f32(dev_bf16(xb), rb))
    ref = oracle.rotate_bf16(xb, rb)
    rel = np.abs(r.astype(np.float64) - ref) / np.maximum(np.abs(ref).max(axis=1, keepdims=True), 1e-30)
    assert rel.max() <= 1e-6
    assert np.array_equal(r, ref)  # numerically equal element by element (+0 == -0)


@pytest.mark.parametrize("m,k,rb", ROT_CASES)
@pytest.mark.parametrize("bits", [4, 8])
def test_activation_quant_bitexact(ck, m, k, rb, bits):
    xb = act(m, k, 200 + m)
    xb[0, :] = 0  # all-zero row: scale 0, codes 0
    q, s = ck.rotate_quantize_act(dev_bf16(xb), rb, bits)
    q_ref, s_ref = oracle.rotate_quantize_act(xb, rb, bits)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)
    assert host(s)[0] == 0 and not host(q)[0].any()


@pytest.mark.parametrize("n,k,rb,group", [
    (64, 256, 128, 0), (17, 384, 128, 0), (300, 3072, 128, 0), (5, 12288, 128, 0),
    (33, 1024, 64, 0), (40, 2048, 256, 0), (64, 512, 128, 128), (37, 3072, 128, 128),
    (16, 1024, 128, 16), (16, 1024, 128, 32), (16, 1024, 128, 64), (16, 1024, 128, 256), (8, 5120, 128, 128),
    (16, 1024, 128, 4), (16, 1024, 128, 8), (5, 3072, 128, 4), (9, 12288, 128, 8), (33, 256, 16, 4),
])
def test_weight_quant_bitexact(ck, n, k, rb, group):
    rng = np.random.default_rng(300 + n)
    w = workloads.make_weight(rng, n, k)
    w[1, :] = 0.0
    w[2, 5] = 3.0  # an outlier
    wp, ws = ck.quantize_weight_convrot(torch.from_numpy(w).cuda(), rb, group)
    wp_ref, ws_ref = oracle.quantize_weight_convrot(w, rb, group)
    assert np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(host(wp), wp_ref)


def _quantised_pair(m, n, k, seed):
    rng = np.random.default_rng(seed)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    xq, sx = oracle.rotate_quantize_act(xb)
    wp, ws = oracle.quantize_weight_convrot(w)
    return xb, xq, sx, wp, ws


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
def test_gemm_acc_i32_bitexact(ck, m, n, k):
    _, xq, _, wp, _ = _quantised_pair(m, n, k, 400 + m + n)
    acc = host(ck.gemm_w4a4_acc_i32(torch.from_numpy(xq).cuda(), torch.from_numpy(wp).cuda()))
    assert np.array_equal(acc, oracle.gemm_acc(xq, wp, k, bits=4))


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_w4a4(ck, m, n, k, with_bias):
    _, xq, sx, wp, ws = _quantised_pair(m, n, k, 500 + m + n)
    bias = np.random.default_rng(1).standard_normal(n).astype(np.float32) if with_bias else None
    y = ck.linear_w4a4(torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(wp).cuda(),
                       torch.from_numpy(ws).cuda(), None if bias is None else torch.from_numpy(bias).cuda())
    acc = oracle.gemm_acc(xq, wp, k)
    y_ref = oracle.epilogue_bf16(acc, sx, ws, bias)
    atol = None
    if bias is not None:
        # fp32 epilogue: a few fp32 roundings of the two summands, then bf16
        terms = np.abs(acc * sx.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]) + np.abs(bias)
        atol = 2.0 ** -21 * terms
    assert_bf16_close(bf16_host_bits(y), y_ref, atol=atol)


def test_linear_zero_rows_and_columns(ck):
    m, n, k = 40, 72, 512
    xb = act(m, k, 7)
    xb[3] = 0
    rng = np.random.default_rng(8)
    w = workloads.make_weight(rng, n, k)
    w[5] = 0
    wp, ws = oracle.quantize_weight_convrot(w)
    y = ck.w4a4_linear(dev_bf16(xb), torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda())
    yb = bf16_host_bits(y)
    assert not yb[3].any() and not yb[:, 5].any()
    assert_bf16_close(yb, oracle.linear_w4a4(xb, wp, ws))


@pytest.mark.parametrize("k", [256, 3072, 12288, 131072])
def test_accumulator_bound_is_reached_exactly(ck, k):
    # codes +7 everywhere (byte 0x77) against +7 / -7 (0x99) rows: acc = +-49 K
    m, n = 16, 8
    a = torch.full((m, k // 2), 0x77, dtype=torch.int8, device="cuda")
    b = torch.full((n, k // 2), 0x77, dtype=torch.int8, device="cuda")
    b[1::2] = torch.tensor(0x99 - 256, dtype=torch.int8)
    acc = host(ck.gemm_w4a4_acc_i32(a, b))
    expect = np.where(np.arange(n) % 2 == 0, 49 * k, -49 * k)
    assert np.array_equal(acc, np.broadcast_to(expect, (m, n)))


def test_repeatable_bitwise(ck):
    xb, xq, sx, wp, ws = _quantised_pair(512, 384, 1024, 9)
    args = [torch.from_numpy(a).cuda() for a in (xq, sx, wp, ws)]
    outs = [bf16_host_bits(ck.linear_w4a4(*args)) for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# --------------------------------------------------------------------------
# Grouped W4A8


@pytest.mark.parametrize("n,k,group", [(64, 256, 128), (1152, 512, 128), (100, 3072, 128), (48, 1024, 16),
                                       (48, 1024, 32), (48, 1024, 64), (48, 2048, 256), (48, 1024, 4),
                                       (48, 1024, 8), (7, 5120, 4)])
def test_w4a8_decode_bitexact(ck, n, k, group):
    rng = np.random.default_rng(600 + n)
    w = workloads.make_weight(rng, n, k)
    w[0] = 0
    wp, gs = oracle.quantize_weight_convrot(w, group=group)
    w8, sr = ck.dequant_w4a8_grouped(torch.from_numpy(wp).cuda(), torch.from_numpy(gs).cuda(), group)
    w8_ref, sr_ref = oracle.decode_w4a8(wp, gs, group)
    assert np.array_equal(host(sr).view(np.uint32), sr_ref.view(np.uint32))
    assert np.array_equal(host(w8), w8_ref)


def test_w4a8_decode_chunks_bitexact(ck):
    rng = np.random.default_rng(601)
    n, k = 1152, 512
    wp, gs = oracle.quantize_weight_convrot(workloads.make_weight(rng, n, k), group=128)
    wpd, gsd = torch.from_numpy(wp).cuda(), torch.from_numpy(gs).cuda()
    full8, fulls = oracle.decode_w4a8(wp, gs, 128)
    for n0 in range(0, n, 384):
        w8, sr = ck.dequant_w4a8_grouped(wpd, gsd, 128, n0, min(384, n - n0))
        assert np.array_equal(host(w8), full8[n0:n0 + 384])
        assert np.array_equal(host(sr), fulls[n0:n0 + 384])


@pytest.mark.parametrize("m,n,k,chunk", [(8, 1152, 512, 384), (8, 1152, 512, 400), (1, 1152, 512, -1),
                                         (64, 1500, 1024, 0), (100, 300, 512, 0), (16, 5120, 5120, 0),
                                         (3, 1000, 768, 0), (40, 77, 1024, 0), (1, 12288, 3072, 0),
                                         (64, 130, 384, 0),
                                         # k = 128 (mod 256) through the fused kernel's half step
                                         (1, 5000, 640, 0), (24, 333, 1152, 0), (64, 1000, 384, 0),
                                         (33, 8200, 1152, 0), (12, 8200, 640, 0)])
def test_w4a8_linear_chunked_equals_single_pass_and_oracle(ck, m, n, k, chunk):
    rng = np.random.default_rng(700 + m + n)
    xb = workloads.make_activations(rng, m, k)
    wp, gs = oracle.quantize_weight_convrot(workloads.make_weight(rng, n, k), group=128)
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    wpd, gsd = torch.from_numpy(wp).cuda(), torch.from_numpy(gs).cuda()
    y = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, 128, chunk))
    y1 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, 128, -1))
    assert np.array_equal(y, y1)
    assert_bf16_close(y, oracle.linear_w4a8_grouped(xb, wp, gs))


@pytest.mark.parametrize("group", [4, 8, 16, 64, 128])
@pytest.mark.parametrize("m", [1, 24, 64])
def test_w4a8_fused_half_step_matches_chunked(ck, m, group):
    """k = 1152, four and a half 256-k steps: the fused kernel's moved-back last window on every decode path."""
    rng = np.random.default_rng(950 + m + group)
    n, k = 333, 1152
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    w[7] = 0
    wp, gs = oracle.quantize_weight_convrot(w, group=group)
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    wpd, gsd = torch.from_numpy(wp).cuda(), torch.from_numpy(gs).cuda()
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, 0))
    yc = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, 128))
    assert np.array_equal(y0, yc)
    assert_bf16_close(y0, oracle.linear_w4a8_grouped(xb, wp, gs, group))


@pytest.mark.parametrize("group", [4, 8, 16, 64, 256])
@pytest.mark.parametrize("m", [1, 24, 64])
def test_w4a8_fused_matches_chunked_for_all_groups(ck, m, group):
    # default policy (fused kernel for m <= 64) against an explicit chunked
    # decode + int8 GEMM, with an all-zero weight row (row scale 0) and a
    # weight row whose groups all share one scale
    rng = np.random.default_rng(900 + m + group)
    n, k = 333, 1536
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    w[7] = 0
    w[11] = 0.5
    wp, gs = oracle.quantize_weight_convrot(w, group=group)
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    wpd, gsd = torch.from_numpy(wp).cuda(), torch.from_numpy(gs).cuda()
    assert ck.w4a8_workspace_bytes(m, n, k, 0) == 0
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, 0))
    yc = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, 128))
    assert np.array_equal(y0, yc)
    assert not y0[:, 7].any()
    assert_bf16_close(y0, oracle.linear_w4a8_grouped(xb, wp, gs, group))


# --------------------------------------------------------------------------
# Grouped W4A8 with E4M3 group scales


def _e4m3_weight(rng, n, k):
    w = workloads.make_weight(rng, n, k)
    w[1] = 0
    w[2] *= 1e-6      # group scales in the E4M3 subnormal range
    w[3] *= 3e4       # group scales above 448: saturate
    return w


@pytest.mark.parametrize("n,k,group", [(64, 256, 128), (40, 1024, 16), (33, 3072, 64), (20, 2048, 256),
                                       (40, 1024, 4), (40, 1024, 8)])
def test_e4m3_weight_prep_and_decode_bitexact(ck, n, k, group):
    rng = np.random.default_rng(1400 + n)
    w = _e4m3_weight(rng, n, k)
    wp, s8 = ck.quantize_weight_convrot_e4m3(torch.from_numpy(w).cuda(), 128, group)
    wp_ref, s8_ref = oracle.quantize_weight_convrot_e4m3(w, group=group)
    assert np.array_equal(host(s8), s8_ref)
    assert np.array_equal(host(wp), wp_ref)
    w8, sr = ck.dequant_w4a8_grouped(wp, s8, group)
    w8_ref, sr_ref = oracle.decode_w4a8(wp_ref, oracle.e4m3_decode(s8_ref), group)
    assert np.array_equal(host(sr).view(np.uint32), sr_ref.view(np.uint32))
    assert np.array_equal(host(w8), w8_ref)


@pytest.mark.parametrize("m,n,k", [(1, 1000, 768), (16, 5120, 5120), (64, 130, 1024), (100, 300, 512)])
def test_e4m3_linear_fused_chunked_single_equal_and_match_oracle(ck, m, n, k):
    rng = np.random.default_rng(1500 + m)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    wp_ref, s8_ref = oracle.quantize_weight_convrot_e4m3(w)
    wpd, s8d = torch.from_numpy(wp_ref).cuda(), torch.from_numpy(s8_ref).cuda()
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, s8d, 128, 0))
    y1 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, s8d, 128, -1))
    yc = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, s8d, 128, 256))
    assert np.array_equal(y0, y1) and np.array_equal(y0, yc)
    assert_bf16_close(y0, oracle.linear_w4a8_grouped_e4m3(xb, wp_ref, s8_ref))


# --------------------------------------------------------------------------
# The FP6 operand path (int4 codes as FP6 E2M3 q / 8 on the f8f6f4 matrix cores)

FP6_CASES = [
    (64, 256, 256), (1, 1, 128), (3, 17, 384), (17, 3, 512), (130, 200, 768), (16, 64, 3072),
    (64, 130, 1024), (257, 129, 640), (33, 77, 256), (8, 1000, 512), (300, 8, 1280), (577, 385, 1152),
    # shapes the launcher sends to the 288 x 192 tile (the benchmarked one):
    # ragged in m and n, an odd number of 128-k steps, and whole tiles
    (2000, 3500, 384), (2304, 3072, 256),
]


@pytest.mark.parametrize("m,k,rb", [(64, 256, 128), (17, 384, 128), (5, 3072, 128), (3, 12288, 128),
                                    (9, 1024, 16), (9, 2048, 256), (2, 16384, 128),
                                    # row counts divisible by 4 (images gathered in LDS), up to k = 4096
                                    (20, 384, 128), (8, 2048, 64), (36, 4096, 128), (132, 3072, 128),
                                    (4, 128, 16)])
def test_fp6_activation_codes_bitexact(ck, m, k, rb):
    xb = act(m, k, 2000 + m + k)
    xb[0] = 0                          # an all-zero row: scale 0, codes 0
    q6, sx = ck.rotate_quantize_act_fp6(dev_bf16(xb), rb)
    q_ref, s_ref = oracle.rotate_quantize_act(xb, rb, 4)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(fp6_layout.decode(host(q6), m, k), oracle.unpack_int4(q_ref))


@pytest.mark.parametrize("n,k,rb", [(64, 256, 128), (300, 3072, 128), (5, 12288, 128), (33, 1024, 64)])
def test_fp6_weight_codes_bitexact(ck, n, k, rb):
    rng = np.random.default_rng(2100 + n)
    w = workloads.make_weight(rng, n, k)
    w[1] = 0
    w[2, 5] = 3.0
    q6, ws = ck.quantize_weight_convrot_fp6(torch.from_numpy(w).cuda(), rb)
    wp_ref, ws_ref = oracle.quantize_weight_convrot(w, rb, 0)
    assert np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(fp6_layout.decode(host(q6), n, k), oracle.unpack_int4(wp_ref))


def _fp6_operands(ck, m, n, k, seed):
    """Oracle codes and scales, and the same codes uploaded in the FP6 layout."""
    rng = np.random.default_rng(seed)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    xq, sx = oracle.rotate_quantize_act(xb, 128, 4)
    wp, ws = oracle.quantize_weight_convrot(w, 128, 0)
    xq6 = torch.from_numpy(fp6_layout.encode(oracle.unpack_int4(xq)).reshape(-1, k * 3 // 4)).cuda()
    wq6 = torch.from_numpy(fp6_layout.encode(oracle.unpack_int4(wp)).reshape(-1, k * 3 // 4)).cuda()
    return xb, xq, sx, wp, ws, xq6, wq6


@pytest.mark.parametrize("m,n,k", FP6_CASES)
def test_fp6_gemm_acc_i32_bitexact(ck, m, n, k):
    _, xq, _, wp, _, xq6, wq6 = _fp6_operands(ck, m, n, k, 2200 + m + n)
    acc = host(ck.gemm_w4a4_fp6_acc_i32(xq6, wq6, m, n))
    assert np.array_equal(acc, oracle.gemm_acc(xq, wp, k, bits=4))


@pytest.mark.parametrize("m,n,k", FP6_CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_fp6_linear_matches_int4_path_and_oracle(ck, m, n, k, with_bias):
    xb, xq, sx, wp, ws, xq6, wq6 = _fp6_operands(ck, m, n, k, 2300 + m + n)
    bias = np.random.default_rng(2301).normal(0, 0.1, n).astype(np.float32) if with_bias else None
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    sxd, wsd = torch.from_numpy(sx).cuda(), torch.from_numpy(ws).cuda()
    y6 = bf16_host_bits(ck.linear_w4a4_fp6(xq6, sxd, wq6, wsd, bd))
    if k >= 256:
        # the int8-MFMA kernel on the same codes gives the same bits
        y4 = bf16_host_bits(ck.linear_w4a4(torch.from_numpy(xq).cuda(), sxd, torch.from_numpy(wp).cuda(), wsd, bd))
        assert np.array_equal(y6, y4)
    acc = oracle.gemm_acc(xq, wp, k, bits=4)
    ref = oracle.epilogue_bf16(acc, sx, ws, bias)
    atol = None
    if bias is not None:
        terms = np.abs(acc * sx.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]) + np.abs(bias)
        atol = 2.0 ** -21 * terms
    assert_bf16_close(y6, ref, atol=atol)


@pytest.mark.parametrize("m,n,k", [(4600, 3000, 1024), (4100, 2900, 512), (2000, 1500, 1536), (1000, 700, 768)])
def test_fp6_ragged_large_equals_int4_path(ck, m, n, k):
    """Ragged edges on both tile sizes of the FP6 GEMM, against the int4 path (itself pinned to the oracle)."""
    rng = np.random.default_rng(3100 + m)
    xb = workloads.make_activations(rng, m, k)
    w = torch.from_numpy(workloads.make_weight(rng, n, k)).cuda()
    bias = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    x = dev_bf16(xb)
    wp, ws = ck.quantize_weight_convrot(w, 128, 0)
    wq6, ws6 = ck.quantize_weight_convrot_fp6(w, 128)
    xq, sx = ck.rotate_quantize_act(x, 128, 4)
    xq6, sx6 = ck.rotate_quantize_act_fp6(x, 128)
    ldy = (n + 7) // 8 * 8 + 4          # rows 8-byte but not 16-byte aligned
    y4 = torch.full((m, ldy), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    y6 = y4.clone()
    ck.linear_w4a4(xq, sx, wp, ws, bias, out=y4[:, :n])
    ck.linear_w4a4_fp6(xq6, sx6, wq6, ws6, bias, out=y6[:, :n])
    assert np.array_equal(bf16_host_bits(y4), bf16_host_bits(y6))
    assert (bf16_host_bits(y6)[:, n:] == 0xFFFF).all()   # nothing written past n
    assert torch.equal(ck.gemm_w4a4_acc_i32(xq, wp), ck.gemm_w4a4_fp6_acc_i32(xq6, wq6, m, n))


@pytest.mark.parametrize("name", ["square_3072", "up_3072_12288", "down_12288_3072"])
def test_fp6_full_size_layer_equals_int4_path(ck, name):
    # the whole layer at full size through both paths, from the same bf16
    # input and fp32 weight: FP6 quantisers + FP6 GEMM against the int4
    # quantisers + int8-MFMA GEMM, bit for bit; the int4 path is pinned to
    # the oracle by test_full_size_layer
    cfg = workloads.WORKLOADS[name]
    lay = workloads.make_layer(cfg["m"], cfg["k"], cfg["n"], seed=7)
    x = dev_bf16(lay.x_bf16)
    w = torch.from_numpy(lay.weights[0]).cuda()
    wq6, ws6 = ck.quantize_weight_convrot_fp6(w, 128)
    wp, ws = ck.quantize_weight_convrot(w, 128, 0)
    assert torch.equal(ws6, ws)
    y6 = bf16_host_bits(ck.w4a4_linear_fp6(x, wq6, ws6))
    y4 = bf16_host_bits(ck.w4a4_linear(x, wp, ws))
    assert np.array_equal(y6, y4)


def _fp6_uniform_block(row_codes) -> np.ndarray:
    """One 1536-byte FP6 operand block (16 rows x 128 k) whose row i holds the code row_codes[i] at every k."""
    q = np.repeat(np.asarray(row_codes, np.int64)[:, None], 128, axis=1)
    return fp6_layout.encode(q)


@pytest.mark.parametrize("k", [128, 3072, 12288, 131072])
@pytest.mark.parametrize("m,n,tile", [(16, 8, (96, 128)), (2304, 3072, (288, 192))])
def test_fp6_accumulator_bound_is_reached_exactly(ck, m, n, tile, k):
    """Codes +7 everywhere against rows of +7 and -7 give acc = +-49 K exactly on both tiles of the FP6 GEMM,
    up to the largest k it accepts ([PR #63] Description: |acc| <= 49 K; the fp32 accumulator of the FP6 matrix
    instruction holds 49 K / 64 exactly for K <= 131072)."""
    assert ck.gemm_fp6_tile(m, n, k) == tile
    blocks = k // 128
    a = torch.from_numpy(_fp6_uniform_block([7] * 16)).cuda().repeat(m // 16 * blocks)
    b = torch.from_numpy(_fp6_uniform_block([7, -7] * 8)).cuda().repeat((n + 15) // 16 * blocks)
    acc = host(ck.gemm_w4a4_fp6_acc_i32(a.view(-1, k * 3 // 4), b.view(-1, k * 3 // 4), m, n))
    expect = np.where(np.arange(n) % 2 == 0, 49 * k, -49 * k).astype(np.int32)
    assert np.array_equal(acc, np.broadcast_to(expect, (m, n)))


def _rows_per_tile_row(m, bm, per_tile, seed):
    """Sample rows so that each bm-row band of output tiles holds `per_tile` of them, plus the first and last."""
    rng = np.random.default_rng(seed)
    rows = [0, m - 1]
    for r0 in range(0, m, bm):
        span = min(bm, m - r0)
        rows.extend(r0 + rng.choice(span, min(per_tile, span), replace=False))
    return np.unique(np.asarray(rows))


@pytest.mark.parametrize("name", ["square_3072", "up_3072_12288", "down_12288_3072"])
def test_fp6_full_size_layer_against_oracle(ck, name):
    """The benchmarked path at full size, seed 0 (the benchmark's inputs), directly against the oracle: the FP6
    quantisers' codes (all rows, decoded from the operand layout) and scales bit-exact, the int32 accumulators of
    the 288 x 192-tile FP6 GEMM bit-exact on two sampled rows of every 288-row band of tiles (all columns), and
    the bf16 outputs of those rows within 1e-2."""
    cfg = workloads.WORKLOADS[name]
    lay = workloads.make_layer(seed=0, **cfg)
    m, k, n = lay.m, lay.k, lay.n
    assert ck.gemm_fp6_tile(m, n, k) == (288, 192)
    xq6, sx6 = ck.rotate_quantize_act_fp6(dev_bf16(lay.x_bf16), 128)
    xq_ref, sx_ref = oracle.rotate_quantize_act(lay.x_bf16)
    assert np.array_equal(host(sx6).view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(fp6_layout.decode(host(xq6), m, k), oracle.unpack_int4(xq_ref))
    wq6, ws6 = ck.quantize_weight_convrot_fp6(torch.from_numpy(lay.weights[0]).cuda(), 128)
    wp_ref, ws_ref = oracle.quantize_weight_convrot(lay.weights[0])
    assert np.array_equal(host(ws6).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(fp6_layout.decode(host(wq6), n, k), oracle.unpack_int4(wp_ref))
    rows = _rows_per_tile_row(m, 288, 2, 11)
    acc = host(ck.gemm_w4a4_fp6_acc_i32(xq6, wq6, m, n))
    acc_ref = oracle.gemm_acc(np.ascontiguousarray(xq_ref[rows]), wp_ref, k)
    assert np.array_equal(acc[rows], acc_ref)
    assert np.abs(acc).max() <= 49 * k
    y = bf16_host_bits(ck.linear_w4a4_fp6(xq6, sx6, wq6, ws6))
    assert_bf16_close(y[rows], oracle.epilogue_bf16(acc_ref, sx_ref[rows], ws_ref))


# --------------------------------------------------------------------------
# Grouped W4A8 with a frozen 16-entry codebook

# an unordered table with a repeated entry, a zero and an asymmetric range
CB_ODD = np.array([0.9, -0.2, 0.05, 0.5, -1.3, 0.0, 0.3, -0.6, 1.1, -0.05, 0.7, 0.5, -0.9, 0.15, -0.35, 0.2],
                  np.float32)


def _codebooks():
    return {"normal": workloads.make_codebook(), "odd": CB_ODD}


@pytest.mark.parametrize("cbname", ["normal", "odd"])
@pytest.mark.parametrize("e4m3", [False, True])
@pytest.mark.parametrize("n,k,group", [(64, 256, 128), (40, 1024, 4), (40, 1024, 8), (33, 3072, 16),
                                       (17, 2048, 64), (9, 12288, 256)])
def test_codebook_weight_prep_and_decode_bitexact(ck, cbname, e4m3, n, k, group):
    cb = _codebooks()[cbname]
    rng = np.random.default_rng(1600 + n + group)
    w = _e4m3_weight(rng, n, k) if e4m3 else workloads.make_weight(rng, n, k)
    w[0] = 0
    wp, gs = ck.quantize_weight_convrot_codebook(torch.from_numpy(w).cuda(), cb, 128, group, e4m3)
    wp_ref, gs_ref = oracle.quantize_weight_convrot_codebook(w, cb, group=group, e4m3=e4m3)
    assert np.array_equal(host(gs).view(np.uint8), gs_ref.view(np.uint8))
    assert np.array_equal(host(wp), wp_ref)
    w8, sr = ck.dequant_w4a8_grouped(wp, gs, group, codebook=cb)
    w8_ref, sr_ref = oracle.decode_w4a8_codebook(wp_ref, gs_ref, cb, group)
    assert np.array_equal(host(sr).view(np.uint32), sr_ref.view(np.uint32))
    assert np.array_equal(host(w8), w8_ref)
    # a chunk of rows decodes to the same bits
    n0, nc = n // 3, n - n // 3
    w8c, src = ck.dequant_w4a8_grouped(wp, gs, group, n0, nc, codebook=cb)
    assert np.array_equal(host(w8c), w8_ref[n0:]) and np.array_equal(host(src), sr_ref[n0:])


@pytest.mark.parametrize("cbname", ["normal", "odd"])
@pytest.mark.parametrize("e4m3", [False, True])
@pytest.mark.parametrize("m,n,k,group", [(1, 1000, 768, 128), (16, 333, 1536, 4), (24, 333, 1536, 8),
                                         (64, 130, 1024, 32), (40, 77, 1024, 256), (100, 300, 512, 64)])
def test_codebook_linear_paths_equal_and_match_oracle(ck, cbname, e4m3, m, n, k, group):
    cb = _codebooks()[cbname]
    rng = np.random.default_rng(1700 + m + group)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    w[7] = 0
    wp_ref, gs_ref = oracle.quantize_weight_convrot_codebook(w, cb, group=group, e4m3=e4m3)
    wpd, gsd = torch.from_numpy(wp_ref).cuda(), torch.from_numpy(gs_ref).cuda()
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, 0, codebook=cb))
    y1 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, -1, codebook=cb))
    yc = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wpd, gsd, group, 128, codebook=cb))
    assert np.array_equal(y0, y1) and np.array_equal(y0, yc)
    assert not y0[:, 7].any()
    assert_bf16_close(y0, oracle.linear_w4a8_codebook(xb, wp_ref, gs_ref, cb, group))


def test_codebook_skinny_full_size(ck):
    # decode shape at full size: N=12288, K=3072, one token, group 128, through
    # the fused kernel (default policy) and the single-pass decode; the oracle
    # checks a sample of output columns through the decoded int8 weight.
    cb = workloads.make_codebook()
    rng = np.random.default_rng(1800)
    n, k = 12288, 3072
    xb = workloads.make_activations(rng, 1, k)
    w = workloads.make_weight(rng, n, k)
    wp, gs = ck.quantize_weight_convrot_codebook(torch.from_numpy(w).cuda(), cb, 128, 128)
    wp_ref, gs_ref = oracle.quantize_weight_convrot_codebook(w, cb, group=128)
    assert np.array_equal(host(wp), wp_ref) and np.array_equal(host(gs), gs_ref)
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wp, gs, 128, 0, codebook=cb))
    y1 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wp, gs, 128, -1, codebook=cb))
    assert np.array_equal(y0, y1)
    cols = np.random.default_rng(1801).choice(n, 256, replace=False)
    cols.sort()
    ref = oracle.linear_w4a8_codebook(xb, wp_ref[cols], gs_ref[cols], cb, 128)
    assert_bf16_close(y0[:, cols], ref)


# --------------------------------------------------------------------------
# Stochastic-rounding weight requantisation


@pytest.mark.parametrize("n,k,group", [(64, 256, 0), (257, 3072, 0), (33, 1024, 128), (12, 4096, 64), (5, 12288, 0),
                                       (33, 1024, 4), (12, 2048, 8)])
def test_sr_weight_quant_bitexact(ck, n, k, group):
    rng = np.random.default_rng(1200 + n)
    w = workloads.make_weight(rng, n, k)
    w[2] = 0
    u = rng.random((n, k), dtype=np.float32)
    u[0, :8] = [0.0, 0.5, 0.99999994, 0.25, 0.0, 0.75, 0.5, 0.0]
    wp, ws = ck.quantize_weight_convrot_sr(torch.from_numpy(w).cuda(), torch.from_numpy(u).cuda(), 128, group)
    wp_ref, ws_ref = oracle.quantize_weight_convrot_sr(w, u, group=group)
    assert np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(host(wp), wp_ref)


def test_sr_weight_quant_row_stride(ck):
    rng = np.random.default_rng(1300)
    n, k = 40, 768
    w = workloads.make_weight(rng, n, k)
    u_wide = rng.random((n, k + 64), dtype=np.float32)
    wp, ws = ck.quantize_weight_convrot_sr(torch.from_numpy(w).cuda(), torch.from_numpy(u_wide).cuda()[:, :k])
    wp_ref, ws_ref = oracle.quantize_weight_convrot_sr(w, np.ascontiguousarray(u_wide[:, :k]))
    assert np.array_equal(host(wp), wp_ref)


# --------------------------------------------------------------------------
# W8A8 rowwise ConvRot linear


@pytest.mark.parametrize("n,k,rb", [(64, 256, 128), (257, 3072, 128), (40, 1024, 64), (9, 4096, 256), (3, 12288, 128)])
def test_w8_weight_quant_bitexact(ck, n, k, rb):
    rng = np.random.default_rng(1000 + n)
    w = workloads.make_weight(rng, n, k)
    w[1] = 0
    wq, ws = ck.quantize_weight_convrot_int8(torch.from_numpy(w).cuda(), rb)
    wq_ref, ws_ref = oracle.quantize_weight_convrot_int8(w, rb)
    assert np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(host(wq), wq_ref)


@pytest.mark.parametrize("m,n,k", [(64, 256, 256), (130, 200, 768), (1, 77, 512), (16, 1000, 3072), (300, 96, 384)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a8_linear(ck, m, n, k, with_bias):
    rng = np.random.default_rng(1100 + m + n)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
    w8, ws = oracle.quantize_weight_convrot_int8(w)
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    y = bf16_host_bits(ck.w8a8_linear(dev_bf16(xb), torch.from_numpy(w8).cuda(), torch.from_numpy(ws).cuda(), bd))
    ref = oracle.linear_w8a8(xb, w8, ws, bias)
    if bias is None:
        assert_bf16_close(y, ref)
    else:
        assert_bf16_close(y, ref, atol=2.0 ** -21 * k)


def test_w8a8_full_size_square_layer(ck):
    lay = workloads.make_layer(seed=0, **workloads.WORKLOADS["square_3072"])
    m, k = lay.m, lay.k
    w8, ws = ck.quantize_weight_convrot_int8(torch.from_numpy(lay.weights[0]).cuda())
    w8_ref, ws_ref = oracle.quantize_weight_convrot_int8(lay.weights[0])
    assert np.array_equal(host(w8), w8_ref) and np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
    y = bf16_host_bits(ck.w8a8_linear(dev_bf16(lay.x_bf16), w8, ws))
    rows = _sample_rows(m, 30, 2)
    xq_ref, sx_ref = oracle.rotate_quantize_act(np.ascontiguousarray(lay.x_bf16[rows]), bits=8)
    acc_ref = oracle.gemm_acc(xq_ref, w8_ref, k, bits=8)
    assert_bf16_close(y[rows], oracle.epilogue_bf16(acc_ref, sx_ref, ws_ref))


# --------------------------------------------------------------------------
# Full-size layers, in the launch configuration the benchmark times


def _sample_rows(m, count, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, count, replace=False)]))
    return rows


@pytest.mark.parametrize("name", ["square_3072", "up_3072_12288", "down_12288_3072", "qkv_3x3072"])
def test_full_size_layer(ck, name):
    cfg = workloads.WORKLOADS[name]
    lay = workloads.make_layer(seed=0, **cfg)
    m, k, n = lay.m, lay.k, lay.n
    xd = dev_bf16(lay.x_bf16)
    xq, sx = ck.rotate_quantize_act(xd, 128, 4)
    xq_ref, sx_ref = oracle.rotate_quantize_act(lay.x_bf16)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(host(xq), xq_ref)
    rows = _sample_rows(m, 30, 1)
    for w in lay.weights:
        wp, ws = ck.quantize_weight_convrot(torch.from_numpy(w).cuda(), 128, 0)
        wp_ref, ws_ref = oracle.quantize_weight_convrot(w)
        assert np.array_equal(host(ws).view(np.uint32), ws_ref.view(np.uint32))
        assert np.array_equal(host(wp), wp_ref)
        y = bf16_host_bits(ck.linear_w4a4(xq, sx, wp, ws))
        acc = host(ck.gemm_w4a4_acc_i32(xq, wp))
        acc_ref = oracle.gemm_acc(np.ascontiguousarray(xq_ref[rows]), wp_ref, k)
        assert np.array_equal(acc[rows], acc_ref)
        assert np.abs(acc).max() <= 49 * k
        assert_bf16_close(y[rows], oracle.epilogue_bf16(acc_ref, sx_ref[rows], ws_ref))


@pytest.mark.parametrize("m,n,k", [(1, 12288, 3072), (2, 5120, 5120), (1, 77, 256), (2, 1000, 8192), (1, 17, 384),
                                   (2, 8200, 1152), (2, 16400, 640), (2, 5, 4096), (1, 3, 2048), (1, 8200, 16384),
                                   (2, 300, 16256), (1, 2000, 12288)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_gemv_equals_mfma_skinny_kernel(ck, m, n, k, with_bias):
    """m <= 2: linear_w4a4 runs the matrix-vector kernel (one or two weight rows per wavefront: n > 8192 or
    not; 1-4 and 8 chunks per lane and row; ragged n and k); the K-split MFMA kernel, reached through the LoRA
    epilogue with t = 0 (bias present or not, as the plain call), must give the same bits, and both stay
    within the oracle's bf16 bound."""
    _, xq, sx, wp, ws = _quantised_pair(m, n, k, 5300 + m + n + k)
    bias = np.random.default_rng(5301).standard_normal(n).astype(np.float32) if with_bias else None
    d = [torch.from_numpy(v).cuda() for v in (xq, sx, wp, ws)]
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    y = bf16_host_bits(ck.linear_w4a4(*d, bd))
    t0 = torch.zeros((frag_layout.rows16(m), 32), dtype=torch.bfloat16, device="cuda")
    b0 = torch.zeros((frag_layout.rows16(n), 32), dtype=torch.bfloat16, device="cuda")
    y_mfma = bf16_host_bits(ck.linear_w4a4_lora(*d, t0, b0, bd))
    if bias is not None:
        assert np.array_equal(y, y_mfma)
    else:
        # without a bias the LoRA epilogue adds + 0 to every value, which turns -0 into +0
        assert np.array_equal(workloads.bf16_bits_to_f32(y), workloads.bf16_bits_to_f32(y_mfma))
    acc = oracle.gemm_acc(xq, wp, k)
    atol = None
    if bias is not None:
        atol = 2.0 ** -21 * (np.abs(acc * sx.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]) +
                             np.abs(bias))
    assert_bf16_close(y, oracle.epilogue_bf16(acc, sx, ws, bias), atol=atol)


# --------------------------------------------------------------------------
# The whole layer from bf16 in one call (one kernel for m <= 2)


LAYER_CASES = [
    # one kernel (m <= 2, k <= 8192): 4, 2 and 1 weight rows per wavefront (n >= 10177, >= 5089,
    # less), 1-4 chunks per lane and row, ragged n and k (a row ending in a partial 1 KB chunk); the
    # last row all zero, tiny (scale below 2^-120) or one 128-block of 1e36 (scale above 2^120)
    (1, 12288, 3072, None), (2, 12288, 3072, "zero"), (1, 5120, 5120, None), (2, 5120, 5120, "huge"),
    (2, 77, 256, "tiny"), (1, 17, 384, None), (2, 8200, 8192, "tiny"), (1, 16400, 1152, None),
    (2, 10300, 6144, "huge"), (2, 999, 640, "zero"), (2, 12345, 2176, "tiny"), (1, 3, 1280, None),
    # quantiser + GEMM: m > 2 or k > 8192
    (3, 5120, 5120, None), (4, 12288, 3072, None), (4, 17, 384, None), (4, 1000, 4096, None),
    (3, 8200, 8192, None), (5, 300, 768, None), (17, 1000, 1024, None), (1, 8200, 16384, None),
    (2, 5100, 16256, "huge"),
]


@pytest.mark.parametrize("m,n,k,special", LAYER_CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_w4a4_bf16_equals_two_calls_and_oracle(ck, m, n, k, special, with_bias):
    """The one-call layer gives the bits of rotate_quantize_act + linear_w4a4 (y, and the x_q and
    x_scales it returns), including all-zero rows and rows whose scale leaves [2^-120, 2^120]
    (the exact-divide path: a tiny row, and a row of one constant 128-block of 1e36: s = 1.6e36, and
    |acc| <= 49 keeps the fp32 epilogue finite),
    and y stays within the oracle's bf16 bound (not checked on tiny rows, whose outputs fall
    among fp32 subnormals, where the epilogue's two roundings are not within 1e-2)."""
    rng = np.random.default_rng(5100 + m + n + k)
    xb = workloads.make_activations(rng, m, k)
    tiny_rows = []

    def make(row, kind):
        if kind == "zero":
            xb[row] = 0
        elif kind == "tiny":
            xb[row] = workloads.f32_to_bf16_bits(rng.standard_normal(k).astype(np.float32) * np.float32(1e-37))
            tiny_rows.append(row)
        elif kind == "huge":
            xb[row] = 0
            xb[row, :128] = workloads.f32_to_bf16_bits(np.full(128, 1e36, dtype=np.float32))

    if special is not None:
        make(m - 1, special)
    elif m >= 4:
        make(1, "zero")
        make(2, "tiny")
        make(3, "huge")
    w = workloads.make_weight(rng, n, k)
    wp, ws = oracle.quantize_weight_convrot(w)
    bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
    xd = dev_bf16(xb)
    wpd, wsd = torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda()
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    y, xq, sx = ck.linear_w4a4_bf16(xd, wpd, wsd, bd)
    xq2, sx2 = ck.rotate_quantize_act(xd, 128, 4)
    y2 = ck.linear_w4a4(xq2, sx2, wpd, wsd, bd)
    assert np.array_equal(host(xq), host(xq2))
    assert np.array_equal(host(sx).view(np.uint32), host(sx2).view(np.uint32))
    assert np.array_equal(bf16_host_bits(y), bf16_host_bits(y2))
    q_ref, s_ref = oracle.rotate_quantize_act(xb)
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
    if m * n * k <= 4 * 8200 * 4096:
        acc = oracle.gemm_acc(q_ref, wp, k)
        ref = oracle.epilogue_bf16(acc, s_ref, ws, bias)
        atol = None
        if bias is not None:
            terms = np.abs(acc * s_ref.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]) + np.abs(bias)
            atol = 2.0 ** -21 * terms
        rows = [i for i in range(m) if i not in tiny_rows]
        assert_bf16_close(bf16_host_bits(y)[rows], ref[rows], atol=None if atol is None else atol[rows])


W4A8_LAYER_CASES = [
    # one kernel (m = 1, n <= 8192, k <= 8192, groups >= 32): 1-4 chunks per lane and row, ragged n and
    # k, fp32 and E4M3 group scales; the row all zero, tiny or one 128-block of 1e36
    (1, 5120, 5120, 128, False, None), (1, 5120, 5120, 64, True, "zero"), (1, 8192, 3072, 128, False, None),
    (1, 77, 256, 32, False, "tiny"), (1, 17, 384, 128, True, None), (1, 8200, 8192, 256, False, "huge"),
    (1, 999, 1152, 128, True, "huge"), (1, 3, 2176, 128, False, None), (1, 4100, 6144, 1024, False, "tiny"),
    # quantiser + W4A8 linear: m > 1, groups below 32, k > 8192, n > 8192
    (2, 5120, 5120, 64, True, "zero"), (2, 999, 1152, 128, False, "huge"), (3, 1000, 1024, 128, False, None),
    (1, 500, 1024, 16, False, None), (1, 300, 12288, 128, True, None), (1, 12288, 3072, 128, True, None),
    (17, 640, 768, 64, False, None),
]


@pytest.mark.parametrize("m,n,k,group,e4m3,special", W4A8_LAYER_CASES)
def test_linear_w4a8_bf16_equals_two_calls_and_oracle(ck, m, n, k, group, e4m3, special):
    """The one-call grouped W4A8 layer gives the bits of rotate_quantize_act(bits=8) + linear_w4a8_grouped
    (y, and the x_q8 and x_scales it returns), with all-zero rows, rows whose scale leaves [2^-120, 2^120]
    (the exact-divide path) and an all-zero weight row, and y stays within the oracle's bf16 bound (tiny
    rows excluded, as in the W4A4 layer test)."""
    rng = np.random.default_rng(5500 + m + n + k + group)
    xb = workloads.make_activations(rng, m, k)
    tiny_rows = []
    r = m - 1
    if special == "zero":
        xb[r] = 0
    elif special == "tiny":
        xb[r] = workloads.f32_to_bf16_bits(rng.standard_normal(k).astype(np.float32) * np.float32(1e-37))
        tiny_rows.append(r)
    elif special == "huge":
        xb[r] = 0
        xb[r, :128] = workloads.f32_to_bf16_bits(np.full(128, 1e36, dtype=np.float32))
    w = workloads.make_weight(rng, n, k)
    w[0] = 0
    wd = torch.from_numpy(w).cuda()
    wp, gs = (ck.quantize_weight_convrot_e4m3 if e4m3 else ck.quantize_weight_convrot)(wd, 128, group)
    xd = dev_bf16(xb)
    y, xq8, sx = ck.linear_w4a8_grouped_bf16(xd, wp, gs, group)
    xq2, sx2 = ck.rotate_quantize_act(xd, 128, 8)
    y2 = ck.linear_w4a8_grouped(xq2, sx2, wp, gs, group, 0)
    assert np.array_equal(host(xq8), host(xq2))
    assert np.array_equal(host(sx).view(np.uint32), host(sx2).view(np.uint32))
    assert np.array_equal(bf16_host_bits(y), bf16_host_bits(y2))
    assert not bf16_host_bits(y)[:, 0].any()
    q_ref, s_ref = oracle.rotate_quantize_act(xb, bits=8)
    assert np.array_equal(host(xq8), q_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
    if m * n * k <= 4 * 8200 * 4096 and special != "huge":
        if e4m3:
            ref = oracle.linear_w4a8_grouped_e4m3(xb, host(wp), host(gs).view(np.uint8), group)
        else:
            ref = oracle.linear_w4a8_grouped(xb, host(wp), host(gs), group)
        rows = [i for i in range(m) if i not in tiny_rows]
        assert_bf16_close(bf16_host_bits(y)[rows], ref[rows])


def test_linear_w4a8_bf16_reused_buffers_and_graph(ck):
    """Caller buffers are used and overwritten (two calls in a row, the second with fewer rows of another
    activation), and the one-call W4A8 layer replays inside a captured graph with the same bits each time."""
    rng = np.random.default_rng(5600)
    n, k, group = 3000, 1024, 128
    wp, gs = ck.quantize_weight_convrot(torch.from_numpy(workloads.make_weight(rng, n, k)).cuda(), 128, group)
    xq = torch.full((4, k), 0x5A, dtype=torch.int8, device="cuda")
    sx = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    y = torch.full((4, n), 1.0, dtype=torch.bfloat16, device="cuda")
    for m in (2, 1):
        xd = dev_bf16(workloads.make_activations(rng, m, k))
        ck.linear_w4a8_grouped_bf16(xd, wp, gs, group, x_q8=xq[:m], x_scales=sx[:m], out=y[:m])
        assert ck.w4a8_workspace_bytes(m, n, k, 0) == 0
        xq2, sx2 = ck.rotate_quantize_act(xd, 128, 8)
        y2 = ck.linear_w4a8_grouped(xq2, sx2, wp, gs, group, 0)
        assert np.array_equal(host(xq[:m]), host(xq2))
        assert np.array_equal(host(sx[:m]).view(np.uint32), host(sx2).view(np.uint32))
        assert np.array_equal(bf16_host_bits(y[:m]), bf16_host_bits(y2))
    xd = dev_bf16(workloads.make_activations(rng, 1, k))
    ref = bf16_host_bits(ck.linear_w4a8_grouped_bf16(xd, wp, gs, group)[0])
    yg = torch.empty((1, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ck.linear_w4a8_grouped_bf16(xd, wp, gs, group, x_q8=xq[:1], x_scales=sx[:1], out=yg)
    for _ in range(3):
        yg.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_host_bits(yg), ref)


def test_linear_w4a4_bf16_reused_buffers(ck):
    """Caller buffers are used and overwritten: two calls in a row into the same x_q, x_scales and y, the
    second with fewer rows of a different activation, each equal to the two-call path."""
    rng = np.random.default_rng(5200)
    n, k = 3000, 1024
    wp, ws = oracle.quantize_weight_convrot(workloads.make_weight(rng, n, k))
    wpd, wsd = torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda()
    xq = torch.full((4, k // 2), 0x5A, dtype=torch.int8, device="cuda")
    sx = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    y = torch.full((4, n), 1.0, dtype=torch.bfloat16, device="cuda")
    for m in (4, 2):
        xd = dev_bf16(workloads.make_activations(rng, m, k))
        ck.linear_w4a4_bf16(xd, wpd, wsd, None, x_q=xq[:m], x_scales=sx[:m], out=y[:m])
        xq2, sx2 = ck.rotate_quantize_act(xd, 128, 4)
        y2 = ck.linear_w4a4(xq2, sx2, wpd, wsd)
        assert np.array_equal(host(xq[:m]), host(xq2))
        assert np.array_equal(host(sx[:m]).view(np.uint32), host(sx2).view(np.uint32))
        assert np.array_equal(bf16_host_bits(y[:m]), bf16_host_bits(y2))


@pytest.mark.parametrize("m,n,k", [(17, 12288, 640), (40, 8200, 384), (64, 8200, 1152), (8, 12288, 1152),
                                   (17, 12288, 3072), (32, 12288, 3072), (33, 8200, 768), (48, 8200, 1280),
                                   (64, 16384, 512), (40, 12288, 256), (24, 8200, 2304), (5, 12288, 3072),
                                   (8, 8200, 768), (16, 12288, 1280)])
def test_skinny_shared_activation_kernel(ck, m, n, k):
    """4 < m <= 64 with at least 512 weight tiles of 16 rows: the kernel whose waves split N over one LDS copy of
    the activation (ragged N leaves a wave with no rows; k = 256 is a single step, k = 128 (mod 256) ends in a half step). It must give the bits of the
    K-split kernel, reached through the LoRA epilogue with t = 0 (bias present, so no -0 can meet the + 0), and
    stay within the oracle's bf16 bound."""
    _, xq, sx, wp, ws = _quantised_pair(m, n, k, 3300 + m)
    bias = np.random.default_rng(3301).standard_normal(n).astype(np.float32)
    d = [torch.from_numpy(v).cuda() for v in (xq, sx, wp, ws)]
    bd = torch.from_numpy(bias).cuda()
    y = bf16_host_bits(ck.linear_w4a4(*d, bd))
    t0 = torch.zeros((frag_layout.rows16(m), 32), dtype=torch.bfloat16, device="cuda")
    b0 = torch.zeros((frag_layout.rows16(n), 32), dtype=torch.bfloat16, device="cuda")
    y_ksplit = bf16_host_bits(ck.linear_w4a4_lora(*d, t0, b0, bd))
    assert np.array_equal(y, y_ksplit)
    acc = oracle.gemm_acc(xq, wp, k)
    # fp32 epilogue: a few fp32 roundings of the two summands, then bf16 (as test_linear_w4a4)
    terms = np.abs(acc * sx.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]) + np.abs(bias)
    assert_bf16_close(y, oracle.epilogue_bf16(acc, sx, ws, bias), atol=2.0 ** -21 * terms)


@pytest.mark.parametrize("m,n,k,group,e4m3", [(17, 12288, 3072, 128, False), (32, 12288, 1024, 64, True),
                                               (33, 12300, 3072, 128, False), (64, 12288, 3072, 256, True),
                                               (48, 16000, 2048, 128, False), (64, 12296, 256, 128, False),
                                               (40, 12288, 4096, 64, False)])
def test_w4a8_fused_wide_n_equals_decode_path(ck, m, n, k, group, e4m3):
    """16 < m <= 64 at large and ragged N (k = 256 is a single step): the fused W4A8 kernel must give the bits of
    one decode pass + the int8 GEMM, and stay within the oracle's bf16 bound."""
    rng = np.random.default_rng(3500 + m + group)
    xb = workloads.make_activations(rng, m, k)
    w = torch.from_numpy(workloads.make_weight(rng, n, k)).cuda()
    if e4m3:
        wp, gs = ck.quantize_weight_convrot_e4m3(w, 128, group)
    else:
        wp, gs = ck.quantize_weight_convrot(w, 128, group)
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wp, gs, group, 0))
    y1 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wp, gs, group, -1))
    assert np.array_equal(y0, y1)
    if e4m3:
        ref = oracle.linear_w4a8_grouped_e4m3(xb, host(wp), host(gs).view(np.uint8), group)
    else:
        ref = oracle.linear_w4a8_grouped(xb, host(wp), host(gs), group)
    assert_bf16_close(y0, ref)


@pytest.mark.parametrize("m,n,k,group,e4m3", [(1, 8192, 3072, 128, False), (2, 5120, 5120, 64, True),
                                               (1, 77, 256, 32, False), (1, 8000, 8192, 256, False),
                                               (1, 17, 384, 128, True), (2, 4000, 1152, 32, False),
                                               (1, 1000, 4096, 1024, True), (1, 3, 640, 128, False),
                                               (2, 4100, 2176, 128, True), (2, 8192, 5120, 512, False),
                                               # just outside the kernel's shapes: the MFMA fused kernel
                                               (2, 8193, 1024, 128, False), (3, 100, 1024, 128, True),
                                               (1, 100, 1024, 16, False), (2, 300, 6144, 128, False)])
def test_w4a8_gemv_equals_decode_path(ck, m, n, k, group, e4m3):
    """m <= 2, n <= 8192, groups of 32 codes or more: the matrix-vector W4A8 kernel (1-4 chunks per lane and row,
    ragged n and k, fp32 and E4M3 scales, an all-zero weight row and one whose groups share a scale) must give the
    bits of one decode pass + the int8 GEMM, and stay within the oracle's bf16 bound."""
    rng = np.random.default_rng(3700 + m + n + group)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    w[0] = 0
    w[min(1, n - 1)] = 0.5
    wd = torch.from_numpy(w).cuda()
    if e4m3:
        wp, gs = ck.quantize_weight_convrot_e4m3(wd, 128, group)
    else:
        wp, gs = ck.quantize_weight_convrot(wd, 128, group)
    xq8, sx = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    assert ck.w4a8_workspace_bytes(m, n, k, 0) == 0
    y0 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wp, gs, group, 0))
    y1 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx, wp, gs, group, -1))
    assert np.array_equal(y0, y1)
    assert not y0[:, 0].any()
    if e4m3:
        ref = oracle.linear_w4a8_grouped_e4m3(xb, host(wp), host(gs).view(np.uint8), group)
    else:
        ref = oracle.linear_w4a8_grouped(xb, host(wp), host(gs), group)
    assert_bf16_close(y0, ref)


def test_random_shapes_kernel_variants_agree(ck):
    """Seeded random shapes through the kernel choices that must give the same bits: the N-split skinny kernel
    against the K-split one (through its LoRA epilogue with t = 0), and the FP6 GEMM (either tile) against the
    int4 GEMM, with a bias, on device-quantised operands."""
    rng = np.random.default_rng(4242)
    for _ in range(8):
        m = int(rng.integers(5, 65))
        n = int(rng.integers(2048, 5000)) * 4
        k = 128 * int(rng.integers(2, 25))
        x = dev_bf16(workloads.make_activations(rng, m, k))
        w = torch.from_numpy(workloads.make_weight(rng, n, k)).cuda()
        bias = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
        wp, ws = ck.quantize_weight_convrot(w, 128, 0)
        xq, sx = ck.rotate_quantize_act(x, 128, 4)
        t0 = torch.zeros((frag_layout.rows16(m), 32), dtype=torch.bfloat16, device="cuda")
        b0 = torch.zeros((frag_layout.rows16(n), 32), dtype=torch.bfloat16, device="cuda")
        y = bf16_host_bits(ck.linear_w4a4(xq, sx, wp, ws, bias))
        assert np.array_equal(y, bf16_host_bits(ck.linear_w4a4_lora(xq, sx, wp, ws, t0, b0, bias))), (m, n, k)
    for _ in range(8):
        m = int(rng.integers(65, 3000))
        n = int(rng.integers(16, 1000)) * 4
        k = 128 * int(rng.integers(2, 17))
        x = dev_bf16(workloads.make_activations(rng, m, k))
        w = torch.from_numpy(workloads.make_weight(rng, n, k)).cuda()
        bias = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
        wp, ws = ck.quantize_weight_convrot(w, 128, 0)
        wq6, ws6 = ck.quantize_weight_convrot_fp6(w, 128)
        xq, sx = ck.rotate_quantize_act(x, 128, 4)
        xq6, sx6 = ck.rotate_quantize_act_fp6(x, 128)
        y4 = bf16_host_bits(ck.linear_w4a4(xq, sx, wp, ws, bias))
        y6 = bf16_host_bits(ck.linear_w4a4_fp6(xq6, sx6, wq6, ws6, bias))
        assert np.array_equal(y4, y6), (m, n, k)


@pytest.mark.parametrize("m", [1, 8, 16, 64])
@pytest.mark.parametrize("n,k", [(12288, 3072), (5120, 5120)])
def test_skinny_layers(ck, m, n, k):
    rng = np.random.default_rng(800 + m)
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    wp, ws = oracle.quantize_weight_convrot(w)
    y = bf16_host_bits(ck.w4a4_linear(dev_bf16(xb), torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda()))
    assert_bf16_close(y, oracle.linear_w4a4(xb, wp, ws))
    wpg, gs = oracle.quantize_weight_convrot(w, group=128)
    xq8, sx8 = ck.rotate_quantize_act(dev_bf16(xb), 128, 8)
    y8 = bf16_host_bits(ck.linear_w4a8_grouped(xq8, sx8, torch.from_numpy(wpg).cuda(), torch.from_numpy(gs).cuda()))
    assert_bf16_close(y8, oracle.linear_w4a8_grouped(xb, wpg, gs))


# --------------------------------------------------------------------------
# Dynamic LoRA: rotated down projection, up projection fused in the epilogue.
# Bars: A R is bit-exact (same fp32 rotation, one RNE rounding). t is within
# one bf16 rounding step (2^-7 relative) of the oracle's, plus the fp32
# accumulation bound (K + 16) 2^-24 alpha sum |bf16(xR)| |A R|, plus the
# elements of x R that may round to a different bf16 on the two sides: the
# kernel accumulates x H on the matrix cores, the oracle with butterflies,
# both in fp32, so an element whose exact value lies within the fp32 error
# bound (b + 2) 2^-24 sum_block |x| / sqrt(b) of a bf16 rounding boundary may
# round either way; each such element adds its two roundings' distance times
# |A R|. y is within the suite's 1e-2 relative plus the fp32 epilogue's
# rounding of both summands (the fp32 base value, 2^-21 of it, and the
# rank + 8 fp32 additions of the LoRA sum).


def f64_of(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("rank,k,rb", [(32, 256, 128), (64, 3072, 128), (128, 1024, 16), (256, 2048, 256),
                                       (32, 16384, 128), (64, 512, 64), (128, 512, 32)])
def test_lora_prepare_down_bitexact(ck, rank, k, rb):
    a, _ = workloads.make_lora(np.random.default_rng(900 + rank + k), rank, k, 1)
    got = bf16_host_bits(ck.lora_prepare_down(torch.from_numpy(a).cuda(), rb))
    assert np.array_equal(frag_layout.unpack(got, rank), oracle.lora_prepare_down(a, rb))


@pytest.mark.parametrize("n,rank", [(1, 32), (40, 64), (3072, 128), (1000, 256), (17, 32)])
def test_lora_prepare_up_is_fragment_order(ck, n, rank):
    rng = np.random.default_rng(905 + n)
    wide = workloads.f32_to_bf16_bits(rng.standard_normal((n, rank + 8)).astype(np.float32))
    got = bf16_host_bits(ck.lora_prepare_up(dev_bf16(wide)[:, :rank]))
    assert np.array_equal(got, frag_layout.pack(np.ascontiguousarray(wide[:, :rank])))


def _lora_down_dev(ck, xd, a_rot, alpha, rb, m):
    """Runs the device down projection from the oracle's A R (packed on the host); returns t [m, rank]."""
    t_pack = ck.lora_down(xd, dev_bf16(frag_layout.pack(a_rot)), alpha, rb)
    return frag_layout.unpack(bf16_host_bits(t_pack), m)


def _t_atol(xb, a_rot, alpha, rb):
    x = f64_of(xb)
    m, k = x.shape
    exact = oracle.rotate_f64(x, rb)
    blk = np.abs(x).reshape(m, k // rb, rb).sum(axis=2, keepdims=True)
    e = np.broadcast_to((rb + 2) * 2.0 ** -24 * blk / np.sqrt(rb) * 1.01, (m, k // rb, rb)).reshape(m, k)
    step = np.abs(f64_of(oracle.to_bf16(exact + e)) - f64_of(oracle.to_bf16(exact - e)))
    ar = np.abs(f64_of(a_rot)).T
    xr = np.abs(f64_of(oracle.to_bf16(oracle.rotate_bf16(xb, rb)))) + step
    return abs(alpha) * ((k + 16) * 2.0 ** -24 * (xr @ ar) + step @ ar)


def _assert_t_close(got_bits, ref_bits, atol):
    g, r = f64_of(got_bits), f64_of(ref_bits)
    bad = np.abs(g - r) > 2.0 ** -7 * 1.01 * np.abs(r) + 1.01 * atol
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside; first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("m,k,rb,rank", [(1, 256, 128, 32), (16, 3072, 128, 64), (17, 1024, 16, 128),
                                         (33, 2048, 256, 256), (100, 512, 64, 32), (130, 384, 128, 64),
                                         (5, 16384, 128, 128), (64, 5120, 128, 128), (47, 1280, 32, 256)])
def test_lora_down(ck, m, k, rb, rank):
    rng = np.random.default_rng(910 + m + rank)
    xb = workloads.make_activations(rng, m, k)
    xb[m // 2] = 0
    a, _ = workloads.make_lora(rng, rank, k, 1)
    a_rot = oracle.lora_prepare_down(a, rb)
    alpha = 0.625
    t = _lora_down_dev(ck, dev_bf16(xb), a_rot, alpha, rb, m)
    assert not f64_of(t[m // 2]).any()
    _assert_t_close(t, oracle.lora_down(xb, a_rot, alpha, rb), _t_atol(xb, a_rot, alpha, rb))


def test_lora_down_row_stride(ck):
    m, k, rank = 40, 1024, 64
    rng = np.random.default_rng(919)
    wide = workloads.make_activations(rng, m, k + 256)
    a, _ = workloads.make_lora(rng, rank, k, 1)
    a_rot = oracle.lora_prepare_down(a)
    t = _lora_down_dev(ck, dev_bf16(wide)[:, :k], a_rot, 1.0, 128, m)
    xb = np.ascontiguousarray(wide[:, :k])
    _assert_t_close(t, oracle.lora_down(xb, a_rot, 1.0), _t_atol(xb, a_rot, 1.0, 128))


def _lora_atol(acc, sx, ws, bias, t_bits, b_bits, rank):
    base = np.abs(acc.astype(np.float64) * sx.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :])
    if bias is not None:
        base = base + np.abs(bias.astype(np.float64))[None, :]
    lora = np.abs(f64_of(t_bits)) @ np.abs(f64_of(b_bits)).T
    return 2.0 ** -21 * base + (rank + 8) * 2.0 ** -24 * (base + lora)


@pytest.mark.parametrize("m,n,k,rank", [(1, 77, 256, 32), (16, 300, 512, 64), (33, 130, 1024, 128),
                                        (16, 300, 640, 64), (130, 257, 384, 32), (64, 1000, 768, 256), (65, 200, 512, 32), (130, 257, 768, 64),
                                        (300, 96, 1280, 128), (1000, 520, 512, 256)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_w4a4_lora_epilogue(ck, m, n, k, rank, with_bias):
    _, xq, sx, wp, ws = _quantised_pair(m, n, k, 920 + m + n)
    rng = np.random.default_rng(930 + rank)
    t = workloads.f32_to_bf16_bits(rng.normal(0.0, 2.0, (m, rank)).astype(np.float32))
    _, b = workloads.make_lora(rng, rank, k, n)
    bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
    y = ck.linear_w4a4_lora(torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(wp).cuda(),
                            torch.from_numpy(ws).cuda(), dev_bf16(frag_layout.pack(t)), dev_bf16(frag_layout.pack(b)),
                            None if bias is None else torch.from_numpy(bias).cuda())
    acc = oracle.gemm_acc(xq, wp, k)
    y_ref = oracle.epilogue_lora(acc, sx, ws, t, b, bias)
    assert_bf16_close(bf16_host_bits(y), y_ref, atol=_lora_atol(acc, sx, ws, bias, t, b, rank))


@pytest.mark.parametrize("m,n,k", [(8, 300, 512), (500, 200, 768)])
def test_lora_with_zero_t_is_plain_linear_bitwise(ck, m, n, k):
    _, xq, sx, wp, ws = _quantised_pair(m, n, k, 940 + m)
    _, b = workloads.make_lora(np.random.default_rng(941), 64, k, n)
    bias = np.random.default_rng(942).standard_normal(n).astype(np.float32)
    dq = [torch.from_numpy(v).cuda() for v in (xq, sx, wp, ws)]
    bd = torch.from_numpy(bias).cuda()
    y0 = bf16_host_bits(ck.linear_w4a4(*dq, bd))
    t0 = torch.zeros((frag_layout.rows16(m), 64), dtype=torch.bfloat16, device="cuda")
    y1 = bf16_host_bits(ck.linear_w4a4_lora(*dq, t0, dev_bf16(frag_layout.pack(b)), bd))
    assert np.array_equal(y0, y1)


@pytest.mark.parametrize("m,n,k,rank,rb", [(1, 3072, 3072, 128, 128), (64, 512, 1024, 64, 64),
                                           (200, 384, 2048, 32, 256), (97, 1000, 512, 256, 16)])
def test_w4a4_lora_layer_end_to_end(ck, m, n, k, rank, rb):
    lay = workloads.make_layer(m, k, n, seed=950 + m)
    a, b = workloads.make_lora(np.random.default_rng(951 + m), rank, k, n)
    alpha = 0.5
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0], rb)
    a_rot = oracle.lora_prepare_down(a, rb)
    y = ck.w4a4_lora_linear(dev_bf16(lay.x_bf16), torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda(),
                            dev_bf16(frag_layout.pack(a_rot)), ck.lora_prepare_up(dev_bf16(b)), alpha, None, rb)
    y_ref = oracle.linear_w4a4_lora(lay.x_bf16, wp, ws, a_rot, b, alpha, g=rb)
    xq, sx = oracle.rotate_quantize_act(lay.x_bf16, rb)
    acc = oracle.gemm_acc(xq, wp, k)
    t_ref = oracle.lora_down(lay.x_bf16, a_rot, alpha, rb)
    # t may differ from the oracle's by its own bound; carry that through B
    dt = 2.0 ** -7 * 1.01 * np.abs(f64_of(t_ref)) + 1.01 * _t_atol(lay.x_bf16, a_rot, alpha, rb)
    atol = _lora_atol(acc, sx, ws, None, t_ref, b, rank) + dt @ np.abs(f64_of(b)).T
    assert_bf16_close(bf16_host_bits(y), y_ref, atol=atol)


@pytest.mark.parametrize("m,n,k,rank,rb", [(200, 384, 2048, 32, 256), (97, 1000, 512, 256, 16),
                                           (4608, 3072, 3072, 128, 128)])
def test_w4a4_lora_layer_fp6_equals_int4_path(ck, m, n, k, rank, rb):
    lay = workloads.make_layer(m, k, n, seed=970 + m)
    a, b = workloads.make_lora(np.random.default_rng(971 + m), rank, k, n)
    w = torch.from_numpy(lay.weights[0]).cuda()
    wp, ws = ck.quantize_weight_convrot(w, rb, 0)
    wq6, ws6 = ck.quantize_weight_convrot_fp6(w, rb)
    a_pack = ck.lora_prepare_down(torch.from_numpy(a).cuda(), rb)
    b_pack = ck.lora_prepare_up(dev_bf16(b))
    bias = torch.from_numpy(np.random.default_rng(972).standard_normal(n).astype(np.float32)).cuda()
    x = dev_bf16(lay.x_bf16)
    y4 = bf16_host_bits(ck.w4a4_lora_linear(x, wp, ws, a_pack, b_pack, 0.5, bias, rb))
    y6 = bf16_host_bits(ck.w4a4_lora_linear_fp6(x, wq6, ws6, a_pack, b_pack, 0.5, bias, rb))
    assert np.array_equal(y4, y6)


def test_full_size_square_layer_with_lora(ck):
    cfg = workloads.WORKLOADS["square_3072"]
    lay = workloads.make_layer(seed=0, **cfg)
    m, k, n = lay.m, lay.k, lay.n
    rank, alpha = 128, 0.5
    a, b = workloads.make_lora(np.random.default_rng(960), rank, k, n)
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0])
    a_rot = oracle.lora_prepare_down(a)
    a_rot_d = ck.lora_prepare_down(torch.from_numpy(a).cuda())
    assert np.array_equal(frag_layout.unpack(bf16_host_bits(a_rot_d), rank), a_rot)
    xd = dev_bf16(lay.x_bf16)
    xq, sx = ck.rotate_quantize_act(xd, 128, 4)
    t = ck.lora_down(xd, a_rot_d, alpha)
    y = bf16_host_bits(ck.linear_w4a4_lora(xq, sx, torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda(), t,
                                           ck.lora_prepare_up(dev_bf16(b))))
    t_all = frag_layout.unpack(bf16_host_bits(t), m)
    rows = _sample_rows(m, 30, 2)
    xr = np.ascontiguousarray(lay.x_bf16[rows])
    t_ref = oracle.lora_down(xr, a_rot, alpha)
    _assert_t_close(t_all[rows], t_ref, _t_atol(xr, a_rot, alpha, 128))
    xq_ref, sx_ref = oracle.rotate_quantize_act(xr)
    acc = oracle.gemm_acc(xq_ref, wp, k)
    # the up projection is checked on the device's own t
    t_dev = t_all[rows]
    y_ref = oracle.epilogue_lora(acc, sx_ref, ws, t_dev, b)
    assert_bf16_close(y[rows], y_ref, atol=_lora_atol(acc, sx_ref, ws, None, t_dev, b, rank))



@pytest.mark.parametrize("m,n,k,rank", [(1, 77, 256, 32), (16, 300, 512, 64), (33, 130, 1024, 128),
                                         (300, 200, 768, 256), (97, 1000, 384, 32)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_fp6_lora_epilogue_matches_int4_path_and_oracle(ck, m, n, k, rank, with_bias):
    xb, xq, sx, wp, ws, xq6, wq6 = _fp6_operands(ck, m, n, k, 2400 + m + rank)
    rng = np.random.default_rng(2410 + rank)
    t = workloads.f32_to_bf16_bits(rng.normal(0.0, 2.0, (m, rank)).astype(np.float32))
    _, b = workloads.make_lora(rng, rank, k, n)
    bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    td, bpd = dev_bf16(frag_layout.pack(t)), dev_bf16(frag_layout.pack(b))
    sxd, wsd = torch.from_numpy(sx).cuda(), torch.from_numpy(ws).cuda()
    y6 = bf16_host_bits(ck.linear_w4a4_fp6_lora(xq6, sxd, wq6, wsd, td, bpd, bd))
    if k >= 256:
        y4 = bf16_host_bits(ck.linear_w4a4_lora(torch.from_numpy(xq).cuda(), sxd, torch.from_numpy(wp).cuda(), wsd,
                                                td, bpd, bd))
        assert np.array_equal(y6, y4)
    acc = oracle.gemm_acc(xq, wp, k)
    assert_bf16_close(y6, oracle.epilogue_lora(acc, sx, ws, t, b, bias),
                      atol=_lora_atol(acc, sx, ws, bias, t, b, rank))


# --------------------------------------------------------------------------
# Graph capture: every path launches only kernels (no memset or allocation
# nodes), so a captured graph replays to the eager result, bit for bit, on
# every replay, with unrelated eager work and synchronisations in between.


def test_graph_replays_match_eager(ck):
    m, n, k, rank = 200, 520, 1024, 64
    lay = workloads.make_layer(m, k, n, seed=970)
    a, b = workloads.make_lora(np.random.default_rng(971), rank, k, n)
    xd = dev_bf16(lay.x_bf16)
    wd = torch.from_numpy(lay.weights[0]).cuda()
    wp, ws = ck.quantize_weight_convrot(wd, 128, 0)
    wg, gs = ck.quantize_weight_convrot(wd, 128, 128)
    a_pack = ck.lora_prepare_down(torch.from_numpy(a).cuda())
    b_pack = ck.lora_prepare_up(dev_bf16(b))
    xs = xd[:8]  # a skinny batch for the fused W4A8 kernel
    xq = torch.empty((m, k // 2), dtype=torch.int8, device="cuda")
    sx = torch.empty((m,), dtype=torch.float32, device="cuda")
    xq8 = torch.empty((8, k), dtype=torch.int8, device="cuda")
    sx8 = torch.empty((8,), dtype=torch.float32, device="cuda")
    t = torch.empty((frag_layout.rows16(m), rank), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    yl = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y8 = torch.empty((8, n), dtype=torch.bfloat16, device="cuda")
    y8c = torch.empty((8, 528), dtype=torch.bfloat16, device="cuda")[:, :n]  # the chunked path needs ldy % 16 == 0
    wsp = torch.empty((ck.w4a8_workspace_bytes(8, n, k, 256),), dtype=torch.uint8, device="cuda")
    # the FP6 operand path, plain and with the LoRA epilogue
    wq6, ws6 = ck.quantize_weight_convrot_fp6(wd, 128)
    xq6 = torch.zeros((frag_layout.rows16(m), k * 3 // 4), dtype=torch.uint8, device="cuda")  # padding rows stay 0
    sx6 = torch.empty((m,), dtype=torch.float32, device="cuda")
    y6 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y6l = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    # and on compact FP6 operands
    wqc, wsc = ck.quantize_weight_convrot_fp6c(wd, 128)
    xqc = torch.zeros((frag_layout.rows16(m), k // 2), dtype=torch.uint8, device="cuda")  # padding rows stay 0
    sxc = torch.empty((m,), dtype=torch.float32, device="cuda")
    yc = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ycl = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    # the N-split skinny kernel (16 < m <= 64, at least 512 weight tiles)
    ns, ms = 8192, 40
    wsk, wssk = ck.quantize_weight_convrot(
        torch.from_numpy(workloads.make_weight(np.random.default_rng(972), ns, k)).cuda(), 128, 0)
    ysk = torch.empty((ms, ns), dtype=torch.bfloat16, device="cuda")
    # the one-call layer's fused kernel (m <= 4)
    xq1 = torch.empty((3, k // 2), dtype=torch.int8, device="cuda")
    sx1 = torch.empty((3,), dtype=torch.float32, device="cuda")
    y1 = torch.empty((3, n), dtype=torch.bfloat16, device="cuda")

    def step():
        ck.rotate_quantize_act(xd, 128, 4, out=xq, scales=sx)
        ck.linear_w4a4(xq, sx, wp, ws, None, out=y)
        ck.lora_down(xd, a_pack, 0.5, 128, out=t)
        ck.linear_w4a4_lora(xq, sx, wp, ws, t, b_pack, None, out=yl)
        ck.rotate_quantize_act(xs, 128, 8, out=xq8, scales=sx8)
        ck.linear_w4a8_grouped(xq8, sx8, wg, gs, 128, 0, out=y8)
        ck.linear_w4a8_grouped(xq8, sx8, wg, gs, 128, 256, out=y8c, workspace=wsp)
        ck.rotate_quantize_act_fp6(xd, 128, out=xq6, scales=sx6)
        ck.linear_w4a4_fp6(xq6, sx6, wq6, ws6, None, out=y6)
        ck.linear_w4a4_fp6_lora(xq6, sx6, wq6, ws6, t, b_pack, None, out=y6l)
        ck.rotate_quantize_act_fp6c(xd, 128, out=xqc, scales=sxc)
        ck.linear_w4a4_fp6c(xqc, sxc, wqc, wsc, None, out=yc)
        ck.linear_w4a4_fp6c_lora(xqc, sxc, wqc, wsc, t, b_pack, None, out=ycl)
        ck.linear_w4a4(xq[:ms], sx[:ms], wsk, wssk, None, out=ysk)
        ck.linear_w4a4_bf16(xd[:3], wp, ws, None, x_q=xq1, x_scales=sx1, out=y1)

    outs = (xq, sx, t, y, yl, y8, y8c, xq6, sx6, y6, y6l, xqc, sxc, yc, ycl, ysk, xq1, sx1, y1)
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    # the three operand forms give the same bits, with and without the LoRA term
    assert torch.equal(yc.view(torch.int16), y.view(torch.int16)) and torch.equal(y6.view(torch.int16), y.view(torch.int16))
    assert torch.equal(ycl.view(torch.int16), yl.view(torch.int16)) and torch.equal(y6l.view(torch.int16), yl.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.zero_()
        junk = torch.randn(4096, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {rep} differs"
        del junk
