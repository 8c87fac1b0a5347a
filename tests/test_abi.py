"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function that include/ck4.h declares, and
reject invalid or unsupported arguments with the documented status before it
touches a device.
"""
import ctypes
import os
import re

import numpy as np

import pytest

import int4_w4a4_quantized_amd as ck
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ck4.h")

FAKE = ctypes.c_void_p(1 << 20)      # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p((1 << 20) + 4)  # misaligned
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ck4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ck.LIB_PATH):
        pytest.fail("libck4.so is not built: run __graft_entry__.build()")
    return ck.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(ck.SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(L):
    assert L.ck4_version().decode().startswith("ck4 ")
    assert L.ck4_status_string(0) == b"ok"
    assert L.ck4_status_string(1) == b"invalid argument"
    assert L.ck4_status_string(2) == b"unsupported shape or option"
    assert L.ck4_status_string(3) == b"device error"


def last(L):
    return L.ck4_last_error().decode()


def test_linear_validation(L):
    f = L.ck4_linear_w4a4
    assert f(NULL, FAKE, FAKE, FAKE, NULL, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID
    assert "null" in last(L)
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 0, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 256, FAKE, 4, NULL) == ck.CK4_ERR_INVALID  # ldy < n
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 256, FAKE, 10, NULL) == ck.CK4_ERR_INVALID  # ldy % 4
    assert f(ODD, FAKE, FAKE, FAKE, NULL, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID  # alignment
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 192, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 128
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 128, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED  # k < 256
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 262144, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED  # k too big
    g = L.ck4_gemm_w4a4_acc_i32
    assert g(FAKE, FAKE, 8, 8, 256, ODD, 8, NULL) == ck.CK4_ERR_INVALID


def test_rotate_validation(L):
    f = L.ck4_rotate_quantize_act
    assert f(FAKE, 4, 256, 256, 128, 5, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # bits
    assert f(FAKE, 4, 256, 256, 96, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # rot_block
    assert f(FAKE, 4, 256, 256, 8, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED
    assert f(FAKE, 4, 384, 384, 256, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % rot_block
    assert f(FAKE, 4, 32768, 32768, 128, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k > 16384
    assert f(FAKE, 4, 256, 200, 128, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID  # ldx < k
    assert f(ODD, 4, 256, 256, 128, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, -1, 256, 256, 128, 4, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    r = L.ck4_rotate_act_f32
    assert r(FAKE, 4, 256, 256, 128, NULL, NULL) == ck.CK4_ERR_INVALID
    sr = L.ck4_quantize_weight_convrot_sr
    assert sr(FAKE, 4, 256, 256, 128, 0, NULL, 256, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID  # u null
    assert sr(FAKE, 4, 256, 256, 128, 0, ODD, 256, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID  # u alignment
    assert sr(FAKE, 4, 256, 256, 128, 0, FAKE, 200, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID  # ldu < k
    assert sr(FAKE, 4, 256, 256, 128, 48, FAKE, 256, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # group
    w8 = L.ck4_quantize_weight_convrot_int8
    assert w8(FAKE, 4, 256, 256, 128, NULL, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert w8(FAKE, 4, 256, 256, 128, ODD, FAKE, NULL) == ck.CK4_ERR_INVALID  # w_q8 alignment
    assert w8(FAKE, 4, 384, 384, 256, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % rot_block
    w = L.ck4_quantize_weight_convrot
    assert w(FAKE, 4, 256, 256, 128, 48, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # group
    assert w(FAKE, 4, 256, 256, 128, 512, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # group > k
    assert w(FAKE, 4, 256, 250, 128, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID


def test_w4a8_validation(L):
    d = L.ck4_dequant_w4a8_grouped
    assert d(FAKE, FAKE, 64, 256, 128, 32, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID  # n0 + nc > n
    assert d(FAKE, FAKE, 64, 256, 100, 0, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED
    f = L.ck4_linear_w4a8_grouped
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 64, 256, 128, FAKE, 64, 128, NULL, 0, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 64, 256, 128, FAKE, 64, -1, NULL, 0, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 64, 200, 128, FAKE, 64, 0, FAKE, 1 << 20, NULL) == ck.CK4_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 64, 256, 128, FAKE, 64, 24, FAKE, 1 << 20, NULL) == ck.CK4_ERR_INVALID
    e = L.ck4_quantize_weight_convrot_e4m3
    assert e(FAKE, 4, 256, 256, 128, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # group 0 has no group scales
    assert e(FAKE, 4, 256, 256, 128, 128, FAKE, NULL, NULL) == ck.CK4_ERR_INVALID
    de = L.ck4_dequant_w4a8_grouped_e4m3
    assert de(FAKE, FAKE, 64, 256, 128, 32, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    fe = L.ck4_linear_w4a8_grouped_e4m3
    assert fe(FAKE, FAKE, FAKE, FAKE, 8, 64, 200, 128, FAKE, 64, 0, FAKE, 1 << 20, NULL) == ck.CK4_ERR_UNSUPPORTED
    l8 = L.ck4_linear_w8a8
    assert l8(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 192, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED


def test_fp6_validation_and_layout_helper(L):
    f = L.ck4_rotate_quantize_act_fp6
    assert f(FAKE, 4, 320, 320, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 128
    assert f(NULL, 4, 256, 256, 128, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, 4, 256, 256, 128, ODD, FAKE, NULL) == ck.CK4_ERR_INVALID       # q6 alignment
    w = L.ck4_quantize_weight_convrot_fp6
    assert w(FAKE, 4, 256, 200, 128, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID      # ldw < k
    g = L.ck4_linear_w4a4_fp6
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 320, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 128
    assert g(ODD, FAKE, FAKE, FAKE, NULL, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID
    a = L.ck4_gemm_w4a4_fp6_acc_i32
    assert a(FAKE, FAKE, 8, 8, 256, ODD, 8, NULL) == ck.CK4_ERR_INVALID
    assert L.ck4_fp6_bytes(17, 256) == 32 * 192 and L.ck4_fp6_bytes(16, 100) == 0
    import fp6_layout
    # worked example: codes 1, -1, 7, -7 are FP6 codes 0x01, 0x21, 0x07, 0x27,
    # packed LSB first into 24 bits: 0x9C7841
    q = np.zeros((16, 128), np.int64)
    q[0, :4] = [1, -1, 7, -7]
    b = fp6_layout.encode(q)
    assert b[:3].tolist() == [0x41, 0x78, 0x9C] and not b[3:].any()
    # row 5, k 40 (k group 1, field 8) lands in image 16 + 5 at bit 48
    q2 = np.zeros((16, 128), np.int64)
    q2[5, 40] = -3
    b2 = fp6_layout.encode(q2)
    assert np.flatnonzero(b2).tolist() == [21 * 24 + 6] and b2[21 * 24 + 6] == 0x23


def test_fp6c_validation_and_layout_helper(L):
    f = L.ck4_rotate_quantize_act_fp6c
    assert f(FAKE, 4, 320, 320, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 128
    assert f(NULL, 4, 256, 256, 128, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, 4, 256, 256, 128, ODD, FAKE, NULL) == ck.CK4_ERR_INVALID       # q6c alignment
    w = L.ck4_quantize_weight_convrot_fp6c
    assert w(FAKE, 4, 256, 200, 128, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID      # ldw < k
    g = L.ck4_linear_w4a4_fp6c
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 8, 8, 320, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 128
    assert g(ODD, FAKE, FAKE, FAKE, NULL, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID
    a = L.ck4_gemm_w4a4_fp6c_acc_i32
    assert a(FAKE, FAKE, 8, 8, 256, ODD, 8, NULL) == ck.CK4_ERR_INVALID
    assert L.ck4_fp6c_bytes(17, 256) == 32 * 128 and L.ck4_fp6c_bytes(16, 100) == 0
    import fp6c_layout
    # worked examples from the definition: codes 1, -1, 7, -7 (FP6 0x9C7841 in
    # V0) keep V0 as it is; code -5 at t = 6 (0x25 at bits 36-41 of W: V1 =
    # 0x250) splits V1 into V1 & Z0 = 0x210 in D0 and V1 & Z2 = 0x040 in D1
    q = np.zeros((16, 128), np.int64)
    q[0, :4] = [1, -1, 7, -7]
    b = fp6c_layout.encode(q)
    assert b.size == 1024 and b[:3].tolist() == [0x41, 0x78, 0x9C] and not b[3:].any()
    q2 = np.zeros((16, 128), np.int64)
    q2[0, 6] = -5
    b2 = fp6c_layout.encode(q2)
    assert b2[:8].tolist() == [0x10, 0x02, 0, 0, 0x40, 0, 0, 0] and not b2[8:].any()
    # the codes of t = 16-31 take the image's second 8 bytes; row 5, k 40 (image
    # 16 + 5, t = 8: 0x23 at bits 16-21 of V1) splits into D0 bits 16, 21 and D1 bit 17
    q3 = np.zeros((16, 128), np.int64)
    q3[0, 16] = 3
    q3[5, 40] = -3
    b3 = fp6c_layout.encode(q3)
    assert np.flatnonzero(b3).tolist() == [8, 21 * 16 + 2, 21 * 16 + 6]
    assert b3[[8, 21 * 16 + 2, 21 * 16 + 6]].tolist() == [0x03, 0x21, 0x02]
    # the masks are disjoint and the map is a bijection on every code at every place
    assert int(fp6c_layout.Z0) & int(fp6c_layout.Z2) == 0
    rng = np.random.default_rng(5)
    for rows, k in [(16, 128), (33, 384), (5, 1024)]:
        qr = rng.integers(-7, 8, size=(rows, k))
        qr[0, :32] = np.arange(-15, 17) % 15 - 7
        assert np.array_equal(fp6c_layout.decode(fp6c_layout.encode(qr), rows, k), qr)
    for t in range(32):
        for v in range(-7, 8):
            qq = np.zeros((16, 128), np.int64)
            qq[3, t] = v
            assert np.array_equal(fp6c_layout.decode(fp6c_layout.encode(qq), 16, 128), qq)


def test_codebook_validation(L):
    cb = (ctypes.c_float * 16)(*[float(i - 8) / 8 for i in range(16)])
    zero = (ctypes.c_float * 16)()
    bad = (ctypes.c_float * 16)(*([0.5] * 15 + [float("nan")]))
    q = L.ck4_quantize_weight_convrot_codebook
    assert q(FAKE, 4, 256, 256, 128, 128, NULL, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert "codebook" in last(L)
    assert q(FAKE, 4, 256, 256, 128, 128, zero, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert q(FAKE, 4, 256, 256, 128, 128, bad, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert "not finite" in last(L)
    assert q(FAKE, 4, 256, 256, 128, 2, cb, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # group < 4
    assert q(FAKE, 4, 256, 256, 128, 0, cb, 0, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # no group scales
    odd2 = ctypes.c_void_p((1 << 20) + 2)
    assert q(FAKE, 4, 256, 256, 128, 128, cb, 0, FAKE, odd2, NULL) == ck.CK4_ERR_INVALID   # fp32 scales misaligned
    d = L.ck4_dequant_w4a8_codebook
    assert d(FAKE, FAKE, 0, NULL, 64, 256, 128, 0, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert d(FAKE, FAKE, 0, cb, 64, 256, 128, 32, 64, FAKE, FAKE, NULL) == ck.CK4_ERR_INVALID  # n0 + nc > n
    f = L.ck4_linear_w4a8_codebook
    assert f(FAKE, FAKE, FAKE, FAKE, 0, zero, 8, 64, 256, 128, FAKE, 64, 0, FAKE, 1 << 20, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 0, cb, 8, 64, 256, 2, FAKE, 64, 0, FAKE, 1 << 20, NULL) == ck.CK4_ERR_UNSUPPORTED
    w = L.ck4_quantize_weight_convrot
    assert w(FAKE, 4, 256, 256, 128, 2, FAKE, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # group 2
    with pytest.raises(ValueError):
        ck._codebook([1.0] * 15)


def test_lora_validation(L):
    p = L.ck4_lora_prepare_down
    assert p(NULL, 32, 256, 256, 128, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert p(FAKE, 32, 256, 200, 128, FAKE, NULL) == ck.CK4_ERR_INVALID  # lda < k
    assert p(FAKE, 32, 256, 256, 128, ODD, NULL) == ck.CK4_ERR_INVALID  # a_rot alignment
    assert p(FAKE, 48, 256, 256, 128, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # rank
    assert p(FAKE, 32, 512, 512, 512, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # rot_block > 256
    d = L.ck4_lora_down
    assert d(FAKE, 8, 256, 256, 128, FAKE, 32, 1.0, NULL, NULL) == ck.CK4_ERR_INVALID
    assert d(FAKE, 0, 256, 256, 128, FAKE, 32, 1.0, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert d(FAKE, 8, 256, 256, 128, FAKE, 32, 1.0, ODD, NULL) == ck.CK4_ERR_INVALID  # t alignment
    assert d(FAKE, 8, 256, 252, 128, FAKE, 32, 1.0, FAKE, NULL) == ck.CK4_ERR_INVALID  # ldx < k
    assert d(FAKE, 8, 320, 320, 64, FAKE, 32, 1.0, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 128
    assert d(FAKE, 8, 256, 256, 128, FAKE, 96, 1.0, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # rank
    assert d(FAKE, 8, 1024, 1024, 512, FAKE, 32, 1.0, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # rot_block
    u = L.ck4_lora_prepare_up
    assert u(NULL, 40, 32, 32, FAKE, NULL) == ck.CK4_ERR_INVALID
    assert u(FAKE, 40, 32, 16, FAKE, NULL) == ck.CK4_ERR_INVALID  # ldb < rank
    assert u(FAKE, 40, 32, 32, ODD, NULL) == ck.CK4_ERR_INVALID  # b_pack alignment
    assert u(FAKE, 40, 48, 48, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # rank
    assert p(FAKE, 32, 272, 272, 16, FAKE, NULL) == ck.CK4_ERR_UNSUPPORTED  # k % 32
    f = L.ck4_linear_w4a4_lora
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, 32, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, FAKE, ODD, 32, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 16, 8, 8, 256, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 32, 8, 8, 192, FAKE, 8, NULL) == ck.CK4_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 32, 8, 8, 256, FAKE, 4, NULL) == ck.CK4_ERR_INVALID


def test_no_cpu_fallback_without_library(tmp_path, monkeypatch):
    # The binding must fail loudly, not compute elsewhere, when the library is absent.
    monkeypatch.setattr(ck, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ck, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        ck.lib()


def test_fragment_order_helper_is_the_documented_permutation():
    import frag_layout
    for rows, cols in ((16, 32), (40, 64), (1, 256), (33, 3072)):
        off = frag_layout.offsets(frag_layout.rows16(rows), cols)
        assert np.array_equal(np.sort(off.reshape(-1)), np.arange(off.size))
        z = np.random.default_rng(rows).integers(0, 65535, (rows, cols), dtype=np.uint16)
        assert np.array_equal(frag_layout.unpack(frag_layout.pack(z), rows), z)
    # a tile holds, at lane l = 16 g + i, slots 0-3 = columns 4 g .. 4 g + 3 and
    # slots 4-7 = columns 16 + 4 g .. of row i
    z = np.arange(16 * 32, dtype=np.uint16).reshape(16, 32)
    t = frag_layout.pack(z).reshape(64, 8)
    assert list(t[16 * 2 + 5]) == [5 * 32 + c for c in (8, 9, 10, 11, 24, 25, 26, 27)]



def test_fp6_tile_query(L):
    """Host-only: the tile the FP6 GEMM launches per shape, and its shape errors."""
    import test_gpu_parity  # the oracle-checked FP6 shapes must reach both tiles
    tiles = {ck.gemm_fp6_tile(m, n, k) for m, n, k in test_gpu_parity.FP6_CASES}
    assert tiles == {(288, 192), (96, 128)}
    for name in ("square_3072", "up_3072_12288", "down_12288_3072"):
        cfg = workloads.WORKLOADS[name]
        assert ck.gemm_fp6_tile(cfg["m"], cfg["n"], cfg["k"]) == (288, 192)
    tm, tn = ctypes.c_int(0), ctypes.c_int(0)
    f = L.ck4_gemm_fp6_tile
    assert f(8, 8, 192, ctypes.byref(tm), ctypes.byref(tn)) == ck.CK4_ERR_UNSUPPORTED
    assert f(0, 8, 128, ctypes.byref(tm), ctypes.byref(tn)) == ck.CK4_ERR_INVALID
    assert f(8, 8, 128, None, ctypes.byref(tn)) == ck.CK4_ERR_INVALID


def test_noalloc_validation(L):
    """The no-allocation W4A8 entry point refuses, before any device call, a single-pass decode larger than its
    fixed buffer, and a non-positive size."""
    f = L.ck4_linear_w4a8_grouped_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 12288, 8192, 128, FAKE, 12288, -1, NULL) == ck.CK4_ERR_UNSUPPORTED
    assert "fixed buffer" in last(L)
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 128, 256, 128, FAKE, 128, 0, NULL) == ck.CK4_ERR_INVALID
