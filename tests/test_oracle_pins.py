"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test ties an oracle function to a closed form, a library routine, an
invariant of the mathematics, a hand-worked fixture under ``tests/golden/`` or
brute force on tiny inputs, chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Hadamard transform


@pytest.mark.parametrize("case", _golden("fwht_worked_example.json")["cases"])
def test_fwht_worked_examples(case):
    x = np.array(case["x"], np.float32)
    assert oracle.fwht(x).tolist() == [float(v) for v in case["y"]]


@pytest.mark.parametrize("g", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_columns_are_sylvester_hadamard(g):
    # scipy builds the Sylvester matrix by Kronecker doubling; FWHT(e_i) must
    # be its column i, and H H^T = g I in exact integer arithmetic.
    eye = np.eye(g, dtype=np.float32)
    cols = oracle.fwht(eye)  # row i = FWHT(e_i)
    H = scipy.linalg.hadamard(g)
    assert np.array_equal(cols.T.astype(np.int64), H)
    Hi = cols.astype(np.int64)
    assert np.array_equal(Hi @ Hi.T, g * np.eye(g, dtype=np.int64))


@pytest.mark.parametrize("g", [4, 16, 128, 256])
def test_fwht_involution_exact_small_ints(g):
    rng = np.random.default_rng(1)
    v = rng.integers(-50, 51, size=(20, g)).astype(np.float32)
    twice = oracle.fwht(oracle.fwht(v))
    assert np.array_equal(twice, g * v)


def _fwht_recursive_f32(v):
    # Independent statement of the Sylvester recursion
    # H_2n [a; b] = [H_n a + H_n b; H_n a - H_n b], in fp32, the halves
    # transformed before they are combined.
    n = v.shape[-1]
    if n == 1:
        return v.copy()
    a = _fwht_recursive_f32(v[..., : n // 2])
    b = _fwht_recursive_f32(v[..., n // 2:])
    return np.concatenate([a + b, a - b], axis=-1).astype(np.float32)


@pytest.mark.parametrize("g", [8, 64, 128])
def test_fwht_f32_bitwise_equals_recursive_definition(g):
    # Pins the butterfly order and indexing bit for bit: the recursion above
    # combines the two halves last, i.e. strides ascend.
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((200, g)) * np.exp(rng.uniform(-8, 8, (200, g)))).astype(np.float32)
    got = oracle.fwht(v)
    ref = _fwht_recursive_f32(v)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_hadamard_scale_constant():
    # c_128 = fp32(1/sqrt(128)); written out by hand as 0x3DB504F3.
    c = oracle.hadamard_scale(128)
    assert np.float32(c).view(np.uint32) == 0x3DB504F3
    for g in [2, 4, 16, 64, 256]:
        assert oracle.hadamard_scale(g) == np.float32(1.0 / math.sqrt(g))


@pytest.mark.parametrize("g", [64, 128, 256])
def test_rotation_f32_within_error_bound_of_exact(g):
    # fp32 rotation against the exact rational transform times 1/sqrt(g):
    # each of the log2(g) stages adds at most u*|partial| with |partial| <=
    # sum|x| over the block, then one more rounding for the scale.
    rng = np.random.default_rng(3)
    k = 2 * g
    x = rng.standard_normal((16, k)).astype(np.float32)
    x[:, 5] *= 20
    r = oracle.rotate_f32(x, g).astype(np.float64)
    H = scipy.linalg.hadamard(g).astype(np.float64)
    u = 2.0 ** -24
    for b in range(k // g):
        blk = x[:, b * g:(b + 1) * g].astype(np.float64)
        exact = blk @ H.T / math.sqrt(g)
        bound = (math.log2(g) + 2) * u * np.abs(blk).sum(axis=1, keepdims=True) / math.sqrt(g) * 1.01
        assert np.all(np.abs(r[:, b * g:(b + 1) * g] - exact) <= bound)


def test_rotation_blocks_are_independent_and_orthonormal():
    rng = np.random.default_rng(4)
    g, k = 128, 512
    x = np.zeros((3, k))
    x[:, 128:256] = rng.standard_normal((3, 128))
    r = oracle.rotate_f64(x, g)
    assert np.all(r[:, :128] == 0) and np.all(r[:, 256:] == 0)
    y = rng.standard_normal((5, k))
    ry = oracle.rotate_f64(y, g)
    np.testing.assert_allclose((ry ** 2).sum(1), (y ** 2).sum(1), rtol=1e-13)


def test_rotation_invariance_of_linear():
    # x W^T == (x H c)(W H c)^T before quantisation: the reason the method
    # rotates both operands by the same block-diagonal Hadamard.
    lay = workloads.make_layer(32, 512, 48, seed=5)
    x = workloads.bf16_bits_to_f32(lay.x_bf16).astype(np.float64)
    w = lay.weights[0].astype(np.float64)
    ref = x @ w.T
    rot64 = oracle.rotate_f64(x) @ oracle.rotate_f64(w).T
    assert np.max(np.abs(rot64 - ref)) <= 1e-12 * np.max(np.abs(ref))
    rot32 = oracle.rotate_bf16(lay.x_bf16).astype(np.float64) @ oracle.rotate_f32(lay.weights[0]).astype(np.float64).T
    assert np.max(np.abs(rot32 - ref)) <= 2e-6 * np.max(np.abs(ref))


def test_rotate_bf16_widening_is_exact():
    rng = np.random.default_rng(6)
    xb = workloads.make_activations(rng, 8, 256)
    a = oracle.rotate_bf16(xb)
    b = oracle.rotate_f32(workloads.bf16_bits_to_f32(xb))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --------------------------------------------------------------------------
# Packing


def test_pack_unpack_all_pairs_roundtrip():
    lo, hi = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    q = np.stack([lo.ravel(), hi.ravel()], axis=1).astype(np.int8).reshape(1, -1)
    p = oracle.pack_int4(q)
    assert p.shape == (1, 256)
    assert np.array_equal(oracle.unpack_int4(p), q)
    # two's-complement identity: int8(byte) = 16 * hi + (lo mod 16)
    pv = p.ravel().astype(np.int64)
    assert np.array_equal(pv, 16 * hi.ravel() + np.mod(lo.ravel(), 16))
    # every byte value appears exactly once
    assert sorted(p.view(np.uint8).ravel().tolist()) == list(range(256))


def test_pack_worked_example():
    fx = _golden("pack_worked_example.json")
    q = np.array([fx["codes"]], np.int8)
    p = oracle.pack_int4(q)
    assert p.view(np.uint8).ravel().tolist() == fx["bytes_u8"]
    assert oracle.unpack_int4(p).ravel().tolist() == fx["codes"]


# --------------------------------------------------------------------------
# Quantiser


@pytest.mark.parametrize("row", _golden("quant_ties.json")["rows"])
def test_quantiser_ties_round_half_even(row):
    r = np.array([row["r"]], np.float32)
    q, s = oracle.quantize_rows(r, 0, 7)
    assert float(s[0]) == row["scale"]
    assert q.ravel().tolist() == row["q"]


@pytest.mark.parametrize("qmax", [7, 127])
def test_quantiser_error_bound_and_range(qmax):
    rng = np.random.default_rng(7)
    r = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    r[3, :] = 0.0
    r[5, 17] *= 50
    q, s = oracle.quantize_rows(r, 0, qmax)
    qi = q.astype(np.int64)
    assert np.all(np.abs(qi) <= qmax)
    nz = np.any(r != 0, axis=1)
    assert np.all(np.abs(qi[nz]).max(axis=1) == qmax)
    assert np.all(qi[~nz] == 0) and np.all(s[~nz] == 0)
    # |r - q s| <= s/2, up to the two fp32 roundings in s and r/s
    err = np.abs(r.astype(np.float64) - qi * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + qmax * 2.0 ** -21))
    # scale = absmax / qmax to within one fp32 rounding
    amax = np.abs(r.astype(np.float64)).max(axis=1)
    np.testing.assert_allclose(s.astype(np.float64), amax / qmax, rtol=2 ** -23)


def test_quantiser_monotone_and_power_of_two_invariant():
    rng = np.random.default_rng(8)
    r = rng.standard_normal((16, 256)).astype(np.float32)
    q, s = oracle.quantize_rows(r, 0, 7)
    for i in range(16):
        order = np.argsort(r[i], kind="stable")
        assert np.all(np.diff(q[i][order].astype(int)) >= 0)
    q2, s2 = oracle.quantize_rows(r * np.float32(2.0 ** 13), 0, 7)
    assert np.array_equal(q, q2)
    assert np.array_equal(s2, s * np.float32(2.0 ** 13))


@pytest.mark.parametrize("G", [4, 8, 128])
def test_grouped_quantiser_per_group(G):
    rng = np.random.default_rng(9)
    r = rng.standard_normal((4, 512)).astype(np.float32)
    r[:, 130] = 40.0
    q, s = oracle.quantize_rows(r, G, 7)
    assert s.shape == (4, 512 // G)
    for gi in range(512 // G):
        qg, sg = oracle.quantize_rows(np.ascontiguousarray(r[:, gi * G:(gi + 1) * G]), 0, 7)
        assert np.array_equal(q[:, gi * G:(gi + 1) * G], qg)
        assert np.array_equal(s[:, gi], sg)


# --------------------------------------------------------------------------
# Integer GEMM


def _unpack_independent(p):
    # int8(byte) = 16*hi + lo_u  =>  hi = floor(int8 / 16), lo = lo_u - 16*[lo_u >= 8]
    b = p.astype(np.int64)
    hi = np.floor_divide(b, 16)
    lo_u = b - 16 * hi
    lo = lo_u - 16 * (lo_u >= 8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 17, 128), (17, 3, 256), (5, 7, 256)])
def test_gemm_bruteforce_tiny(m, n, k):
    rng = np.random.default_rng(m * 100 + n)
    qa = rng.integers(-7, 8, (m, k)).astype(np.int8)
    qb = rng.integers(-7, 8, (n, k)).astype(np.int8)
    acc = oracle.gemm_acc(oracle.pack_int4(qa), oracle.pack_int4(qb), k, bits=4)
    ua = _unpack_independent(oracle.pack_int4(qa))
    ub = _unpack_independent(oracle.pack_int4(qb))
    for i in range(m):
        for j in range(n):
            assert acc[i, j] == sum(int(ua[i, t]) * int(ub[j, t]) for t in range(k))


@pytest.mark.parametrize("k", [128, 3072, 12288])
def test_gemm_bound_is_tight(k):
    a = oracle.pack_int4(np.full((2, k), 7, np.int8))
    b = oracle.pack_int4(np.stack([np.full(k, 7), np.full(k, -7)]).astype(np.int8))
    acc = oracle.gemm_acc(a, b, k, bits=4)
    assert acc.tolist() == [[49 * k, -49 * k], [49 * k, -49 * k]]


def test_gemm_matches_float64_matmul_of_codes():
    # fp64 matmul of integer codes is exact here (|partial sums| < 2^53)
    rng = np.random.default_rng(10)
    m, n, k = 40, 56, 384
    qa = rng.integers(-7, 8, (m, k)).astype(np.int8)
    qb = rng.integers(-7, 8, (n, k)).astype(np.int8)
    acc = oracle.gemm_acc(oracle.pack_int4(qa), oracle.pack_int4(qb), k, bits=4)
    assert np.array_equal(acc, (qa.astype(np.float64) @ qb.astype(np.float64).T).astype(np.int64))
    a8 = rng.integers(-127, 128, (m, k)).astype(np.int8)
    b8 = rng.integers(-127, 128, (n, k)).astype(np.int8)
    acc8 = oracle.gemm_acc(a8, b8, k, bits=8)
    assert np.array_equal(acc8, (a8.astype(np.float64) @ b8.astype(np.float64).T).astype(np.int64))


# --------------------------------------------------------------------------
# Epilogue and bf16 rounding


@pytest.mark.parametrize("case", _golden("bf16_rounding.json")["cases"])
def test_bf16_rounding_worked_examples(case):
    v = eval(case["v"], {"__builtins__": {}})  # fixture arithmetic only
    assert oracle.f64_to_bf16(v) == case["bits"]


def _bf16_value(bits):
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def test_bf16_rounding_is_nearest_even_bruteforce():
    rng = np.random.default_rng(11)
    vals = rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))
    for v in vals:
        b = oracle.f64_to_bf16(v)
        y = Fraction(_bf16_value(b))
        fv = Fraction(float(v))
        # neighbours on the bf16 grid (same sign, magnitude +-1 pattern)
        up = Fraction(_bf16_value(b + 1))
        dn = Fraction(_bf16_value(b - 1)) if (b & 0x7FFF) else Fraction(0)
        d = abs(fv - y)
        assert d <= abs(fv - up) and d <= abs(fv - dn)
        if d == abs(fv - up) or d == abs(fv - dn):
            assert b % 2 == 0


def test_linear_epilogue_within_half_ulp_of_exact_dequant():
    lay = workloads.make_layer(24, 256, 40, seed=12)
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0])
    xq, sx = oracle.rotate_quantize_act(lay.x_bf16)
    y = oracle.linear_w4a4(lay.x_bf16, wp, ws)
    # exact value from dequantised codes, in rationals
    qa = _unpack_independent(xq)
    qb = _unpack_independent(wp)
    acc = qa @ qb.T
    for i in range(0, 24, 5):
        for j in range(0, 40, 3):
            exact = Fraction(int(acc[i, j])) * Fraction(float(sx[i])) * Fraction(float(ws[j]))
            got = Fraction(_bf16_value(int(y[i, j])))
            if exact == 0:
                assert got == 0
                continue
            ulp = Fraction(2) ** (math.frexp(float(exact))[1] - 8)
            assert abs(got - exact) <= ulp / 2


def test_linear_within_quantisation_error_bound_of_float():
    # End-to-end: |y - x W^T| is bounded by the two quantisation errors in the
    # rotated basis (|dx| <= s_x/2, |dw| <= s_w/2), the fp32 rotations and the
    # final bf16 rounding. A wrong sign, index or transposed operand anywhere
    # in rotation, scale, packing or GEMM breaks it.
    lay = workloads.make_layer(32, 512, 48, seed=13)
    x = workloads.bf16_bits_to_f32(lay.x_bf16).astype(np.float64)
    w = lay.weights[0].astype(np.float64)
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0])
    _, sx = oracle.rotate_quantize_act(lay.x_bf16)
    y = workloads.bf16_bits_to_f32(oracle.linear_w4a4(lay.x_bf16, wp, ws)).astype(np.float64)
    ref = x @ w.T
    rx = np.abs(oracle.rotate_f64(x))
    rw = np.abs(oracle.rotate_f64(w))
    sx = sx.astype(np.float64)[:, None]
    sw = ws.astype(np.float64)[None, :]
    k = x.shape[1]
    bound = (rx @ np.ones((k, 1))) * sw / 2 + sx * (rw.sum(1)[None, :]) / 2 + k * sx * sw / 4
    bound = bound * 1.001 + 1e-5 * (np.abs(x) @ np.abs(w).T) + np.abs(ref) * 2.0 ** -8
    assert np.all(np.abs(y - ref) <= bound)
    # and the bound is not vacuous: the typical error is far inside it
    assert np.median(np.abs(y - ref) / bound) < 0.2


# --------------------------------------------------------------------------
# Grouped W4A8 decode


@pytest.mark.parametrize("G", [4, 8, 16, 32, 64, 128])
def test_w4a8_decode_invariants(G):
    # the pages test the decode over group sizes 4 to 64 ([PR97] Testing)
    rng = np.random.default_rng(14)
    n, k = 64, 512
    w = workloads.make_weight(rng, n, k)
    w[:, 3] *= 30
    wp, gs = oracle.quantize_weight_convrot(w, group=G)
    assert gs.shape == (n, k // G)
    w8, srow = oracle.decode_w4a8(wp, gs, G)
    q = _unpack_independent(wp)
    assert np.all(np.abs(w8.astype(int)) <= 127)
    np.testing.assert_allclose(srow.astype(np.float64), gs.max(1).astype(np.float64) * 7 / 127, rtol=3 * 2 ** -24)
    # decoded value approximates the grouped dequantised value within half a step
    deq = q * np.repeat(gs.astype(np.float64), G, axis=1)
    err = np.abs(w8.astype(np.float64) * srow.astype(np.float64)[:, None] - deq)
    assert np.all(err <= srow.astype(np.float64)[:, None] * (0.5 + 1e-5))
    # in each row's max-scale group, codes +-7 decode to +-127 exactly
    for i in range(n):
        gi = int(np.argmax(gs[i]))
        sl = slice(gi * G, (gi + 1) * G)
        sev = np.abs(q[i, sl]) == 7
        assert np.all(np.abs(w8[i, sl][sev].astype(int)) == 127)


def test_w4a8_chunked_equals_single_pass():
    # A chunk boundary must not change a bit, including a short trailing
    # chunk (the pages test N=1152 with 384-column chunks).
    rng = np.random.default_rng(15)
    n, k, G = 1152, 256, 128
    wp, gs = oracle.quantize_weight_convrot(workloads.make_weight(rng, n, k), group=G)
    full8, fulls = oracle.decode_w4a8(wp, gs, G)
    for cols in (384, 500):
        parts = [oracle.decode_w4a8(wp, gs, G, n0, min(cols, n - n0)) for n0 in range(0, n, cols)]
        assert np.array_equal(np.concatenate([p[0] for p in parts]), full8)
        assert np.array_equal(np.concatenate([p[1] for p in parts]), fulls)


def test_w4a8_zero_row():
    wp = np.zeros((2, 128), np.int8)
    gs = np.zeros((2, 2), np.float32)
    w8, srow = oracle.decode_w4a8(wp, gs, 128)
    assert np.all(w8 == 0) and np.all(srow == 0)


def test_w4a8_linear_close_to_float():
    lay = workloads.make_layer(16, 512, 64, seed=16)
    wp, gs = oracle.quantize_weight_convrot(lay.weights[0], group=128)
    y = workloads.bf16_bits_to_f32(oracle.linear_w4a8_grouped(lay.x_bf16, wp, gs)).astype(np.float64)
    ref = workloads.bf16_bits_to_f32(lay.x_bf16).astype(np.float64) @ lay.weights[0].astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    # W4 weights dominate the error; the pages report 0.02-0.055 relative for
    # their eager W4A8 path against full precision.
    assert rel < 0.15


# --------------------------------------------------------------------------
# W8A8 (the int8 layout the int4 one extends)


def test_w8_weight_prep_equals_activation_path_on_bf16_values():
    # Weights that are exact bf16 values take the same fp32 rotation and the
    # same absmax/127 quantiser whether they enter as fp32 (weight prep) or
    # as bf16 (dynamic activation path): two separate oracle code paths.
    rng = np.random.default_rng(41)
    xb = workloads.make_activations(rng, 9, 512)
    w = workloads.bf16_bits_to_f32(xb)
    q_w, s_w = oracle.quantize_weight_convrot_int8(w)
    q_x, s_x = oracle.rotate_quantize_act(xb, bits=8)
    assert np.array_equal(q_w, q_x)
    assert np.array_equal(s_w.view(np.uint32), s_x.view(np.uint32))
    assert np.abs(q_w).max() == 127


def test_w8a8_linear_within_quantisation_error_of_float():
    rng = np.random.default_rng(42)
    m, k, n = 12, 768, 40
    xb = workloads.make_activations(rng, m, k)
    w = workloads.make_weight(rng, n, k)
    w8, ws = oracle.quantize_weight_convrot_int8(w)
    y = oracle.bf16_bits_to_f64(oracle.linear_w8a8(xb, w8, ws))
    ref = oracle.bf16_bits_to_f64(xb) @ w.astype(np.float64).T
    # int8 codes: per-element error <= s/2 on both sides; bound the dot product
    xr = oracle.rotate_f64(oracle.bf16_bits_to_f64(xb))
    wr = oracle.rotate_f64(w.astype(np.float64))
    sx = np.abs(xr).max(axis=1) / 127
    sw = np.abs(wr).max(axis=1) / 127
    bound = (np.abs(xr).sum(axis=1)[:, None] * sw[None, :] / 2 + sx[:, None] * np.abs(wr).sum(axis=1)[None, :] / 2
             + k * sx[:, None] * sw[None, :] / 4)
    err = np.abs(y - ref)
    assert np.all(err <= bound * 1.01 + np.abs(ref) * 2 ** -7)


# --------------------------------------------------------------------------
# Stochastic-rounding requantisation (u supplied by the caller)


def _quotients(r, s):
    """fp32 r / s per row; 0 for the all-zero rows (s == 0)."""
    sd = np.where(s == 0, np.float32(1), s).astype(np.float32)
    return np.where(s[:, None] == 0, np.float32(0), r.astype(np.float32) / sd[:, None]).astype(np.float32)


def test_sr_with_u_zero_is_floor_and_half_is_round_half_up():
    rng = np.random.default_rng(51)
    r = (rng.standard_normal((6, 256)) * 3).astype(np.float32)
    r[2] = 0
    q_near, s = oracle.quantize_rows(r)
    x = _quotients(r, s)
    q0, s0 = oracle.quantize_rows_sr(r, np.zeros_like(r))
    assert np.array_equal(s0.view(np.uint32), s.view(np.uint32))
    assert np.array_equal(q0, np.clip(np.floor(x), -7, 7).astype(np.int8))
    qh, _ = oracle.quantize_rows_sr(r, np.full_like(r, 0.5))
    assert np.array_equal(qh, np.clip(np.floor(x + np.float32(0.5)), -7, 7).astype(np.int8))
    assert not q0[2].any() and not qh[2].any()


def test_sr_codes_are_floor_or_ceil_and_unbiased():
    rng = np.random.default_rng(52)
    r = (rng.standard_normal((1, 128)) * 2).astype(np.float32)
    _, s = oracle.quantize_rows(r)
    x = _quotients(r, s)[0]
    draws = 4000
    rr = np.repeat(r, draws, axis=0)
    u = rng.random(rr.shape, dtype=np.float32)
    q, _ = oracle.quantize_rows_sr(rr, u)
    fl = np.floor(x)
    assert np.all((q == fl) | (q == fl + 1))
    # E[q] = x: each code is a Bernoulli(frac(x)) step above floor(x)
    p = x - fl
    sigma = np.sqrt(np.maximum(p * (1 - p), 1e-12) / draws)
    assert np.all(np.abs(q.mean(axis=0) - x) <= 5 * sigma + 1e-6)


def test_sr_weight_prep_matches_nearest_scales_and_packs():
    rng = np.random.default_rng(53)
    w = workloads.make_weight(rng, 17, 512)
    w[4] = 0
    u = rng.random(w.shape, dtype=np.float32)
    for group in (0, 128):
        wp, ws = oracle.quantize_weight_convrot_sr(w, u, group=group)
        _, ws_near = oracle.quantize_weight_convrot(w, group=group)
        assert np.array_equal(ws.view(np.uint32), ws_near.view(np.uint32))
        q = oracle.unpack_int4(wp)
        assert np.abs(q).max() <= 7 and not q[4].any()


# --------------------------------------------------------------------------
# E4M3 group scales (OCP FP8 E4M3: bias 7, largest 448, no infinities)


def test_e4m3_decode_anchor_values_and_structure():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    assert d[0x7E] == 448.0 and d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9
    assert d[0x07] == 0.875 * 2.0 ** -6 and d[0x38] == 1.0 and d[0x00] == 0.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # strictly increasing codes
    assert np.array_equal(d[0x80:0xFF], -pos)            # sign bit
    for e in range(1, 16):                               # spacing 2^(e-10) inside binade e
        codes = [(e << 3) | m for m in range(8) if (e << 3) | m < 0x7F]
        assert np.all(np.diff(d[codes]) == 2.0 ** (e - 10))


def test_e4m3_encode_is_nearest_ties_even_saturating():
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    rng = np.random.default_rng(61)
    x = np.concatenate([rng.random(300) * 460, 2.0 ** rng.uniform(-12, 9, 300)]).astype(np.float32)
    b = oracle.e4m3_encode(x)
    got = oracle.e4m3_decode(b).astype(np.float64)
    best = np.min(np.abs(x.astype(np.float64)[:, None] - vals[None, :]), axis=1)
    inside = x.astype(np.float64) < 448
    assert np.all(np.abs(x.astype(np.float64) - got)[inside] == best[inside])
    assert np.all(b[~inside] == 0x7E)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    exact = mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2
    bm = oracle.e4m3_encode(mids[exact])
    assert np.all(bm % 2 == 0)                           # ties go to the even code
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), np.arange(0x7F, dtype=np.uint8))
    assert oracle.e4m3_encode(np.float32(1e6)) == 0x7E and oracle.e4m3_encode(np.float32(-1.0)) == 0xB8


def test_e4m3_weight_prep_rounds_fp32_scales_and_bounds_codes():
    rng = np.random.default_rng(62)
    w = workloads.make_weight(rng, 9, 1024)
    w[3] = 0
    w[4] *= 1e-6          # scales in the subnormal range
    for group in (32, 128):
        wp, s8 = oracle.quantize_weight_convrot_e4m3(w, group=group)
        _, s32 = oracle.quantize_weight_convrot(w, group=group)
        assert np.array_equal(s8, oracle.e4m3_encode(s32))
        sd = oracle.e4m3_decode(s8).astype(np.float64)
        q = oracle.unpack_int4(wp).astype(np.float64).reshape(9, -1, group)
        r = oracle.rotate_f32(w).astype(np.float64).reshape(9, -1, group)
        ok = sd > 0
        sdb = np.broadcast_to(sd[..., None], r.shape)
        okb = np.broadcast_to(ok[..., None], r.shape)
        err = np.abs(r - q * sdb)
        unclipped = np.abs(r) <= 7 * sdb
        sel = okb & unclipped
        assert np.all(err[sel] <= sdb[sel] / 2 * (1 + 2 ** -20))   # nearest code against the decoded scale
        assert np.all(np.abs(q[okb & ~unclipped]) == 7)           # beyond 7 s8: clamped
        assert not q[~okb].any() and not q[3].any()


# --------------------------------------------------------------------------
# Codebook W4A8 ([PR97] What this adds, On #96): code u stands for cb[u]
# times the group scale; prep picks the nearest entry, decode re-expresses
# cb[u] * s_g against the row scale max_g s_g * cmax / 127.

# The uniform int4 levels as a codebook: u -> q for u < 8, u - 16 above,
# with the unused -8 replaced by -7 so that cmax = 7 as in the int4 path.
CB_UNIFORM = np.array([0, 1, 2, 3, 4, 5, 6, 7, -7, -7, -6, -5, -4, -3, -2, -1], np.float32)


@pytest.mark.parametrize("G", [4, 8, 16, 32, 64, 128])
@pytest.mark.parametrize("e4m3", [False, True])
def test_codebook_of_uniform_levels_is_the_int4_path(G, e4m3):
    # Nearest entry of the uniform table = rint clamped to +-7 (no exact
    # half-integer quotients occur in these draws), so the codebook prep and
    # decode must reproduce the independently pinned int4 prep and decode.
    rng = np.random.default_rng(70)
    w = workloads.make_weight(rng, 24, 512)
    w[5] = 0
    w[7, :64] = 0
    wp_c, s_c = oracle.quantize_weight_convrot_codebook(w, CB_UNIFORM, group=G, e4m3=e4m3)
    if e4m3:
        wp_u, s_u = oracle.quantize_weight_convrot_e4m3(w, group=G)
        s_uf = oracle.e4m3_decode(s_u)
    else:
        wp_u, s_u = oracle.quantize_weight_convrot(w, group=G)
        s_uf = s_u
    assert np.array_equal(s_c, s_u)
    u = _unpack_independent(wp_c) & 15
    assert np.array_equal(CB_UNIFORM[u], _unpack_independent(wp_u).astype(np.float32))
    w8_c, sr_c = oracle.decode_w4a8_codebook(wp_c, s_c, CB_UNIFORM, G)
    w8_u, sr_u = oracle.decode_w4a8(wp_u, s_uf, G)
    assert np.array_equal(w8_c, w8_u) and np.array_equal(sr_c, sr_u)


def test_codebook_prep_picks_nearest_entry_bruteforce():
    # Unordered table with a repeated entry (index 11 repeats index 3, so it
    # must never be chosen), a zero and an asymmetric range (cmax from a
    # negative entry). Checked in float64 against every entry.
    cb = np.array([0.9, -0.2, 0.05, 0.5, -1.3, 0.0, 0.3, -0.6, 1.1, -0.05, 0.7, 0.5, -0.9, 0.15, -0.35, 0.2],
                  np.float32)
    cmax = 1.3
    rng = np.random.default_rng(71)
    w = workloads.make_weight(rng, 6, 256)
    G = 16
    wp, s = oracle.quantize_weight_convrot_codebook(w, cb, group=G)
    r = oracle.rotate_f32(w).astype(np.float64).reshape(6, -1, G)
    amax = np.abs(r).max(axis=2)
    np.testing.assert_allclose(s.astype(np.float64), amax / cmax, rtol=2 * 2 ** -24)
    u = (_unpack_independent(wp) & 15).reshape(6, -1, G)
    t = r / s.astype(np.float64)[..., None]
    d = np.abs(t[..., None] - cb.astype(np.float64))          # [6, groups, G, 16]
    chosen = np.take_along_axis(d, u[..., None], axis=3)[..., 0]
    assert np.all(chosen <= d.min(axis=3) + 2 ** -20 * (1 + np.abs(t)))
    assert not np.any(u == 11)
    # every entry but the repeated one is used somewhere
    assert set(np.unique(u)) == set(range(16)) - {11}


def test_codebook_zero_group_takes_the_entry_nearest_zero():
    cb = np.array([0.5, -0.25, 0.25, 1, -1, 0.75, -0.5, -0.75, 0.125, -0.125, 0.875, -0.875, 0.375, -0.375, 0.625,
                   -0.625], np.float32)
    w = np.zeros((2, 256), np.float32)
    w[1, 128:] = np.linspace(-1, 1, 128, dtype=np.float32)
    wp, s = oracle.quantize_weight_convrot_codebook(w, cb, group=128)
    assert s[0].tolist() == [0, 0] and s[1, 0] == 0 and s[1, 1] > 0
    u = _unpack_independent(wp) & 15
    assert np.all(u[0] == 8) and np.all(u[1, :128] == 8)      # 0.125 and -0.125 tie: lower index 8
    w8, srow = oracle.decode_w4a8_codebook(wp, s, cb, 128)
    assert np.all(w8[0] == 0) and srow[0] == 0 and np.all(w8[1, :128] == 0)


@pytest.mark.parametrize("G", [4, 8, 32, 128])
def test_codebook_decode_approximates_dequantised_value(G):
    cb = workloads.make_codebook()
    rng = np.random.default_rng(72)
    n, k = 32, 512
    w = workloads.make_weight(rng, n, k)
    w[:, 7] *= 25
    wp, s = oracle.quantize_weight_convrot_codebook(w, cb, group=G)
    w8, srow = oracle.decode_w4a8_codebook(wp, s, cb, G)
    u = _unpack_independent(wp) & 15
    cmax = float(np.abs(cb.astype(np.float64)).max())
    np.testing.assert_allclose(srow.astype(np.float64), s.max(1).astype(np.float64) * cmax / 127,
                               rtol=3 * 2 ** -24)
    deq = cb.astype(np.float64)[u] * np.repeat(s.astype(np.float64), G, axis=1)
    sr = srow.astype(np.float64)[:, None]
    assert np.all(np.abs(w8.astype(np.float64) * sr - deq) <= sr * (0.5 + 1e-5))
    assert np.all(np.abs(w8.astype(int)) <= 127)
    # a decode that keeps 7 in place of cmax (the int4 formula) breaks the bound
    w8_bad, srow_bad = oracle.decode_w4a8(wp, s, G)
    srb = srow_bad.astype(np.float64)[:, None]
    assert np.any(np.abs(w8_bad.astype(np.float64) * srb - deq) > srb * 0.5 + 1e-3 * np.abs(deq).max())


def test_codebook_e4m3_scales_round_the_fp32_scales():
    cb = workloads.make_codebook()
    rng = np.random.default_rng(73)
    w = workloads.make_weight(rng, 8, 512)
    w[2] *= 1e-6
    for G in (8, 64):
        wp8, s8 = oracle.quantize_weight_convrot_codebook(w, cb, group=G, e4m3=True)
        _, s32 = oracle.quantize_weight_convrot_codebook(w, cb, group=G)
        assert np.array_equal(s8, oracle.e4m3_encode(s32))
        # the codes are the nearest entries against the decoded byte
        sd = oracle.e4m3_decode(s8).astype(np.float64)
        r = oracle.rotate_f32(w).astype(np.float64).reshape(8, -1, G)
        u = (_unpack_independent(wp8) & 15).reshape(8, -1, G)
        ok = sd > 0
        t = np.where(ok[..., None], r / np.where(ok, sd, 1)[..., None], 0.0)
        d = np.abs(t[..., None] - cb.astype(np.float64))
        chosen = np.take_along_axis(d, u[..., None], axis=3)[..., 0]
        assert np.all(chosen <= d.min(axis=3) + 2 ** -20 * (1 + np.abs(t)))


def test_codebook_linear_close_to_float():
    lay = workloads.make_layer(16, 512, 64, seed=74)
    cb = workloads.make_codebook()
    wp, s = oracle.quantize_weight_convrot_codebook(lay.weights[0], cb, group=32)
    y = workloads.bf16_bits_to_f32(oracle.linear_w4a8_codebook(lay.x_bf16, wp, s, cb, 32)).astype(np.float64)
    ref = workloads.bf16_bits_to_f32(lay.x_bf16).astype(np.float64) @ lay.weights[0].astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.15


# --------------------------------------------------------------------------
# Dynamic LoRA: the down projection is rotated like the weights, so that
# x A^T = (x R)(A R)^T for the orthonormal block rotation R.


def _rot_err_f32(v, g=128):
    """Per-element bound on |fp32 rotation - exact rotation| (the bound pinned above)."""
    v = np.abs(np.asarray(v, np.float64))
    m, k = v.shape
    blk = v.reshape(m, k // g, g).sum(axis=2, keepdims=True)
    e = (math.log2(g) + 2) * 2.0 ** -24 * blk / math.sqrt(g) * 1.01
    return np.broadcast_to(e, (m, k // g, g)).reshape(m, k)


def _bf16(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def test_lora_prepare_down_is_rotation_rounded_once():
    rng = np.random.default_rng(40)
    a, _ = workloads.make_lora(rng, 32, 512, 8)
    got = _bf16(oracle.lora_prepare_down(a))
    exact = oracle.rotate_f64(a.astype(np.float64))
    e32 = _rot_err_f32(a)
    # bf16 keeps 8 significant bits: one rounding is within 2^-8 relative
    bound = 2.0 ** -8 * (np.abs(exact) + e32) + e32
    assert np.all(np.abs(got - exact) <= bound)
    # the rows keep their inner products (R is orthonormal), up to the bf16 rounding
    gram = got @ got.T
    ref = a.astype(np.float64) @ a.astype(np.float64).T
    assert np.all(np.abs(gram - ref) <= 2.0 ** -6.9 * (np.abs(got) @ np.abs(got).T))
    # the bound is not vacuous: an unrotated A is far outside it
    assert np.any(np.abs(_bf16(oracle.to_bf16(a)) - exact) > bound)


def test_lora_down_equals_unrotated_product_within_rounding():
    lay = workloads.make_layer(24, 512, 8, seed=41)
    a, _ = workloads.make_lora(np.random.default_rng(42), 64, 512, 8)
    alpha = 0.75
    t = _bf16(oracle.lora_down(lay.x_bf16, oracle.lora_prepare_down(a), alpha))
    x = _bf16(lay.x_bf16)
    ref = alpha * x @ a.astype(np.float64).T
    rx = np.abs(oracle.rotate_f64(x))
    ra = np.abs(oracle.rotate_f64(a.astype(np.float64)))
    # each operand is the fp32 rotation rounded once to bf16 (2^-8 relative),
    # then t itself is rounded once
    ex = _rot_err_f32(x) * (1 + 2.0 ** -7) + 2.0 ** -8 * rx
    ea = _rot_err_f32(a) * (1 + 2.0 ** -7) + 2.0 ** -8 * ra
    prod_err = ex @ ra.T + rx @ ea.T + ex @ ea.T
    bound = alpha * prod_err * 1.001 + 2.0 ** -8 * np.abs(t) * 1.001
    assert np.all(np.abs(t - ref) <= bound)
    assert np.median(np.abs(t - ref) / bound) < 0.2
    # a down projection left unrotated (a plausible slip) breaks the bound
    xr = _bf16(oracle.to_bf16(oracle.rotate_bf16(lay.x_bf16)))
    t_bad = _bf16(oracle.to_bf16(alpha * xr @ _bf16(oracle.to_bf16(a)).T))
    assert np.any(np.abs(t_bad - ref) > bound)


def test_lora_zero_alpha_is_plain_linear():
    lay = workloads.make_layer(9, 256, 40, seed=43)
    a, b = workloads.make_lora(np.random.default_rng(44), 32, 256, 40)
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0])
    a_rot = oracle.lora_prepare_down(a)
    assert np.all(_bf16(oracle.lora_down(lay.x_bf16, a_rot, 0.0)) == 0)
    y0 = oracle.linear_w4a4_lora(lay.x_bf16, wp, ws, a_rot, b, 0.0)
    assert np.array_equal(y0, oracle.linear_w4a4(lay.x_bf16, wp, ws))


def test_lora_up_adds_rank_terms_exactly():
    m, n, k, rank = 10, 24, 256, 32
    lay = workloads.make_layer(m, k, n, seed=45)
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0])
    xq, sx = oracle.rotate_quantize_act(lay.x_bf16)
    acc = oracle.gemm_acc(xq, wp, k)
    rng = np.random.default_rng(46)
    # t[:, 0] = 2^e_m (exact in bf16), b[:, 0] = c_n; column 7 of t is noise
    # whose b column is zero; every other entry is zero
    e = rng.integers(-3, 4, m)
    t = np.zeros((m, rank), np.uint16)
    t[:, 0] = workloads.f32_to_bf16_bits(np.ldexp(np.ones(m, np.float32), e))
    t[:, 7] = workloads.f32_to_bf16_bits(rng.standard_normal(m).astype(np.float32))
    b = np.zeros((n, rank), np.uint16)
    c = workloads.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    b[:, 0] = c
    y = oracle.epilogue_lora(acc, sx, ws, t, b)
    cf = workloads.bf16_bits_to_f32(c)
    for i in range(m):
        for j in range(n):
            exact = (Fraction(int(acc[i, j])) * Fraction(float(sx[i])) * Fraction(float(ws[j]))
                     + Fraction(2) ** int(e[i]) * Fraction(float(cf[j])))
            got = Fraction(_bf16_value(int(y[i, j])))
            if exact == 0:
                assert got == 0
                continue
            ulp = Fraction(2) ** (math.frexp(float(exact))[1] - 8)
            assert abs(got - exact) <= ulp / 2
    # with t = e_0 for every row the LoRA term is a column bias: same rounding as the plain epilogue
    t1 = np.zeros((m, rank), np.uint16)
    t1[:, 0] = 0x3F80
    assert np.array_equal(oracle.epilogue_lora(acc, sx, ws, t1, b), oracle.epilogue_bf16(acc, sx, ws, cf))


def test_lora_layer_is_base_layer_plus_float_lora():
    m, n, k, rank = 16, 40, 512, 64
    lay = workloads.make_layer(m, k, n, seed=47)
    a, b = workloads.make_lora(np.random.default_rng(48), rank, k, n)
    alpha = 0.5
    wp, ws = oracle.quantize_weight_convrot(lay.weights[0])
    a_rot = oracle.lora_prepare_down(a)
    y = _bf16(oracle.linear_w4a4_lora(lay.x_bf16, wp, ws, a_rot, b, alpha))
    y0 = _bf16(oracle.linear_w4a4(lay.x_bf16, wp, ws))
    x = _bf16(lay.x_bf16)
    bf = _bf16(b)
    ref_t = alpha * x @ a.astype(np.float64).T
    t = _bf16(oracle.lora_down(lay.x_bf16, a_rot, alpha))
    # |t - ref_t| is pinned above; measure it here and carry it through B
    dt = np.abs(t - ref_t)
    bound = 2.0 ** -8 * (np.abs(y) + np.abs(y0)) + dt @ np.abs(bf).T * 1.001 + 2.0 ** -20
    assert np.all(np.abs((y - y0) - ref_t @ bf.T) <= bound)

