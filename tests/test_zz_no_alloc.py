"""The no-allocation entry point ck4_linear_w4a8_grouped_noalloc against
ck4_linear_w4a8_grouped (the entry point it is a variant of), bit for bit,
on each of its three paths and on two calls in a row, the second smaller
than the first (the fixed buffer keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ck():
    import int4_w4a4_quantized_amd as ck
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    return ck


def _operands(m, n, k, group, seed):
    rng = np.random.default_rng(seed)
    xb = workloads.make_activations(rng, m, k)
    wp, gs = oracle.quantize_weight_convrot(workloads.make_weight(rng, n, k), group=group)
    return xb, torch.from_numpy(wp).cuda(), torch.from_numpy(gs).cuda()


def _bits(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("calls", [
    # (m, n, k, group, chunk_cols): single pass then a smaller chunked call
    [(100, 3000, 3072, 128, -1), (40, 1000, 1024, 64, 256)],
    # default policy: single pass for m > 64, then chunked at the L2 width
    [(130, 2048, 2048, 128, 0), (8, 1500, 512, 128, 512)],
    # chunked, then the fused kernel (no buffer used), then chunked again, smaller
    [(64, 4096, 4096, 32, 1024), (16, 333, 1536, 16, 0), (3, 200, 768, 128, 128)],
])
def test_noalloc_equals_workspace_entry_point(ck, calls):
    for i, (m, n, k, group, chunk) in enumerate(calls):
        xb, wp, gs = _operands(m, n, k, group, 9100 + 10 * i + m)
        xq8, sx = ck.rotate_quantize_act(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda(), 128, 8)
        ldy = (n + 15) // 16 * 16
        y_ref = torch.full((m, ldy), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        y_na = y_ref.clone()
        ck.linear_w4a8_grouped(xq8, sx, wp, gs, group, chunk, out=y_ref[:, :n])
        ck.linear_w4a8_grouped_noalloc(xq8, sx, wp, gs, group, chunk, out=y_na[:, :n])
        a, b = _bits(y_ref), _bits(y_na)
        assert np.array_equal(a, b), f"call {i} {(m, n, k, group, chunk)} differs"
        assert (b[:, n:] == -1).all()


def test_noalloc_refuses_oversized_decode(ck):
    L = ck.lib()
    buf = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    # a single pass over n x k = 12288 x 8192 int8 codes needs 96 MiB
    rc = L.ck4_linear_w4a8_grouped_noalloc(p, p, p, p, 4, 12288, 8192, 128, p, 12288, -1, None)
    assert rc == ck.CK4_ERR_UNSUPPORTED and "fixed buffer" in L.ck4_last_error().decode()
    rc = L.ck4_linear_w4a8_grouped_noalloc(p, p, p, p, 4, 12288, 8192, 128, p, 12288, 12288, None)
    assert rc == ck.CK4_ERR_UNSUPPORTED
