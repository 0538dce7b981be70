"""GPU parity of the fused stack quantizers (RMS norm, SiLU * mul, each
followed by the activation quantizer in one kernel) against the oracle.

h is checked against the oracle's binary64 RMS norm / SiLU * mul within a
bound derived from the binary32 arithmetic; the codes, E4M3 scale bytes and
tensor scale must then be bit-identical to the oracle quantizer applied to the
GPU's own h (the quantizer is exact given its input; the device exp may
differ from the host's by a few ulp, so h itself is compared by tolerance)."""

import numpy as np
import pytest

import oracle
from gpu_util import note, to_dev_bf16
from workloads import activations_bf16, bf16_bits, bf16_to_f32

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24          # binary32 unit roundoff


@pytest.fixture(scope="module")
def nv():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import nvfp4_decode_linear_amd as nv
    return nv


def _sync():
    import torch
    torch.cuda.synchronize()


def _assert_quant_of(q, h32):
    ref = oracle.quantize(h32)
    gs = q.gscale.cpu().numpy().view(np.uint32)[0]
    assert gs == np.asarray(ref.gscale, np.float32).view(np.uint32)
    s, c = q.scales.cpu().numpy(), q.codes.cpu().numpy()
    bad = np.nonzero(s != ref.scales)
    assert bad[0].size == 0, f"scale mismatch at {bad[0][:4]},{bad[1][:4]}"
    bad = np.nonzero(c != ref.codes)
    assert bad[0].size == 0, f"code mismatch at {bad[0][:4]},{bad[1][:4]}"


def _run(nv, mode, x16, K, spin=0):
    import torch
    M = x16.shape[0]
    xd = to_dev_bf16(x16)
    h = torch.empty((M, K), dtype=torch.float32, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    nv.set_option("spin_limit", spin)
    try:
        if mode == "rms":
            q = nv.rmsnorm_quantize_act(xd, 1e-6, h_out=h, ws=ws)
        else:
            q = nv.silu_mul_quantize_act(xd, h_out=h, ws=ws)
        _sync()
    finally:
        nv.set_option("spin_limit", 0)
    assert ws.cpu().numpy().view(np.uint32)[:4].tolist() == [0, 0, 0, 0]
    return q, h.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1, 512), (3, 5120), (8, 5120), (8, 4096), (2, 25600),
                                 (8, 32768), (5, 16)])
def test_rmsnorm_quantize(nv, M, K):
    note(f"rmsnorm quant M={M} K={K}")
    x16 = activations_bf16(5, K % 11, M, K, "student_t")
    q, h = _run(nv, "rms", x16, K)
    ref = oracle.rms_norm_rows(bf16_to_f32(x16).astype(np.float64))
    # sum of squares (positive terms): <= 32 sequential adds per thread, a
    # 6-level wave tree, 15 adds over the waves: relative error <= 53 u;
    # the square root halves it; / K, + eps, sqrt, 1 / and * add <= 5 u:
    # bound 31.5 u, 40 u tested
    err = np.abs(h - ref)
    assert np.all(err <= 40 * U32 * np.abs(ref) + 1e-38), err.max()
    _assert_quant_of(q, h)


@pytest.mark.parametrize("M,K", [(1, 512), (3, 5120), (8, 25600), (1, 25600), (2, 12288),
                                 (5, 16)])
def test_silu_mul_quantize(nv, M, K):
    note(f"silu_mul quant M={M} K={K}")
    gu16 = activations_bf16(5, K % 13, M, 2 * K, "student_t")
    q, h = _run(nv, "silu", gu16, K)
    ref = oracle.silu_mul(bf16_to_f32(gu16).astype(np.float64))
    # exp within a few ulp, then 1 + e, g / (.), * u each correctly rounded;
    # sigmoid is well conditioned: 16 u relative, plus an absolute term for
    # the underflowing tail (g << 0, where h is ~ g * exp(g))
    err = np.abs(h - ref)
    assert np.all(err <= 16 * U32 * np.abs(ref) + 1e-30), err.max()
    _assert_quant_of(q, h)


@pytest.mark.parametrize("mode", ["rms", "silu"])
def test_fused_quantize_forced_fallback(nv, mode):
    """With the spin limit forced to 1 the rows' workgroups mostly compute
    every row's h themselves for the tensor maximum: same bits."""
    M, K = 8, 5120
    note(f"{mode} quant forced fallback M={M} K={K}")
    x16 = activations_bf16(5, 3, M, K if mode == "rms" else 2 * K, "outlier")
    q0, h0 = _run(nv, mode, x16, K)
    q1, h1 = _run(nv, mode, x16, K, spin=1)
    assert np.array_equal(h0.view(np.uint32), h1.view(np.uint32))
    for a, b in ((q0.codes, q1.codes), (q0.scales, q1.scales), (q0.gscale, q1.gscale)):
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("K", [512, 25600])
def test_silu_mul_one_row_without_workspace(nv, K):
    """At M = 1 the workspace is optional: without one a single workgroup
    does the row, with one the blocks spread over workgroups.  Both must
    give the same h, codes, scales and tensor scale."""
    import ctypes
    import torch
    note(f"silu_mul quant M=1 K={K}, with and without workspace")
    gu16 = activations_bf16(5, 7, 1, 2 * K, "student_t")
    q1, h1 = _run(nv, "silu", gu16, K)
    xd = to_dev_bf16(gu16)
    q0 = nv.empty_act(1, K)
    h0 = torch.empty((1, K), dtype=torch.float32, device="cuda")
    st = nv._silu_mul_quantize_act(xd.data_ptr(), 1, K, xd.stride(0), q0.codes.data_ptr(),
                                   q0.scales.data_ptr(), q0.gscale.data_ptr(), h0.data_ptr(),
                                   None, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    _sync()
    assert np.array_equal(h0.cpu().numpy().view(np.uint32), h1.view(np.uint32))
    for a, b in ((q0.codes, q1.codes), (q0.scales, q1.scales), (q0.gscale, q1.gscale)):
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())
    _assert_quant_of(q0, h0.cpu().numpy())


def test_fused_quantize_edges(nv):
    import torch
    note("rmsnorm quant zero row and constant row")
    x = np.zeros((2, 64), np.float32)
    x[1, :] = -3.0
    x16 = bf16_bits(x)
    q, h = _run(nv, "rms", x16, 64)
    assert np.all(h[0] == 0) and np.allclose(h[1], -1.0, rtol=1e-6)
    _assert_quant_of(q, h)
    note("silu_mul quant large magnitudes")
    gu = np.zeros((1, 128), np.float32)
    gu[0, :64] = np.linspace(-90, 90, 64)
    gu[0, 64:] = 1.0
    gu16 = bf16_bits(gu)
    q, h = _run(nv, "silu", gu16, 64)
    ref = oracle.silu_mul(bf16_to_f32(gu16).astype(np.float64))
    assert np.all(np.isfinite(h))
    assert np.all(np.abs(h - ref) <= 16 * U32 * np.abs(ref) + 1e-30)
    _assert_quant_of(q, h)
    note("fused quant strided input (ld = 2K + 64)")
    K = 512
    wide = activations_bf16(5, 7, 3, 2 * K + 64, "outlier")
    xd = to_dev_bf16(wide)[:, :2 * K]
    hh = torch.empty((3, K), dtype=torch.float32, device="cuda")
    qq = nv.silu_mul_quantize_act(xd, h_out=hh)
    _sync()
    _assert_quant_of(qq, hh.cpu().numpy())
