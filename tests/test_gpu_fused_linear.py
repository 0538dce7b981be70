"""nvfp4_quantize_linear: the activation quantizer inside the GEMV's
prologue.  Its output and the quantized activation it writes must be
bit-identical to the two-launch path (nvfp4_quantize_act, then nvfp4_linear),
the quantized activation bit-exact to the oracle, and the output within the
oracle's tolerance on its own; shapes past the fused kernel's limit take the
two launches."""

import numpy as np
import pytest

import oracle
from gpu_util import note, to_dev_bf16
from workloads import QWEN3_8B, QWEN3_32B, activations_bf16, bf16_to_f32, weights_bf16

pytestmark = pytest.mark.gpu


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


def _same(a, b):
    return np.array_equal(a.cpu().contiguous().view(-1).view(__import__("torch").uint8).numpy(),
                          b.cpu().contiguous().view(-1).view(__import__("torch").uint8).numpy())


def _check_vs_oracle(y, w16, x16, out_bf16):
    """The fused call's own y against the oracle (not only against the
    two-launch path): the oracle quantizes the activation and a sample of
    weight rows (all rows of small weights) itself, with the tensor scale of
    the whole weight, and y must lie within 1e-3 * sum |x_hat w_hat| (plus
    half a bf16 ulp for bf16 output)."""
    N = w16.shape[0]
    rng = np.random.default_rng(N)
    cols = np.arange(N) if N <= 512 else np.unique(np.concatenate(
        [np.arange(64), np.arange(N - 64, N), rng.choice(N, 256, replace=False)]))
    wf = bf16_to_f32(w16)
    _, sg = oracle.global_scale(wf)
    wc, ws = oracle.quantize_blocks(wf[cols], sg)
    ow = oracle.NVFP4Tensor(wc, ws, np.asarray(sg, np.float32))
    ox = oracle.quantize(bf16_to_f32(x16))
    ref = oracle.linear_ref(ox, ow)
    bound = oracle.tolerance_bound(ox, ow)
    got = y.float().cpu().numpy()[:, cols].astype(np.float64)
    if out_bf16:
        bound = bound + 0.5 * np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300))}"


def _both(nv, x, wq, out_dtype):
    y1, q1 = nv.quantize_linear(x, wq, out_dtype=out_dtype)
    _sync()
    nv.set_option("fuse_quant", 0)
    try:
        y0, q0 = nv.quantize_linear(x, wq, out_dtype=out_dtype)
        _sync()
    finally:
        nv.set_option("fuse_quant", 1)
    return (y1, q1), (y0, q0)


# (the prologue quantizes up to 2048 blocks, 4096 from M = 4: 4096 x 8192 at
# M = 8 is the largest fused case, 256 x 8704 at M = 8 takes two launches)
SHAPES = [(256, 512, 1), (6144, 4096, 1), (4096, 4096, 2), (24576, 4096, 4), (4096, 12288, 1),
          (4096, 4096, 8), (100, 1040, 3), (33, 16, 8), (5120, 25600, 1), (10240, 5120, 8),
          (256, 5632, 8), (5120, 8192, 8), (256, 8704, 8), (300, 8192, 5)]


@pytest.fixture(params=[0, 1, 2], ids=["tiles_auto", "full_tiles", "half_tiles"])
def half_tiles(nv, request):
    nv.set_option("half_tiles", request.param)
    yield request.param
    nv.set_option("half_tiles", 0)


@pytest.mark.parametrize("N,K,M", SHAPES)
def test_fused_matches_two_launches_and_oracle(nv, half_tiles, N, K, M):
    import torch
    note(f"quantize_linear N={N} K={K} M={M}")
    w16 = weights_bf16(8, N % 7, N, K)
    x16 = activations_bf16(8, K % 5, M, K, "outlier")
    wq = nv.quantize_weight(to_dev_bf16(w16))
    x = to_dev_bf16(x16)
    for od in (torch.float32, torch.bfloat16):
        (y1, q1), (y0, q0) = _both(nv, x, wq, od)
        assert _same(y1, y0), f"output differs from the two-launch path ({od})"
        _check_vs_oracle(y1, w16, x16, od == torch.bfloat16)
        for a, b in ((q1.codes, q0.codes), (q1.scales, q0.scales), (q1.gscale, q0.gscale)):
            assert _same(a, b)
    ref = oracle.quantize(bf16_to_f32(x16))
    assert np.array_equal(q1.codes.cpu().numpy(), ref.codes)
    assert np.array_equal(q1.scales.cpu().numpy(), ref.scales)
    assert q1.gscale.cpu().numpy().view(np.uint32)[0] == np.asarray(ref.gscale,
                                                                    np.float32).view(np.uint32)


def test_fused_strided_input_and_graph_replay(nv):
    import torch
    L = QWEN3_8B[0]
    M = 2
    note(f"quantize_linear strided + graph replay N={L.N} K={L.K} M={M}")
    w16 = weights_bf16(8, 1, L.N, L.K)
    wq = nv.quantize_weight(to_dev_bf16(w16))
    wide = torch.empty((M, L.K + 64), dtype=torch.bfloat16, device="cuda")
    x = wide[:, :L.K]
    y = torch.empty((M, L.N), dtype=torch.float32, device="cuda")
    q = nv.empty_act(M, L.K)
    ws = nv.workspace(M, L.N, L.K)
    wide.copy_(to_dev_bf16(activations_bf16(8, 2, M, L.K + 64, "outlier")))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.quantize_linear(x, wq, out=y, xq=q, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        nv.quantize_linear(x, wq, out=y, xq=q, ws=ws)
    for r in range(3):
        x16 = activations_bf16(8, 10 + r, M, L.K + 64, "student_t")
        wide.copy_(to_dev_bf16(x16))
        torch.empty(1 << 20, device="cuda").fill_(3.0)
        _sync()
        g.replay()
        _sync()
        xq = nv.quantize_act(wide[:, :L.K])
        y0 = nv.linear(xq, wq)
        _sync()
        assert _same(y, y0), f"replay {r}"
        assert _same(q.codes, xq.codes) and _same(q.scales, xq.scales)


RMS_SHAPES = [(6144, 4096, 1), (24576, 4096, 2), (10240, 5120, 1), (10240, 5120, 3),
              (51200, 5120, 1), (10240, 5120, 8), (100, 1040, 3), (33, 16, 8), (256, 5632, 8),
              (51200, 5120, 8), (256, 8704, 8)]
U32 = 2.0 ** -24


@pytest.mark.parametrize("N,K,M", RMS_SHAPES)
def test_rmsnorm_quantize_linear(nv, half_tiles, N, K, M):
    """RMS norm, quantization and the linear in one call (one kernel up to
    2048 activation blocks, 4096 from M = 4, else the standalone fused
    quantizer and the linear): h within the binary32 bound of the oracle, the
    codes exactly the oracle quantizer of that h, y bit-identical to the
    linear alone on the written quantized activation."""
    import torch
    note(f"rmsnorm_quantize_linear N={N} K={K} M={M}")
    w16 = weights_bf16(9, N % 7, N, K)
    x16 = activations_bf16(9, K % 5, M, K, "student_t")
    wq = nv.quantize_weight(to_dev_bf16(w16))
    x = to_dev_bf16(x16)
    h = torch.empty((M, K), dtype=torch.float32, device="cuda")
    y, q = nv.rmsnorm_quantize_linear(x, wq, 1e-6, out_dtype=torch.bfloat16, h_out=h)
    _sync()
    hn = h.cpu().numpy()
    ref = oracle.rms_norm_rows(bf16_to_f32(x16).astype(np.float64))
    # row sums: <= 64 sequential adds per thread (a thread holds at most 4
    # blocks of one row: 2048 blocks per row at most over 512 threads), a
    # 6-level wave tree, <= 7 adds over the waves: 40 u covers the square
    # root and the five correctly rounded steps, as for the standalone
    # quantizer
    assert np.all(np.abs(hn - ref) <= 40 * U32 * np.abs(ref) + 1e-38)
    oq = oracle.quantize(hn)
    assert np.array_equal(q.codes.cpu().numpy(), oq.codes)
    assert np.array_equal(q.scales.cpu().numpy(), oq.scales)
    assert q.gscale.cpu().numpy().view(np.uint32)[0] == np.asarray(oq.gscale,
                                                                   np.float32).view(np.uint32)
    y0 = nv.linear(q, wq, out_dtype=torch.bfloat16)
    _sync()
    assert _same(y, y0)


@pytest.mark.parametrize("rms", [0, 1])
def test_exact_queried_workspace_unfused(nv, rms):
    """The C entry points with a workspace of exactly
    nvfp4_quantize_linear_workspace_bytes, on the two-launch path
    (fuse_quant = 0) where the quantizer needs the sync record at M > 1:
    the call succeeds and matches the fused call."""
    import ctypes
    import torch
    M, N, K = 2, 4096, 4096
    note(f"exact queried workspace rms={rms} M={M} N={N} K={K}")
    need = nv._quantize_linear_workspace_bytes(M, N, K)
    assert need >= 16
    wq = nv.quantize_weight(to_dev_bf16(weights_bf16(8, 3, N, K)))
    x = to_dev_bf16(activations_bf16(8, 3, M, K, "outlier"))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    nv.workspace_init(ws)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q = nv.empty_act(M, K)
    vp = ctypes.c_void_p
    args = [vp(wq.codes.data_ptr()), vp(wq.scales.data_ptr()), vp(wq.gscale.data_ptr()),
            vp(y.data_ptr()), nv.OUT_F32, vp(q.codes.data_ptr()), vp(q.scales.data_ptr()),
            vp(q.gscale.data_ptr())]
    tail = [vp(ws.data_ptr()), need, vp(torch.cuda.current_stream().cuda_stream)]
    nv.set_option("fuse_quant", 0)
    try:
        if rms:
            st = nv._lib.nvfp4_rmsnorm_quantize_linear(M, N, K, vp(x.data_ptr()), K,
                                                       ctypes.c_float(1e-6), *args, None, *tail)
        else:
            st = nv._lib.nvfp4_quantize_linear(M, N, K, vp(x.data_ptr()), K, *args, *tail)
    finally:
        nv.set_option("fuse_quant", 1)
    assert st == nv.OK, nv.NVFP4Error(st, "two-launch call")
    _sync()
    if rms:
        # (the RMS norm's row sums run in another order when fused, so h may
        # differ from the fused call's in the last bits: compare y with the
        # linear of the quantized activation this call wrote instead)
        y1 = nv.linear(q, wq)
        _sync()
        assert _same(y, y1)
    else:
        y1, q1 = nv.quantize_linear(x, wq)
        _sync()
        assert _same(q.codes, q1.codes) and _same(q.scales, q1.scales) and _same(y, y1)
