"""The static (caller-supplied) activation tensor scale: checkpoints from an
offline NVFP4 conversion ("ReSET" GitHub README, "Quantize a model to NVFP4")
can carry a calibrated activation scale instead of computing one per call.

* nvfp4_quantize_act_static: codes and scale bytes bit-exact against the
  oracle quantizer's block steps with that scale (oracle.quantize_blocks),
  for scales equal to, below (blocks saturate at 448 / +-6) and above the
  tensor's own.
* nvfp4_quantize_linear_static: bit-identical to the static quantizer
  followed by nvfp4_linear, fused or not, and within the oracle's tolerance
  on its own."""

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


def _bytes(t):
    import torch
    return t.detach().cpu().contiguous().view(-1).view(torch.uint8).numpy()


def _scales_for(xf):
    """The tensor's own scale, one 16x smaller (many blocks saturate) and one
    3x larger (no block reaches 448), each rounded to binary32."""
    _, sg = oracle.global_scale(xf)
    return [np.float32(sg), np.float32(sg / np.float32(16.0)), np.float32(sg * np.float32(3.0))]


def _check_act(q, xf, sg):
    rc, rs = oracle.quantize_blocks(xf, sg)
    assert np.array_equal(q.codes.cpu().numpy(), rc)
    assert np.array_equal(q.scales.cpu().numpy(), rs)


@pytest.mark.parametrize("M,K", [(1, 512), (1, 4096), (4, 5120), (8, 4096), (8, 25600), (3, 1040),
                                 (8, 16)])
def test_static_act_quant_bit_exact(nv, M, K):
    import torch
    x16 = activations_bf16(12, K % 7, M, K, "outlier")
    xf = bf16_to_f32(x16)
    x = to_dev_bf16(x16)
    for sg in _scales_for(xf):
        note(f"static act quant M={M} K={K} sg={sg!r}")
        g = torch.tensor([sg], dtype=torch.float32, device="cuda")
        q = nv.quantize_act_static(x, g)
        _sync()
        _check_act(q, xf, sg)
        if sg < _scales_for(xf)[0]:
            assert np.any(q.scales.cpu().numpy() == 0x7E)            # saturated blocks


@pytest.mark.parametrize("N,K,M", [(256, 512, 1), (6144, 4096, 1), (4096, 4096, 8),
                                   (24576, 4096, 2), (10240, 5120, 8), (5120, 25600, 1),
                                   (100, 1040, 3)])
def test_static_linear_matches_two_launches_and_oracle(nv, N, K, M):
    import torch
    w16 = weights_bf16(13, N % 5, N, K)
    x16 = activations_bf16(13, K % 5, M, K, "student_t")
    wq = nv.quantize_weight(to_dev_bf16(w16))
    x = to_dev_bf16(x16)
    xf = bf16_to_f32(x16)
    wf = bf16_to_f32(w16)
    _, wsg = oracle.global_scale(wf)
    cols = np.unique(np.concatenate([np.arange(min(N, 64)), np.arange(max(0, N - 64), N),
                                     np.random.default_rng(N).choice(N, min(N, 192),
                                                                     replace=False)]))
    wc, wsb = oracle.quantize_blocks(wf[cols], wsg)
    ow = oracle.NVFP4Tensor(wc, wsb, np.asarray(wsg, np.float32))
    for sg in _scales_for(xf)[:2]:
        note(f"static quantize_linear N={N} K={K} M={M} sg={sg!r}")
        g = torch.tensor([sg], dtype=torch.float32, device="cuda")
        y1, q1 = nv.quantize_linear_static(x, g, wq)
        nv.set_option("fuse_quant", 0)
        try:
            y2, q2 = nv.quantize_linear_static(x, g, wq)
        finally:
            nv.set_option("fuse_quant", 1)
        qa = nv.quantize_act_static(x, g)
        y0 = nv.linear(qa, wq)
        _sync()
        for y in (y1, y2):
            assert np.array_equal(_bytes(y), _bytes(y0))
        for q in (q1, q2):
            assert np.array_equal(_bytes(q.codes), _bytes(qa.codes))
            assert np.array_equal(_bytes(q.scales), _bytes(qa.scales))
        _check_act(q1, xf, sg)
        rc, rs = oracle.quantize_blocks(xf, sg)
        ox = oracle.NVFP4Tensor(rc, rs, np.asarray(sg, np.float32))
        ref = oracle.linear_ref(ox, ow)
        bound = oracle.tolerance_bound(ox, ow)
        err = np.abs(y1.cpu().numpy()[:, cols].astype(np.float64) - ref)
        assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300))}"


def test_static_scale_graph_replay(nv):
    """The static path captured into a HIP graph: replays with a new scale
    value and new inputs (read on the device at every replay) match eager
    calls."""
    import torch
    L = QWEN3_8B[0]
    M = 4
    note(f"static quantize_linear graph replay N={L.N} K={L.K} M={M}")
    wq = nv.quantize_weight(to_dev_bf16(weights_bf16(13, 9, L.N, L.K)))
    x = torch.empty((M, L.K), dtype=torch.bfloat16, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    y = torch.empty((M, L.N), dtype=torch.float32, device="cuda")
    q = nv.empty_act(M, L.K)
    ws = nv.workspace(M, L.N, L.K)
    x.copy_(to_dev_bf16(activations_bf16(13, 1, M, L.K, "outlier")))
    g.fill_(0.01)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.quantize_linear_static(x, g, wq, out=y, xq=q, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        nv.quantize_linear_static(x, g, wq, out=y, xq=q, ws=ws)
    for r in range(3):
        x16 = activations_bf16(13, 20 + r, M, L.K, "student_t")
        x.copy_(to_dev_bf16(x16))
        g.fill_(0.003 * (r + 1))
        torch.empty(1 << 20, device="cuda").fill_(1.0)
        _sync()
        graph.replay()
        _sync()
        y0, q0 = nv.quantize_linear_static(x, g, wq)
        _sync()
        assert np.array_equal(_bytes(y), _bytes(y0)), f"replay {r}"
        assert np.array_equal(_bytes(q.codes), _bytes(q0.codes))
        _check_act(q, bf16_to_f32(x16), np.float32(0.003 * (r + 1)))
