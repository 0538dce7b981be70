"""SiLU * mul between the gate_up and down projections without a quantizer
launch of its own:

* nvfp4_quantize_linear_silu_mul: the bf16 gate/up outputs it rounds (its
  optional gu_out) within the oracle's tolerance of the linear on its own
  quantized activation (itself bit-exact against the oracle quantizer of
  the input, or of the RMS-normalised input it writes); h bit-identical to
  the standalone SiLU quantizer's h on that bf16 output and within a few
  ulp of the oracle's SiLU * mul; the maxima record's largest word is max
  |h|.
* nvfp4_quantize_act_f32: codes, scales and tensor scale bit-exact against
  the oracle quantizer, with and without the record.
* nvfp4_quantize_linear_f32: the written activation bit-exact against the
  oracle, y within the oracle's tolerance on it on every path (the K-slice
  plan with the record, the whole-activation kernel, the two launches) and,
  without the record, bit-identical to nvfp4_linear on those codes.
* nvfp4_quantize_weight_gate_up: byte-identical to nvfp4_quantize_weight of
  the rows in the interleaved order.
* Both calls in a graph, replayed with fresh inputs.

Shapes: the Qwen3-8B and Qwen3-32B gate_up / down projections (FFN 12288 /
25600, hidden 4096 / 5120) at M = 1, 2, 8, and small ragged ones."""

import numpy as np
import pytest

import oracle
from gpu_util import note, to_dev_bf16
from parity_util import check_linear, check_quant, sample_rows
from workloads import activations_bf16, bf16_to_f32, weights_bf16

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


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


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


# (M, F, K): gate_up weight [2F][K]
GATE_UP = [
    (1, 12288, 4096), (8, 12288, 4096),          # Qwen3-8B
    (1, 25600, 5120), (8, 25600, 5120),          # Qwen3-32B
    (3, 96, 272), (2, 32, 16), (5, 160, 1040), (8, 64, 4096), (2, 48, 256), (1, 16, 64),
]


def _interleave(F):
    """Source row of each tiled row of the interleaved gate_up order."""
    t, r = np.divmod(np.arange(2 * F), 32)
    return np.where(r < 16, 16 * t + r, F + 16 * t + r - 16)


@pytest.mark.parametrize("F,K", [(16, 64), (48, 272), (12288, 4096), (25600, 5120)])
def test_gate_up_weight_is_the_interleaved_rows(nv, F, K):
    """nvfp4_quantize_weight_gate_up = nvfp4_quantize_weight of the rows in
    the interleaved order, byte for byte (the latter is pinned against the
    oracle quantizer elsewhere)."""
    note(f"gate_up weight interleave F={F} K={K}")
    w16 = weights_bf16(34, F % 1000, 2 * F, K)
    a = nv.quantize_weight_gate_up(to_dev_bf16(w16))
    b = nv.quantize_weight(to_dev_bf16(w16[_interleave(F)]))
    _sync()
    assert np.array_equal(a.codes.cpu().numpy(), b.codes.cpu().numpy())
    assert np.array_equal(a.scales.cpu().numpy(), b.scales.cpu().numpy())
    assert np.array_equal(_bits(a.gscale), _bits(b.gscale))


@pytest.mark.parametrize("rms", [True, False])
@pytest.mark.parametrize("shape", GATE_UP)
def test_silu_mul_epilogue(nv, shape, rms):
    import torch
    M, F, K = shape
    big = F >= 12288
    if big and not rms:
        pytest.skip("the model shapes run with the RMS norm, as in the stack")
    note(f"silu_mul epilogue M={M} F={F} K={K} rms={rms}")
    w16 = weights_bf16(30, F % 1000, 2 * F, K)
    wq = nv.quantize_weight_gate_up(to_dev_bf16(w16))
    x = to_dev_bf16(activations_bf16(30, K % 1000, M, K, "outlier"))
    gu = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    xh = torch.empty((M, K), dtype=torch.float32, device="cuda") if rms else None
    h, rec, xq = nv.quantize_linear_silu_mul(x, wq, rmsnorm=rms, eps=1e-6, gu_out=gu, xh_out=xh)
    _sync()
    # the activation against the oracle quantizer (of the normalised rows the
    # call wrote, themselves within a few ulp of the oracle's RMS norm)
    xin = bf16_to_f32(x.cpu().view(torch.int16).numpy().view(np.uint16))
    if rms:
        hin = xh.cpu().numpy()
        ref = oracle.rms_norm_rows(xin.astype(np.float64))
        assert np.all(np.abs(hin - ref) <= 40 * U32 * np.abs(ref) + 1e-38)
    else:
        hin = xin
        xs = nv.quantize_act(x)                       # the standalone quantizer, bit for bit
        _sync()
        assert np.array_equal(xq.codes.cpu().numpy(), xs.codes.cpu().numpy())
        assert np.array_equal(xq.scales.cpu().numpy(), xs.scales.cpu().numpy())
        assert np.array_equal(_bits(xq.gscale), _bits(xs.gscale))
    check_quant(xq, hin)
    # the linear against the oracle (sampled columns at the model shapes)
    check_linear(gu, xq, w16, sample_rows(2 * F, 7) if big else None)
    # h: the standalone SiLU quantizer's, on the same bf16 gu
    hs = torch.empty((M, F), dtype=torch.float32, device="cuda")
    nv.silu_mul_quantize_act(gu, h_out=hs)
    _sync()
    assert np.array_equal(_bits(h), _bits(hs))
    gin = bf16_to_f32(gu.cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    ref = oracle.silu_mul(gin)
    hv = h.cpu().numpy()
    assert np.all(np.abs(hv - ref) <= 16 * U32 * np.abs(ref) + 1e-30)
    # the record: its largest word is max |h|; the words are |h| patterns
    r = rec.cpu().numpy().view(np.uint32)
    assert r.max() == np.max(hv.view(np.uint32) & 0x7FFFFFFF)
    assert np.all(r <= r.max()) and np.count_nonzero(r) <= 256


# (M, N, K): down weight [N][K], K = F
DOWN = [
    (1, 4096, 12288), (8, 4096, 12288), (2, 4096, 12288),     # Qwen3-8B
    (1, 5120, 25600), (8, 5120, 25600), (2, 5120, 25600),     # Qwen3-32B
    (3, 100, 272), (1, 33, 16), (8, 64, 4096), (4, 200, 8192),
]


def _h_and_record(nv, M, K, seed):
    """A SiLU * mul output of realistic spread and its maxima record, from
    the fused gate_up at this K (= F, a multiple of 16) with a small hidden
    width."""
    F = K
    w16 = weights_bf16(31, seed, 2 * F, 256)
    wq = nv.quantize_weight_gate_up(to_dev_bf16(w16))
    x = to_dev_bf16(activations_bf16(31, seed, M, 256, "outlier"))
    h, rec, _ = nv.quantize_linear_silu_mul(x, wq, rmsnorm=True, eps=1e-6)
    return h, rec


@pytest.mark.parametrize("shape", DOWN)
def test_quantize_act_f32(nv, shape):
    M, _, K = shape
    note(f"quantize_act_f32 M={M} K={K}")
    h, rec = _h_and_record(nv, M, K, 1)
    a1 = nv.quantize_act_f32(h, amax=rec)
    a0 = nv.quantize_act_f32(h)
    _sync()
    hv = h.cpu().numpy()
    check_quant(a1, hv)
    check_quant(a0, hv)


@pytest.mark.parametrize("shape", DOWN)
def test_quantize_linear_f32(nv, shape):
    """Every path: the record with the K-slice plan forced (f32_slices = 2),
    only where the activation does not fit one prologue (1) and by the
    default rule (0); no record (the whole-activation kernel or the two
    launches, both on nvfp4_linear's plan: bit-identical to it); fusion off."""
    import torch
    M, N, K = shape
    big = N >= 4096
    note(f"quantize_linear_f32 M={M} N={N} K={K}")
    w16 = weights_bf16(32, N % 1000, N, K)
    wq = nv.quantize_weight(to_dev_bf16(w16))
    if K % 16 == 0 and K >= 16:
        h, rec = _h_and_record(nv, M, K, 2)
    else:
        rng = np.random.default_rng(K)
        h = torch.from_numpy((rng.standard_normal((M, K)) * 0.3).astype(np.float32)).cuda()
        rec = None
    _sync()
    hv = h.cpu().numpy()
    cols = sample_rows(N, 9) if big else None
    try:
        for mode in (2, 1, 0):
            nv.set_option("f32_slices", mode)
            for amax in ([rec, None] if rec is not None else [None]):
                y, xq = nv.quantize_linear_f32(h, wq, amax=amax, out_dtype=torch.bfloat16)
                _sync()
                check_quant(xq, hv)
                check_linear(y, xq, w16, cols)
                if amax is None:
                    yl = nv.linear(xq, wq, out_dtype=torch.bfloat16)
                    _sync()
                    assert np.array_equal(y.cpu().view(torch.int16).numpy(),
                                          yl.cpu().view(torch.int16).numpy())
        nv.set_option("f32_slices", 0)
        nv.set_option("fuse_quant", 0)
        y2, xq2 = nv.quantize_linear_f32(h, wq, amax=rec, out_dtype=torch.bfloat16)
        _sync()
    finally:
        nv.set_option("f32_slices", 0)
        nv.set_option("fuse_quant", 1)
    check_quant(xq2, hv)
    check_linear(y2, xq2, w16, cols)


def test_fused_mlp_graph_replay(nv):
    """gate_up + SiLU * mul and quantize + down (the K-slice path at M = 8,
    Qwen3-32B shapes) captured once and replayed with fresh inputs: every
    replay equals the eager calls bit for bit."""
    import torch
    M, hidden, F = 8, 5120, 25600
    note("fused mlp graph replay")
    wg = nv.quantize_weight_gate_up(to_dev_bf16(weights_bf16(33, 0, 2 * F, hidden)))
    wd = nv.quantize_weight(to_dev_bf16(weights_bf16(33, 1, hidden, F)))
    x = to_dev_bf16(activations_bf16(33, 0, M, hidden, "outlier")).clone()
    h = torch.empty((M, F), dtype=torch.float32, device="cuda")
    rec = torch.empty(256, dtype=torch.int32, device="cuda")
    y = torch.empty((M, hidden), dtype=torch.bfloat16, device="cuda")
    xa = nv.empty_act(M, hidden)
    xb = nv.empty_act(M, F)
    ws = nv.workspace(M, hidden, F, need=max(256, nv._quantize_linear_f32_workspace_bytes(M, hidden, F)))

    def step():
        nv.quantize_linear_silu_mul(x, wg, rmsnorm=True, eps=1e-6, h=h, amax=rec, xq=xa, ws=ws)
        nv.quantize_linear_f32(h, wd, amax=rec, out=y, xq=xb, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for r in range(3):
        x.copy_(to_dev_bf16(activations_bf16(33, 10 + r, M, hidden, "normal" if r else "outlier")))
        torch.empty(1 << 20, device="cuda").fill_(1.0)
        _sync()
        g.replay()
        _sync()
        yg, hg = y.clone(), h.clone()
        step()
        _sync()
        assert np.array_equal(_bits(hg), _bits(h)), f"replay {r}: h"
        assert np.array_equal(yg.cpu().view(torch.int16).numpy(),
                              y.cpu().view(torch.int16).numpy()), f"replay {r}: y"
