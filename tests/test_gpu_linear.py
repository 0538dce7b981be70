"""GPU parity of the NVFP4 W4A4 decode linear against the CPU oracle.

* Unit-scale special case: every block scale 1.0 and both tensor scales 1,
  so every partial sum is a quarter-integer below 2^22 and the binary32
  output must equal the oracle bit for bit, whatever the summation order.
* Real distributions: |y - y_ref| <= 1e-3 * sum_k |x_hat w_hat| per element
  (plus half a bf16 ulp for bf16 output), at full size on sampled output
  columns computed by the oracle from its own quantization.
* Run-to-run bit stability (split-K), knob sweeps, and HIP graph replay.
"""

import numpy as np
import pytest

import oracle
from gpu_util import note, tile_weight, to_dev_bf16, to_dev_u8
from workloads import (QWEN3_8B, QWEN3_32B, WORKLOADS, activations_bf16, bf16_to_f32,
                       weights_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import nvfp4_decode_linear_amd as nv
    yield nv
    for k, v in (("split_k", 0), ("chunks_per_wave", 0), ("nontemporal", 1), ("gemv_max_m", 8),
                 ("waves", 0), ("kernel", 0)):
        nv.set_option(k, v)


def _sync():
    import torch
    torch.cuda.synchronize()


def _unit_operands(nv, M, N, K, seed, scale_bytes=None):
    """Random codes with unit (or given) block scales and tensor scale 1."""
    import torch
    rng = np.random.default_rng(seed)
    xc = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    wc = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    if scale_bytes is None:
        xs = np.full((M, K // 16), 0x38, np.uint8)
        ws = np.full((N, K // 16), 0x38, np.uint8)
    else:
        xs = rng.choice(scale_bytes, (M, K // 16)).astype(np.uint8)
        ws = rng.choice(scale_bytes, (N, K // 16)).astype(np.uint8)
    one = np.array(1.0, np.float32)
    ox, ow = oracle.NVFP4Tensor(xc, xs, one), oracle.NVFP4Tensor(wc, ws, one)
    ct, st = tile_weight(wc, ws, N, K)
    d = torch.device("cuda:0")
    xq = nv.QuantAct(to_dev_u8(xc), to_dev_u8(xs), torch.ones(1, device=d), M, K)
    wq = nv.QuantWeight(to_dev_u8(ct), to_dev_u8(st), torch.ones(1, device=d), N, K)
    return xq, wq, ox, ow


UNIT_SHAPES = [(256, 512), (4096, 4096), (24576, 4096), (4096, 12288), (5120, 8192),
               (100, 1040), (33, 16), (64, 25600)]


KERNELS = {  # name: (kernel option, split_k option, half_tiles option)
    "auto": (0, 0, 0), "valu_stream": (1, 0, 0), "split": (2, 0, 0), "mfma": (3, 1, 1),
    "mfma_split3": (3, 3, 1), "mfma_h16": (3, 0, 2),
}


@pytest.fixture
def kernel(nv, request):
    """Force one GEMV kernel (K slice count, tile height) for the test;
    "auto" is the library's own choice."""
    k, sp, hh = KERNELS[request.param]
    nv.set_option("kernel", k)
    nv.set_option("split_k", sp)
    nv.set_option("half_tiles", hh)
    yield request.param
    nv.set_option("kernel", 0)
    nv.set_option("split_k", 0)
    nv.set_option("half_tiles", 0)


@pytest.mark.parametrize("kernel", ["auto", "split", "mfma", "mfma_split3", "mfma_h16"],
                         indirect=True)
@pytest.mark.parametrize("N,K", UNIT_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_unit_scale_bit_exact(nv, kernel, M, N, K):
    note(f"linear unit-scale kernel={kernel} M={M} N={N} K={K}")
    xq, wq, ox, ow = _unit_operands(nv, M, N, K, seed=M * 7 + N % 13)
    y = nv.linear(xq, wq)
    _sync()
    ref = oracle.linear_ref(ox, ow)
    assert np.all(np.abs(ref) < 2.0 ** 22)
    got = y.cpu().numpy()
    bad = np.nonzero(got.astype(np.float64) != ref)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first at {bad[0][0]},{bad[1][0]}: " \
                             f"{got[bad[0][0], bad[1][0]]} vs {ref[bad[0][0], bad[1][0]]}"


@pytest.mark.parametrize("kernel", ["auto", "valu_stream", "split", "mfma", "mfma_h16"],
                         indirect=True)
@pytest.mark.parametrize("M", [1, 3, 4, 8])
def test_power_of_two_scales_bit_exact(nv, kernel, M):
    """Block scales 2^-2 .. 2^2 keep every partial sum a small dyadic
    rational, still exact in binary32."""
    N, K = 512, 2048
    note(f"linear pow2-scale kernel={kernel} M={M} N={N} K={K}")
    xq, wq, ox, ow = _unit_operands(nv, M, N, K, seed=11 + M,
                                    scale_bytes=[0x28, 0x30, 0x38, 0x40, 0x48])
    y = nv.linear(xq, wq)
    _sync()
    ref = oracle.linear_ref(ox, ow)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def _quantized_pair(nv, cfg, lin, L, M, kind):
    w16 = weights_bf16(cfg, lin, L.N, L.K)
    x16 = activations_bf16(cfg, lin, M, L.K, kind)
    wq = nv.quantize_weight(to_dev_bf16(w16))
    xq = nv.quantize_act(to_dev_bf16(x16))
    return w16, x16, wq, xq


def _check_sampled(nv, y, w16, x16, wq, cols, out_bf16=False):
    """Oracle on sampled output columns: the oracle quantizes the sampled
    weight rows itself (tensor scale from the whole weight)."""
    wf = bf16_to_f32(w16)
    _, sg = oracle.global_scale(wf)
    wc, ws = oracle.quantize_blocks(wf[cols], sg)
    ow = oracle.NVFP4Tensor(wc, ws, np.asarray(sg, np.float32))
    ox = oracle.quantize(bf16_to_f32(x16))
    # the GPU's quantization of the same rows must be the oracle's, bit for bit
    gc, gs = nv.unpack_weight(wq)
    assert np.array_equal(gc.cpu().numpy()[cols], wc)
    assert np.array_equal(gs.cpu().numpy()[cols], ws)
    ref = oracle.linear_ref(ox, ow)
    bound = oracle.tolerance_bound(ox, ow)
    if out_bf16:
        import torch
        got = y.float().cpu().numpy()[:, cols].astype(np.float64)
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)     # bf16 ulp at |ref|
        bound = bound + 0.5 * ulp
        del torch
    else:
        got = y.cpu().numpy()[:, cols].astype(np.float64)
    err = np.abs(got - ref)
    worst = np.max(err / np.maximum(bound, 1e-300))
    assert np.all(err <= bound), f"max err/bound {worst}"
    return worst


def _cols(N, rng, n=384):
    return np.unique(np.concatenate([np.arange(min(N, 64)), np.arange(max(0, N - 64), N),
                                     rng.choice(N, min(N, n), replace=False)]))


def test_tiny_full(nv):
    L = WORKLOADS[1].linears[0]
    note(f"linear tiny M=1 N={L.N} K={L.K} full")
    w16, x16, wq, xq = _quantized_pair(nv, 1, 0, L, 1, "outlier")
    y = nv.linear(xq, wq)
    _sync()
    _check_sampled(nv, y, w16, x16, wq, np.arange(L.N))


@pytest.mark.parametrize("kernel", ["auto", "mfma", "mfma_h16"], indirect=True)
@pytest.mark.parametrize("lin", range(4))
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_8b_shapes_sampled(nv, kernel, lin, M):
    L = QWEN3_8B[lin]
    note(f"linear 8B {L.name} kernel={kernel} M={M} N={L.N} K={L.K}")
    w16, x16, wq, xq = _quantized_pair(nv, 3, lin, L, M, "outlier")
    y = nv.linear(xq, wq)
    _sync()
    _check_sampled(nv, y, w16, x16, wq, _cols(L.N, np.random.default_rng(lin)))


@pytest.mark.parametrize("kernel", ["auto", "mfma", "mfma_h16"], indirect=True)
@pytest.mark.parametrize("lin", range(4))
@pytest.mark.parametrize("M", [1, 4, 8])
def test_32b_shapes_sampled(nv, kernel, lin, M):
    L = QWEN3_32B[lin]
    note(f"linear 32B {L.name} kernel={kernel} M={M} N={L.N} K={L.K}")
    w16, x16, wq, xq = _quantized_pair(nv, 4, lin, L, M, "student_t")
    y = nv.linear(xq, wq)
    _sync()
    _check_sampled(nv, y, w16, x16, wq, _cols(L.N, np.random.default_rng(10 + lin)))


@pytest.mark.parametrize("M", [1, 8])
def test_bf16_output(nv, M):
    import torch
    L = QWEN3_8B[3]
    note(f"linear bf16 out M={M} N={L.N} K={L.K}")
    w16, x16, wq, xq = _quantized_pair(nv, 3, 3, L, M, "outlier")
    y = nv.linear(xq, wq, out_dtype=torch.bfloat16)
    _sync()
    _check_sampled(nv, y, w16, x16, wq, _cols(L.N, np.random.default_rng(5)), out_bf16=True)


@pytest.mark.parametrize("kernel", ["auto", "split", "mfma", "mfma_split3", "mfma_h16"],
                         indirect=True)
@pytest.mark.parametrize("N,K,M", [(1, 16, 1), (33, 16, 8), (100, 1040, 3), (4097, 784, 5),
                                   (31, 25600, 7), (300, 8000, 2)])
def test_ragged_and_degenerate(nv, kernel, N, K, M):
    note(f"linear ragged kernel={kernel} M={M} N={N} K={K}")
    w16 = weights_bf16(1, 7, N, K)
    x16 = activations_bf16(1, 7, M, K)
    wq = nv.quantize_weight(to_dev_bf16(w16))
    xq = nv.quantize_act(to_dev_bf16(x16))
    y = nv.linear(xq, wq)
    _sync()
    _check_sampled(nv, y, w16, x16, wq, np.arange(N))


def test_zero_activation_gives_zero(nv):
    import torch
    L = QWEN3_8B[1]
    note("linear zero activation")
    wq = nv.quantize_weight(to_dev_bf16(weights_bf16(2, 1, L.N, L.K)))
    xq = nv.quantize_act(torch.zeros((2, L.K), dtype=torch.bfloat16, device="cuda"))
    y = nv.linear(xq, wq)
    _sync()
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("kernel", ["auto", "split", "mfma", "mfma_split3", "mfma_h16"],
                         indirect=True)
def test_run_to_run_bit_stable(nv, kernel):
    L = QWEN3_8B[3]
    note(f"linear determinism kernel={kernel} M=8 N={L.N} K={L.K}")
    w16, x16, wq, xq = _quantized_pair(nv, 3, 3, L, 8, "outlier")
    ys = [nv.linear(xq, wq).cpu() for _ in range(5)]
    for y in ys[1:]:
        assert np.array_equal(y.numpy().view(np.uint32), ys[0].numpy().view(np.uint32))


KNOBS = [  # (kernel, split_k, chunks_per_wave, waves)
    (2, 1, 0, 0), (2, 2, 0, 0), (2, 3, 0, 0), (2, 7, 0, 0), (2, 0, 4, 0), (2, 0, 8, 0),
    (2, 0, 12, 0), (2, 0, 16, 0), (2, 0, 4, 8), (2, 0, 16, 8), (2, 0, 4, 16), (2, 0, 8, 16),
    (2, 2, 0, 16), (1, 0, 0, 0), (1, 0, 0, 8), (1, 0, 0, 16), (1, 2, 0, 0), (1, 4, 0, 8),
    (3, 0, 0, 0), (3, 0, 0, 4), (3, 0, 0, 8), (3, 1, 0, 16), (3, 2, 0, 0), (3, 3, 0, 8),
    (3, 5, 0, 4), (3, 16, 0, 0),
]


@pytest.mark.parametrize("kernel,split,cpw,waves", KNOBS)
def test_knobs_keep_results_in_tolerance(nv, kernel, split, cpw, waves):
    L = QWEN3_8B[3]
    note(f"linear knobs kernel={kernel} split_k={split} chunks_per_wave={cpw} waves={waves}")
    nv.set_option("kernel", kernel)
    nv.set_option("split_k", split)
    nv.set_option("chunks_per_wave", cpw)
    nv.set_option("waves", waves)
    try:
        for M in (1, 3, 8):
            w16, x16, wq, xq = _quantized_pair(nv, 3, 3, L, M, "outlier")
            y = nv.linear(xq, wq)
            _sync()
            _check_sampled(nv, y, w16, x16, wq, _cols(L.N, np.random.default_rng(2), 128))
    finally:
        for k in ("kernel", "split_k", "chunks_per_wave", "waves"):
            nv.set_option(k, 0)


def test_ordinary_loads_match_nontemporal(nv):
    L = QWEN3_8B[0]
    note("linear nontemporal on/off")
    w16, x16, wq, xq = _quantized_pair(nv, 3, 0, L, 4, "outlier")
    a = nv.linear(xq, wq).cpu()
    nv.set_option("nontemporal", 0)
    try:
        b = nv.linear(xq, wq).cpu()
    finally:
        nv.set_option("nontemporal", 1)
    assert np.array_equal(a.numpy().view(np.uint32), b.numpy().view(np.uint32))


def test_graph_replay_matches_eager(nv):
    """Activation quantization + linear captured into one HIP graph and
    replayed several times, with eager work in between, against the eager
    result (the split-K counters reset themselves between replays)."""
    import torch
    L = QWEN3_8B[3]
    note(f"linear graph replay N={L.N} K={L.K}")
    w16 = weights_bf16(3, 3, L.N, L.K)
    wq = nv.quantize_weight(to_dev_bf16(w16))
    x = to_dev_bf16(activations_bf16(3, 3, 4, L.K))
    xq = nv.empty_act(4, L.K)
    ws = nv.workspace(4, L.N, L.K)
    y = torch.empty((4, L.N), dtype=torch.float32, device="cuda")
    nv.quantize_act(x, out=xq)
    nv.linear(xq, wq, out=y, ws=ws)
    _sync()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            nv.quantize_act(x, out=xq)
            nv.linear(xq, wq, out=y, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        _sync()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), eager.cpu().numpy().view(np.uint32)), i
        nv.linear(xq, wq, out=y, ws=ws)          # eager call between replays
        _sync()


def test_workspace_shared_across_shapes(nv):
    """One zero-initialised workspace serves calls of different shapes in any
    order: the split-K counters sit in a fixed region, so a small shape never
    reads a larger shape's partial sums as counters."""
    import torch
    shapes = [(5120, 8192, 1), (100, 1040, 1), (4096, 12288, 8), (33, 784, 3), (4096, 4096, 2)]
    need = max(nv.linear_workspace_bytes(M, N, K) for N, K, M in shapes)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    nv.workspace_init(ws)
    for rep in range(2):
        for N, K, M in shapes:
            note(f"shared workspace rep={rep} M={M} N={N} K={K}")
            xq, wq, ox, ow = _unit_operands(nv, M, N, K, seed=N + K + M)
            y = nv.linear(xq, wq, ws=ws)
            _sync()
            assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.linear_ref(ox, ow))
