"""GPU parity of the NVFP4 quantizers and the tiled layout against the CPU
oracle: codes, E4M3 scale bytes and binary32 tensor-scale bits must be
bit-identical."""

import numpy as np
import pytest

import oracle
from gpu_util import note, pad_dims, tile_weight, to_dev_bf16, to_dev_u8
from workloads import (QWEN3_8B, QWEN3_32B, activations_bf16, bf16_bits, bf16_to_f32,
                       weights_bf16)

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


def _gs_bits(t):
    return t.cpu().numpy().view(np.uint32)[0]


def _assert_act_equal(q, x_f32, per_row=False):
    ref = oracle.quantize(x_f32)
    assert _gs_bits(q.gscale) == np.asarray(ref.gscale, np.float32).view(np.uint32)
    s = q.scales.cpu().numpy()
    c = q.codes.cpu().numpy()
    bad = np.nonzero(s != ref.scales)
    assert bad[0].size == 0, f"scale mismatch at {bad[0][:4]},{bad[1][:4]}"
    bad = np.nonzero(c != ref.codes)
    assert bad[0].size == 0, f"code mismatch at {bad[0][:4]},{bad[1][:4]}"


def test_act_quant_tiny(nv):
    note("act quant M=1 K=512 (tiny workload)")
    x = activations_bf16(1, 0, 1, 512)
    q = nv.quantize_act(to_dev_bf16(x))
    _sync()
    _assert_act_equal(q, bf16_to_f32(x))


@pytest.mark.parametrize("K", sorted({l.K for l in QWEN3_8B + QWEN3_32B} | {5120 * 5}))
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_act_quant_model_shapes(nv, M, K):
    for cfg, kind in ((3, "outlier"), (4, "student_t")):
        note(f"act quant M={M} K={K} {kind}")
        x = activations_bf16(cfg, K % 7, M, K, kind)
        q = nv.quantize_act(to_dev_bf16(x))
        _sync()
        _assert_act_equal(q, bf16_to_f32(x))


def _tie_suite(q=0, width=16 * 160):
    """Rows of bf16 values that drive every E4M3 scale byte and every E2M1
    rounding tie (and its bf16 neighbours) through the quantizer.

    The tensor amax is 2688 * 2^q, so s_g = 2^q and d = s_g * 6 = 6 * 2^q
    exactly.  A block whose maximum is a = 6 v 2^q then has sigma = v exactly
    (6 v has at most 7 significant bits, so a is a bf16 value).  A block with
    maximum 6 * 2^(k+q) has sigma = 2^k, S = 2^k, T = 2^(k+q) and r = 1/T
    exactly, so an element t * 2^(k+q) lands on y = t exactly."""
    amax = 2688.0 * 2.0 ** q
    blocks = []
    first = np.zeros(16, np.float32)
    first[0] = amax
    blocks.append(first)
    grid = oracle.e4m3_decode(np.arange(0x7F))
    sig = list(grid[1:]) + [0.5 * (a + b) for a, b in zip(grid[:-1], grid[1:])]
    for v in sig:
        b = np.zeros(16, np.float32)
        b[0] = 6.0 * v * 2.0 ** q
        b[1] = -0.37 * b[0]
        blocks.append(b)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for t in ties:
        tb = bf16_bits(np.array([t], np.float32))[0]
        for u in (tb, tb + 1, tb - 1):
            f = bf16_to_f32(np.array([u], np.uint16))[0]
            vals += [f, -f]
    vals += [0.0, -0.0, 6.0, -6.0, 0.1, -0.1]
    for k in (-6, -2, 0, 3, 8):
        for j in range(0, len(vals), 15):
            b = np.zeros(16, np.float32)
            b[0] = 6.0 * 2.0 ** (k + q)
            for i, v in enumerate(vals[j:j + 15]):
                b[1 + i] = np.float32(v) * np.float32(2.0 ** (k + q))
            blocks.append(b)
    flat = np.concatenate(blocks)
    flat = np.pad(flat, (0, (-flat.size) % width))
    x = flat.reshape(-1, width)
    return bf16_bits(x)


def test_e2m1_instruction_encoder_exhaustive(nv):
    """The quantizers round y = x * r to E2M1 with gfx950's packed FP4
    conversion at unit scale.  Over every finite binary32 pattern (and its
    negation) it must give the code of the stated rounding rule: nearest,
    ties to the even code, saturating at 6, sign bit from y."""
    note("e2m1 encoder self-check over all finite binary32 patterns")
    bad, seen = nv.selftest_e2m1()
    assert seen == (1 << 32) - (1 << 24)
    assert bad == 0


def test_act_quant_ties_and_every_scale_byte(nv):
    x = _tie_suite()
    assert x.shape[0] <= 8
    xf = bf16_to_f32(x)
    ref = oracle.quantize(xf)
    used = set(np.unique(ref.scales).tolist())
    assert set(range(0x7F)) <= used, sorted(set(range(0x7F)) - used)[:8]
    note(f"act quant tie suite M={x.shape[0]} K={x.shape[1]}")
    q = nv.quantize_act(to_dev_bf16(x))
    _sync()
    _assert_act_equal(q, xf)


def test_act_quant_edges(nv):
    import torch
    for M, K in ((1, 16), (8, 16), (3, 48), (7, 272)):
        note(f"act quant edge M={M} K={K}")
        x = activations_bf16(1, 1, M, K)
        q = nv.quantize_act(to_dev_bf16(x))
        _sync()
        _assert_act_equal(q, bf16_to_f32(x))
    note("act quant all zeros / negative zeros")
    z = np.zeros((2, 64), np.uint16)
    z[1, ::2] = 0x8000
    q = nv.quantize_act(to_dev_bf16(z))
    _sync()
    _assert_act_equal(q, bf16_to_f32(z))
    assert q.gscale.item() == 1.0
    note("act quant strided rows (ldx = K + 64)")
    wide = activations_bf16(2, 0, 4, 4096 + 64)
    xd = to_dev_bf16(wide)[:, :4096]
    assert xd.stride(0) == 4096 + 64
    q = nv.quantize_act(xd)
    _sync()
    _assert_act_equal(q, bf16_to_f32(wide[:, :4096]))
    del torch


def _sync_words(ws):
    return ws[:16].cpu().numpy().view(np.uint32).tolist()


@pytest.mark.parametrize("M,K", [(8, 25600), (3, 8192), (8, 4096), (8, 524288)])
def test_act_quant_multi_workgroup_and_forced_fallback(nv, M, K):
    """Tensors of more than 1024 blocks are spread over several workgroups
    that combine their maxima through the workspace; with the spin limit
    forced to 1 most workgroups give up polling and compute the amax alone.
    Both paths must give the oracle's bits, and leave the record zero."""
    import torch
    x = activations_bf16(4, 9, M, K, "student_t")
    xd = to_dev_bf16(x)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    assert nv.act_workspace_bytes(M, K) == 16
    for spin in (0, 1):
        note(f"act quant multi-workgroup M={M} K={K} spin_limit={spin}")
        nv.set_option("spin_limit", spin)
        try:
            q = nv.quantize_act(xd, ws=ws)
            _sync()
        finally:
            nv.set_option("spin_limit", 0)
        _assert_act_equal(q, bf16_to_f32(x))
        assert _sync_words(ws) == [0, 0, 0, 0]


def test_act_quant_record_reuse_and_graph_replay(nv):
    """One workspace serves consecutive calls of different sizes, and a
    captured quantization replays correctly (inputs refreshed between
    replays, eager work and synchronisation in between)."""
    import torch
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for i, (M, K) in enumerate(((8, 25600), (2, 5120), (8, 12288), (1, 512), (5, 8192))):
        note(f"act quant reuse M={M} K={K}")
        x = activations_bf16(3, i, M, K)
        q = nv.quantize_act(to_dev_bf16(x), ws=ws)
        _sync()
        _assert_act_equal(q, bf16_to_f32(x))
        assert _sync_words(ws) == [0, 0, 0, 0]
    M, K = 8, 12288
    note(f"act quant graph replay M={M} K={K}")
    xin = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    xin.copy_(to_dev_bf16(activations_bf16(3, 0, M, K)))
    q = nv.empty_act(M, K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.quantize_act(xin, out=q, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        nv.quantize_act(xin, out=q, ws=ws)
    for r in range(4):
        x = activations_bf16(4, 20 + r, M, K, "student_t" if r % 2 else "outlier")
        xin.copy_(to_dev_bf16(x))
        torch.empty(1 << 20, device="cuda").fill_(1.0)         # eager work between replays
        _sync()
        g.replay()
        _sync()
        _assert_act_equal(q, bf16_to_f32(x))
        assert _sync_words(ws) == [0, 0, 0, 0]


def _check_weight(nv, w16, rows=None):
    import torch
    N, K = w16.shape
    wq = nv.quantize_weight(to_dev_bf16(w16))
    c, s = nv.unpack_weight(wq)
    _sync()
    wf = bf16_to_f32(w16)
    _, sg = oracle.global_scale(wf)
    assert _gs_bits(wq.gscale) == np.asarray(sg, np.float32).view(np.uint32)
    if rows is None:
        rows = np.arange(N)
    rc, rs = oracle.quantize_blocks(wf[rows], sg)
    gc, gsc = c.cpu().numpy()[rows], s.cpu().numpy()[rows]
    bad = np.nonzero(gsc != rs)
    assert bad[0].size == 0, f"scale mismatch rows {rows[bad[0][:4]]} blocks {bad[1][:4]}"
    bad = np.nonzero(gc != rc)
    assert bad[0].size == 0, f"code mismatch rows {rows[bad[0][:4]]} bytes {bad[1][:4]}"
    del torch
    return wq


def test_weight_quant_tiny_full(nv):
    note("weight quant N=256 K=512 full")
    _check_weight(nv, weights_bf16(1, 0, 256, 512))


@pytest.mark.parametrize("N,K", [(33, 16), (100, 48), (40, 272), (97, 1040), (1, 4096)])
def test_weight_quant_ragged_full_and_padding(nv, N, K):
    note(f"weight quant ragged N={N} K={K}")
    w16 = weights_bf16(1, 3, N, K)
    wq = _check_weight(nv, w16)
    # padding rows / columns of the tiled layout are zero
    codes_rm = oracle.quantize(bf16_to_f32(w16))
    ct, st = tile_weight(codes_rm.codes, codes_rm.scales, N, K)
    assert np.array_equal(wq.codes.cpu().numpy(), ct)
    assert np.array_equal(wq.scales.cpu().numpy(), st)


@pytest.mark.parametrize("lin", range(4))
@pytest.mark.parametrize("family", ["8b", "32b"])
def test_weight_quant_model_shapes_all_rows(nv, family, lin):
    """Every row of every Qwen3-8B and Qwen3-32B projection weight, bit for
    bit: the oracle quantizes the whole weight (in chunks of rows, with the
    tensor scale of the whole weight) and every code and scale byte of the
    GPU's tiled result, unpacked, must match."""
    cfg, shapes = (2, QWEN3_8B) if family == "8b" else (4, QWEN3_32B)
    L = shapes[lin]
    note(f"weight quant {family} {L.name} N={L.N} K={L.K} (all rows)")
    w16 = weights_bf16(cfg, lin, L.N, L.K)
    wq = nv.quantize_weight(to_dev_bf16(w16))
    c, s = nv.unpack_weight(wq)
    _sync()
    gc, gsc = c.cpu().numpy(), s.cpu().numpy()
    del c, s
    wf = bf16_to_f32(w16)
    _, sg = oracle.global_scale(wf)
    assert _gs_bits(wq.gscale) == np.asarray(sg, np.float32).view(np.uint32)
    step = 2048
    for r0 in range(0, L.N, step):
        rc, rs = oracle.quantize_blocks(wf[r0:r0 + step], sg)
        bad = np.nonzero(gsc[r0:r0 + step] != rs)
        assert bad[0].size == 0, f"scale mismatch rows {r0 + bad[0][:4]} blocks {bad[1][:4]}"
        bad = np.nonzero(gc[r0:r0 + step] != rc)
        assert bad[0].size == 0, f"code mismatch rows {r0 + bad[0][:4]} bytes {bad[1][:4]}"


def test_weight_every_scale_byte(nv):
    """The tie suite as a weight (tensor scale 2^-3): every E4M3 byte, every
    E2M1 tie and its bf16 neighbours."""
    w16 = _tie_suite(q=-3, width=16 * 48)
    ref = oracle.quantize(bf16_to_f32(w16))
    assert set(range(0x7F)) <= set(np.unique(ref.scales).tolist())
    note(f"weight quant tie suite N={w16.shape[0]} K={w16.shape[1]}")
    _check_weight(nv, w16)


def test_unpack_matches_test_side_tiling(nv):
    """Random bytes tiled by the test's own reading of the layout come back
    unchanged through the library's inverse tiling."""
    import torch
    rng = np.random.default_rng(3)
    N, K = 70, 784
    codes = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    scales = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    ct, st = tile_weight(codes, scales, N, K)
    from nvfp4_decode_linear_amd import QuantWeight
    q = QuantWeight(to_dev_u8(ct), to_dev_u8(st), torch.ones(1, device="cuda"), N, K)
    note(f"unpack N={N} K={K}")
    c, s = nv.unpack_weight(q)
    _sync()
    assert np.array_equal(c.cpu().numpy(), codes)
    assert np.array_equal(s.cpu().numpy(), scales)
    Np, Kp = pad_dims(N, K)
    assert ct.size == Np * Kp // 2
