"""The layer-stack driver (nvfp4_stack_*): the graph-replayed decode step
against the same step issued op by op through the C ABI (bit-identical: the
same kernels in the same order), replays with fresh inputs and eager work in
between, and, teacher-forced on the first and last layer, every op of the
step against the oracle (the quantizers bit-exact given their input, the
linears within the tolerance bound).  Toy widths check every output; the
Qwen3-32B decoder shapes (two layers at M = 1 and M = 8) check every op of
both layers, the linears on sampled output columns; and the 64-layer
Qwen3-32B stack the bench times is checked at full depth (graph against call
by call, bit for bit; layers 0, 31 and 63 teacher-forced against the
oracle)."""

import numpy as np
import pytest

import oracle
from gpu_util import note, to_dev_bf16
from parity_util import check_linear as _check_linear, check_quant as _check_quant
from parity_util import sample_rows as _sample_rows
from workloads import activations_bf16, bf16_to_f32, weights_bf16

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
CONFIGS = [  # M, hidden, qkv_n, q_cols, ffn, layers
    (2, 512, 768, 512, 1024, 3),
    (1, 256, 384, 256, 512, 2),
    (8, 512, 640, 384, 768, 2),
    # M = 8 at the 32B hidden width with a small FFN: 8 x 5120 / 16 = 2560
    # activation blocks, past the fused prologue, so the RMS norm and the q
    # slice are quantized by their own kernels on the shared workspace
    (8, 5120, 1024, 1024, 512, 2),
    # gate_up weights in plain row order: gate_up writes bf16 and the SiLU
    # quantizer runs on its own (every other config fuses it)
    (2, 256, 384, 256, 528, 2),
]
# The Qwen3-32B decoder shapes (hidden 5120, QKV 10240, q slice 8192, FFN
# 25600) of the 64-layer decode step that the "ReSET" GitHub README's demo
# caption times (batch 1, graph replay, 1,500 tokens); two layers, at one row
# and at eight.
CONFIGS_32B = [
    (1, 5120, 10240, 8192, 25600, 2),
    (8, 5120, 10240, 8192, 25600, 2),
]


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


def _fused(cfg):
    return cfg[4] != 528          # the one config kept on the unfused SiLU path


def _weights(nv, cfg):
    M, hidden, qkv_n, q_cols, ffn, layers = cfg
    shapes = [(qkv_n, hidden), (hidden, q_cols), (2 * ffn, hidden), (hidden, ffn)]
    src, q = [], []
    for l in range(layers):
        w16 = [weights_bf16(6, 10 * l + j, N, K) for j, (N, K) in enumerate(shapes)]
        src.append(w16)
        q.append(tuple(nv.quantize_weight_gate_up(to_dev_bf16(w)) if j == 2 and _fused(cfg)
                       else nv.quantize_weight(to_dev_bf16(w)) for j, w in enumerate(w16)))
    return src, q


def _eager(nv, cfg, wq, x, trace=False):
    """The step call by call through the binding (the calls the stack makes:
    RMS norm + quantize + QKV, quantize + O, then with interleaved gate_up
    weights RMS norm + quantize + gate_up + SiLU * mul and quantize + down,
    else RMS norm + quantize + gate_up, SiLU * mul + quantize, down);
    with trace, the inputs and outputs of every op of every layer."""
    import torch
    M, hidden, qkv_n, q_cols, ffn, layers = cfg
    ops = []
    cur = x
    for l in range(layers):
        qkv_w, o_w, gu_w, dn_w = wq[l]
        h1 = torch.empty((M, hidden), dtype=torch.float32, device="cuda")
        qkv, a1 = nv.rmsnorm_quantize_linear(cur, qkv_w, 1e-6, out_dtype=torch.bfloat16, h_out=h1)
        o, a2 = nv.quantize_linear(qkv[:, :q_cols], o_w, out_dtype=torch.bfloat16)
        h3 = torch.empty((M, hidden), dtype=torch.float32, device="cuda")
        if gu_w.gate_up:
            gu = torch.empty((M, 2 * ffn), dtype=torch.bfloat16, device="cuda") if trace else None
            h4, rec, a3 = nv.quantize_linear_silu_mul(o, gu_w, rmsnorm=True, eps=1e-6, gu_out=gu,
                                                      xh_out=h3)
            dn, a4 = nv.quantize_linear_f32(h4, dn_w, amax=rec, out_dtype=torch.bfloat16)
        else:
            gu, a3 = nv.rmsnorm_quantize_linear(o, gu_w, 1e-6, out_dtype=torch.bfloat16, h_out=h3)
            h4 = torch.empty((M, ffn), dtype=torch.float32, device="cuda")
            a4 = nv.silu_mul_quantize_act(gu, h_out=h4)
            dn = nv.linear(a4, dn_w, out_dtype=torch.bfloat16)
        if trace:
            ops.append(dict(x=cur, h1=h1, a1=a1, qkv=qkv, a2=a2, o=o, h3=h3, a3=a3, gu=gu, h4=h4,
                            a4=a4, dn=dn))
        cur = dn
    return cur, ops


@pytest.mark.parametrize("cfg", CONFIGS + CONFIGS_32B)
def test_stack_graph_matches_op_by_op(nv, cfg):
    import torch
    M, hidden, qkv_n, q_cols, ffn, layers = cfg
    note(f"stack graph vs eager cfg={cfg}")
    src, wq = _weights(nv, cfg)
    x = torch.empty((M, hidden), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, hidden), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(activations_bf16(7, 0, M, hidden, "normal")))
    st = nv.Stack(M, hidden, qkv_n, q_cols, ffn, wq, x, y)
    try:
        for r in range(3):
            x.copy_(to_dev_bf16(activations_bf16(7, r, M, hidden, "normal" if r else "outlier")))
            torch.empty(1 << 20, device="cuda").fill_(2.0)      # eager work between replays
            _sync()
            ref, _ = _eager(nv, cfg, wq, x)
            _sync()
            st.run(1)
            _sync()
            assert np.array_equal(y.cpu().view(torch.int16).numpy(),
                                  ref.cpu().view(torch.int16).numpy()), f"replay {r}"
            y.zero_()
            st.run_eager()
            _sync()
            assert np.array_equal(y.cpu().view(torch.int16).numpy(),
                                  ref.cpu().view(torch.int16).numpy()), f"eager {r}"
        st.run(5)                                          # replays back to back
        _sync()
        assert np.array_equal(y.cpu().view(torch.int16).numpy(),
                              ref.cpu().view(torch.int16).numpy())
    finally:
        st.close()


@pytest.mark.parametrize("cfg", CONFIGS + CONFIGS_32B)
def test_stack_ops_teacher_forced_vs_oracle(nv, cfg):
    import torch
    M, hidden, qkv_n, q_cols, ffn, layers = cfg
    big = cfg in CONFIGS_32B
    note(f"stack teacher-forced cfg={cfg}: weights")
    src, wq = _weights(nv, cfg)
    x = to_dev_bf16(activations_bf16(7, 5, M, hidden, "outlier"))
    _, ops = _eager(nv, cfg, wq, x, trace=True)
    _sync()
    for l in range(layers) if big else sorted({0, layers - 1}):
        note(f"stack teacher-forced layer {l} cfg={cfg}")
        _teacher_forced_layer(nv, cfg, ops[l], src[l], l, big)


def _teacher_forced_layer(nv, cfg, t, w16, l, big):
    """Every op of one traced layer against the oracle, each on the GPU's own
    input to that op: the norms within their ulp bounds, the quantizers
    bit-exact, the linears within the tolerance (sampled output columns when
    big)."""
    import torch
    M, hidden, qkv_n, q_cols, ffn, layers = cfg
    xin = bf16_to_f32(t["x"].cpu().view(torch.int16).numpy().view(np.uint16))
    h1 = t["h1"].cpu().numpy()
    ref = oracle.rms_norm_rows(xin.astype(np.float64))
    assert np.all(np.abs(h1 - ref) <= 40 * U32 * np.abs(ref) + 1e-38)
    _check_quant(t["a1"], h1)
    cs = (lambda N, j: _sample_rows(N, 100 * l + j)) if big else (lambda N, j: None)
    _check_linear(t["qkv"], t["a1"], w16[0], cs(qkv_n, 0))
    qs = bf16_to_f32(t["qkv"].cpu().view(torch.int16).numpy().view(np.uint16))[:, :q_cols]
    _check_quant(t["a2"], qs)
    _check_linear(t["o"], t["a2"], w16[1], cs(hidden, 1))
    oin = bf16_to_f32(t["o"].cpu().view(torch.int16).numpy().view(np.uint16))
    h3 = t["h3"].cpu().numpy()
    ref = oracle.rms_norm_rows(oin.astype(np.float64))
    assert np.all(np.abs(h3 - ref) <= 40 * U32 * np.abs(ref) + 1e-38)
    _check_quant(t["a3"], h3)
    _check_linear(t["gu"], t["a3"], w16[2], cs(2 * ffn, 2))
    gin = bf16_to_f32(t["gu"].cpu().view(torch.int16).numpy().view(np.uint16))
    h4 = t["h4"].cpu().numpy()
    ref = oracle.silu_mul(gin.astype(np.float64))
    assert np.all(np.abs(h4 - ref) <= 16 * U32 * np.abs(ref) + 1e-30)
    if _fused(cfg):
        # the fused epilogue's h is the standalone SiLU quantizer's on the same bf16 gu
        h4s = torch.empty((M, ffn), dtype=torch.float32, device="cuda")
        nv.silu_mul_quantize_act(t["gu"], h_out=h4s)
        assert np.array_equal(h4.view(np.uint32), h4s.cpu().numpy().view(np.uint32))
    _check_quant(t["a4"], h4)
    _check_linear(t["dn"], t["a4"], w16[3], cs(hidden, 3))


@pytest.mark.parametrize("M", [1, 8])
def test_stack_qwen3_32b_full_depth(nv, M):
    """The 64-layer Qwen3-32B stack the bench times (hidden 5120, QKV 10240,
    q slice 8192, FFN 25600): one seeded layer's weights copied on the
    device into 64 distinct layers; the graph-replayed step bit-identical to
    the same step call by call at full depth, and layers 0, 31 and 63
    teacher-forced against the oracle (sampled output columns)."""
    import torch
    hidden, qkv_n, q_cols, ffn, layers = 5120, 10240, 8192, 25600, 64
    cfg = (M, hidden, qkv_n, q_cols, ffn, layers)
    note(f"stack full depth M={M}: weights")
    shapes = [(qkv_n, hidden), (hidden, q_cols), (2 * ffn, hidden), (hidden, ffn)]
    w16 = [weights_bf16(9, j, N, K) for j, (N, K) in enumerate(shapes)]
    q0 = tuple(nv.quantize_weight_gate_up(to_dev_bf16(w)) if j == 2
               else nv.quantize_weight(to_dev_bf16(w)) for j, w in enumerate(w16))
    wq = [q0] + [tuple(nv.QuantWeight(w.codes.clone(), w.scales.clone(), w.gscale.clone(), w.N,
                                      w.K, w.gate_up) for w in q0) for _ in range(layers - 1)]
    x = to_dev_bf16(activations_bf16(9, M, M, hidden, "normal"))
    y = torch.empty((M, hidden), dtype=torch.bfloat16, device="cuda")
    _sync()
    note(f"stack full depth M={M}: graph and call by call")
    st = nv.Stack(M, hidden, qkv_n, q_cols, ffn, wq, x, y)
    try:
        st.run(2)
        _sync()
        ref, ops = _eager(nv, cfg, wq, x, trace=True)
        _sync()
        assert np.array_equal(y.cpu().view(torch.int16).numpy(),
                              ref.cpu().view(torch.int16).numpy())
        assert np.all(np.isfinite(y.float().cpu().numpy()))
    finally:
        st.close()
    for l in (0, 31, 63):
        note(f"stack full depth M={M}: teacher-forced layer {l}")
        _teacher_forced_layer(nv, cfg, ops[l], w16, l, True)
