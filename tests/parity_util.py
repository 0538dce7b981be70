"""Parity checks shared by the GPU tests: a quantized activation against
the oracle's quantizer (bit-exact), and a linear's output against the
oracle's linear on the GPU's own quantized activation (within the tolerance
bound plus the output's bf16 rounding)."""

import numpy as np

import oracle
from workloads import bf16_to_f32


def oracle_act(a):
    return oracle.NVFP4Tensor(a.codes.cpu().numpy(), a.scales.cpu().numpy(),
                              np.asarray(a.gscale.cpu().numpy()[0], np.float32))


def check_quant(a, h32):
    ref = oracle.quantize(h32)
    assert np.array_equal(a.codes.cpu().numpy(), ref.codes)
    assert np.array_equal(a.scales.cpu().numpy(), ref.scales)
    assert a.gscale.cpu().numpy().view(np.uint32)[0] == np.asarray(ref.gscale,
                                                                   np.float32).view(np.uint32)


def sample_rows(N, seed, n=256):
    """Output columns checked at the large shapes: both ends of the row range
    (the first and the ragged last tiles) and a random sample."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(N, 48)), np.arange(max(0, N - 48), N),
                                     rng.choice(N, min(N, n), replace=False)]))


def check_linear(y_bf16, a, w16, cols=None):
    """The linear's bf16 output against the oracle on the GPU's quantized
    activation (itself checked against the oracle quantizer before); the
    oracle quantizes the weight rows (all, or the sampled `cols`) itself,
    with the tensor scale of the whole weight."""
    wf = bf16_to_f32(w16)
    if cols is None:
        ow = oracle.quantize(wf)
    else:
        _, sg = oracle.global_scale(wf)
        wc, ws = oracle.quantize_blocks(wf[cols], sg)
        ow = oracle.NVFP4Tensor(wc, ws, np.asarray(sg, np.float32))
    ox = oracle_act(a)
    ref = oracle.linear_ref(ox, ow)
    bound = oracle.tolerance_bound(ox, ow) + 0.5 * np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    got = y_bf16.float().cpu().numpy().astype(np.float64)
    if cols is not None:
        got = got[:, cols]
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300))}"
