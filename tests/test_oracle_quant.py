"""Pins for the oracle's quantizer and dequantizer: a hand-worked block,
invariants that hold for every input, and metamorphic relations.  CPU only."""

import numpy as np
import pytest

from oracle import (dequantize, e2m1_decode, e4m3_decode, global_scale, quantize,
                    quantize_blocks, unpack_nibbles)
from workloads import activations_bf16, bf16_bits, bf16_to_f32, weights_bf16


def _load_worked(golden):
    rows = golden("worked_block.txt")
    x = np.zeros((2, 32), np.float32)
    codes = np.zeros((2, 32), np.uint8)
    scales = {}
    gs = None
    for r in rows:
        if r[0] == "x":
            x[int(r[1]), int(r[2])] = np.float32(float(r[3]))
        elif r[0] == "code":
            codes[int(r[1]), int(r[2])] = int(r[3])
        elif r[0] == "scale":
            scales[(int(r[1]), int(r[2]))] = int(r[3], 16)
        elif r[0] == "gscale":
            gs = np.float32(float(r[1]))
    sc = np.array([[scales[(i, j)] for j in range(2)] for i in range(2)], np.uint8)
    return x, codes, sc, gs


def test_worked_block(golden):
    x, codes, sc, gs = _load_worked(golden)
    q = quantize(x)
    assert q.gscale == gs
    assert np.array_equal(q.scales, sc)
    assert np.array_equal(unpack_nibbles(q.codes), codes)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 lies halfway between two bf16 values: ties go to even (1.0);
    # 1 + 3 * 2^-8 lies halfway as well and rounds up to 1 + 2^-6.
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0], np.float32)
    got = bf16_to_f32(bf16_bits(x))
    assert got.tolist() == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.0]


def _rand(seed, R, K, scale=1.0):
    rng = np.random.default_rng(seed)
    return bf16_to_f32(bf16_bits(rng.standard_normal((R, K)).astype(np.float32) * np.float32(scale)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_amax_block_invariant(seed):
    x = _rand(seed, 8, 512, 3.0)
    q = quantize(x)
    r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q.scales[r, k // 16] == 0x7E
    c = unpack_nibbles(q.codes)[r, k]
    assert c == (0xF if x[r, k] < 0 else 0x7)


@pytest.mark.parametrize("seed", [3, 4])
def test_normal_range_blocks_hit_six(seed):
    x = _rand(seed, 16, 1024)
    x[:, 64:128] *= np.float32(1e-3)              # push some blocks down the E4M3 range
    q = quantize(x)
    _, sg = global_scale(x)
    sigma = np.max(np.abs(x.reshape(16, -1, 16)), axis=2) / np.float32(sg * np.float32(6))
    codes = unpack_nibbles(q.codes).reshape(16, -1, 16)
    idx = np.argmax(np.abs(x.reshape(16, -1, 16)), axis=2)
    cmax = np.take_along_axis(codes, idx[:, :, None], axis=2)[:, :, 0]
    normal = sigma >= 2.0 ** -6
    assert normal.sum() > 100
    assert np.all((cmax[normal] & 7) == 7)


@pytest.mark.parametrize("seed", [5, 6])
def test_reconstruction_error_bound(seed):
    """|x - x_hat| <= T * (1 + 2^-19) where T = S * s_g: at most a half-gap
    of the E2M1 grid (<= 1 in y units) or a saturation error (<= 0.4)."""
    x = _rand(seed, 8, 2048, 2.0)
    x[:, :32] *= np.float32(1e-4)
    q = quantize(x)
    xh = dequantize(q)
    T = np.repeat(e4m3_decode(q.scales) * float(q.gscale), 16, axis=1)
    assert np.all(np.abs(x - xh) <= T * (1 + 2.0 ** -19))


def test_zero_block_and_zero_tensor():
    x = _rand(7, 2, 64)
    x[1, 16:32] = 0
    q = quantize(x)
    assert q.scales[1, 1] == 0
    assert np.all(unpack_nibbles(q.codes)[1, 16:32] == 0)
    z = np.zeros((3, 32), np.float32)
    qz = quantize(z)
    assert qz.gscale == np.float32(1.0)
    assert np.all(qz.scales == 0) and np.all(qz.codes == 0)
    zn = -z
    assert np.all(unpack_nibbles(quantize(zn).codes) == 8)


@pytest.mark.parametrize("k", [-20, -3, 1, 7])
def test_power_of_two_scaling(k):
    x = _rand(8, 4, 256)
    q0 = quantize(x)
    q1 = quantize(x * np.float32(2.0 ** k))
    assert np.array_equal(q0.codes, q1.codes)
    assert np.array_equal(q0.scales, q1.scales)
    assert q1.gscale == np.float32(q0.gscale * np.float32(2.0 ** k))


def test_negation_flips_only_sign_bits():
    x = _rand(9, 4, 256)
    q0 = quantize(x)
    q1 = quantize(-x)
    assert np.array_equal(q0.scales, q1.scales) and q0.gscale == q1.gscale
    assert np.array_equal(unpack_nibbles(q0.codes) ^ 8, unpack_nibbles(q1.codes))


def test_row_and_block_permutation():
    x = _rand(10, 6, 256)
    q = quantize(x)
    p = np.random.default_rng(0).permutation(6)
    qp = quantize(x[p])
    assert np.array_equal(qp.codes, q.codes[p]) and np.array_equal(qp.scales, q.scales[p])
    bp = np.random.default_rng(1).permutation(16)
    xb = x.reshape(6, 16, 16)[:, bp].reshape(6, 256)
    qb = quantize(xb)
    assert np.array_equal(qb.scales, q.scales[:, bp])
    assert np.array_equal(unpack_nibbles(qb.codes).reshape(6, 16, 16),
                          unpack_nibbles(q.codes).reshape(6, 16, 16)[:, bp])


def test_whole_tensor_scale_couples_rows():
    """A row's codes depend on its batchmates through the tensor scale; the
    per-row flag removes the coupling."""
    x = _rand(11, 2, 128)
    x[1] *= np.float32(64.0)
    alone = quantize(x[:1])
    both = quantize(x)
    assert not np.array_equal(both.scales[0], alone.scales[0])
    per_row = quantize(x, per_row=True)
    assert np.array_equal(per_row.scales[0], alone.scales[0])
    assert np.array_equal(per_row.codes[0], alone.codes[0])
    assert per_row.gscale[0] == alone.gscale


def test_quantize_blocks_given_scale_matches_quantize():
    x = _rand(12, 5, 512)
    q = quantize(x)
    c, s = quantize_blocks(x[2:4], q.gscale)
    assert np.array_equal(c, q.codes[2:4]) and np.array_equal(s, q.scales[2:4])


def test_dequantize_closed_form_on_crafted_codes():
    from oracle import NVFP4Tensor
    codes = np.arange(32, dtype=np.uint8) % 16
    packed = (codes[0::2] | (codes[1::2] << 4))[None, :]
    q = NVFP4Tensor(packed, np.array([[0x38, 0x7E]], np.uint8), np.array(0.5, np.float32))
    want = np.concatenate([e2m1_decode(codes[:16]) * 1.0, e2m1_decode(codes[16:]) * 448.0]) * 0.5
    assert np.array_equal(dequantize(q)[0], want)


def test_workload_generators_are_deterministic_and_shaped():
    w = weights_bf16(2, 1, 64, 256)
    assert w.dtype == np.uint16 and w.shape == (64, 256)
    assert np.array_equal(w, weights_bf16(2, 1, 64, 256))
    x8 = activations_bf16(2, 1, 8, 512)
    x2 = activations_bf16(2, 1, 2, 512)
    assert np.array_equal(x8[:2], x2)
    xf = bf16_to_f32(x8)
    big = np.abs(xf).max(axis=0) > 8
    assert 3 <= big.sum() <= 8          # round(0.01 * 512) = 5 outlier channels
