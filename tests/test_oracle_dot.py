"""Pins for the oracle's linear: exact rational sums, an integer closed form
in the unit-scale case, and the tolerance bound.  CPU only."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (NVFP4Tensor, linear_exact, linear_ref, quantize, rms_norm_rows, silu_mul,
                    tolerance_bound)
from workloads import activations_bf16, bf16_to_f32, weights_bf16


@pytest.mark.parametrize("M,N,K", [(1, 3, 16), (2, 5, 32), (8, 16, 64)])
def test_fp64_matmul_vs_exact_rationals(M, N, K):
    x = bf16_to_f32(activations_bf16(1, 0, M, K))
    w = bf16_to_f32(weights_bf16(1, 0, N, K))
    xq, wq = quantize(x), quantize(w)
    ref = linear_ref(xq, wq)
    ex = linear_exact(xq, wq)
    bound = tolerance_bound(xq, wq, rel=1.0) * K * 2.0 ** -52
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(ref[m, n])) - ex[m][n]) <= Fraction(float(bound[m, n]))


def _unit_scale(codes_mk):
    """NVFP4 tensor with the given 4-bit codes, every block scale 1.0 (0x38)
    and tensor scale 1."""
    R, K = codes_mk.shape
    packed = (codes_mk[:, 0::2] | (codes_mk[:, 1::2] << 4)).astype(np.uint8)
    return NVFP4Tensor(packed, np.full((R, K // 16), 0x38, np.uint8), np.array(1.0, np.float32))


def test_unit_scale_integer_closed_form(golden):
    """With unit scales every product is (2a)(2w)/4 for small integers 2a,
    2w from the E2M1 table, so y is an exact quarter-integer computed here
    with integer arithmetic only."""
    table = {int(c): float(v) for c, v in golden("e2m1_values.txt")}
    twice = np.array([int(round(2 * table[c])) for c in range(16)], np.int64)
    rng = np.random.default_rng(5)
    M, N, K = 3, 7, 96
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    want = np.zeros((M, N), np.int64)
    for m in range(M):
        for n in range(N):
            want[m, n] = sum(int(twice[cx[m, k]]) * int(twice[cw[n, k]]) for k in range(K))
    got = linear_ref(_unit_scale(cx), _unit_scale(cw))
    assert np.array_equal(got * 4, want.astype(np.float64))


def test_tolerance_bound_definition():
    x = bf16_to_f32(activations_bf16(1, 0, 2, 64))
    w = bf16_to_f32(weights_bf16(1, 0, 3, 64))
    xq, wq = quantize(x), quantize(w)
    b = tolerance_bound(xq, wq)
    ex = linear_exact(xq, wq)
    # The bound is 1e-3 times the sum of |products|, which is at least |y|.
    for m in range(2):
        for n in range(3):
            assert b[m, n] >= 1e-3 * abs(float(ex[m][n])) and b[m, n] > 0


def test_rms_norm_vs_torch():
    x = np.random.default_rng(0).standard_normal((3, 640)) * 7.0
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (640,), eps=1e-6).numpy()
    assert np.allclose(rms_norm_rows(x), ref, rtol=1e-14, atol=0)


def test_silu_mul_vs_torch():
    gu = np.random.default_rng(1).standard_normal((2, 512)) * 4.0
    t = torch.from_numpy(gu)
    ref = (torch.nn.functional.silu(t[:, :256]) * t[:, 256:]).numpy()
    assert np.allclose(silu_mul(gu), ref, rtol=1e-14, atol=1e-300)
