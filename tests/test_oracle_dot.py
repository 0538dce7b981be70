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


def _golden_values(golden):
    """E2M1 code -> value and E4M3 byte -> value from the spec tables under
    tests/golden/ (not from the oracle's decoders)."""
    e2 = {int(c): Fraction(v) for c, v in golden("e2m1_values.txt")}
    e4 = {int(b, 16): Fraction(v) for b, v in golden("e4m3_landmarks.txt") if v != "nan"}
    return e2, e4


def _sum_abs_products(cx, sx, gx, cw, sw, gw, e2, e4):
    """sum_k |x_hat[m,k] * w_hat[n,k]| in exact rationals, decoding with the
    golden tables: x_hat = e2m1(code) * e4m3(block scale) * tensor scale."""
    M, K = cx.shape
    N = cw.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        xh = [e2[int(cx[m, k])] * e4[int(sx[m, k // 16])] * gx for k in range(K)]
        for n in range(N):
            out[m][n] = sum((abs(a * e2[int(cw[n, k])] * e4[int(sw[n, k // 16])] * gw)
                             for k, a in enumerate(xh)), Fraction(0))
    return out


def _tensor(codes, scales, g):
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return NVFP4Tensor(packed, scales.astype(np.uint8), np.array(g, np.float32))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tolerance_bound_exact_rationals(golden, seed):
    """tolerance_bound(rel=1) is exactly sum_k |x_hat w_hat| (every term is a
    dyadic rational with few bits, so the float64 sum is exact here), and the
    default rel is 1e-3: pinned against sums built from the spec tables with
    distinct block scales per (row, block) and distinct tensor scales, so a
    dropped abs, a missing scale, a transposed operand or a wrong rel fails."""
    e2, e4 = _golden_values(golden)
    rng = np.random.default_rng(40 + seed)
    M, N, K = 3, 5, 64
    scale_bytes = np.array([0x30, 0x38, 0x39, 0x3F, 0x40, 0x08, 0x78])
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sx = rng.choice(scale_bytes, (M, K // 16))
    sw = rng.choice(scale_bytes, (N, K // 16))
    gx, gw = Fraction(3, 4), Fraction(3)
    want = _sum_abs_products(cx, sx, gx, cw, sw, gw, e2, e4)
    xq, wq = _tensor(cx, sx, 0.75), _tensor(cw, sw, 3.0)
    b1 = tolerance_bound(xq, wq, rel=1.0)
    b = tolerance_bound(xq, wq)
    assert b1.shape == (M, N)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(b1[m, n])) == want[m][n]
            assert b[m, n] == 1e-3 * float(want[m][n])


def test_tolerance_bound_is_not_the_output():
    """Sign flips change y but not the bound; exact cancellation gives y = 0
    with a positive bound (the bound sums magnitudes, not the signed dot)."""
    K = 32
    cx = np.zeros((1, K), np.uint8)
    cx[0, :2] = [0x2, 0x2]                        # +1, +1
    cw = np.zeros((2, K), np.uint8)
    cw[0, :2] = [0x4, 0xC]                        # +2, -2: cancels
    cw[1, :2] = [0x4, 0x4]                        # +2, +2
    ones_x = np.full((1, K // 16), 0x38, np.uint8)
    ones_w = np.full((2, K // 16), 0x38, np.uint8)
    xq, wq = _tensor(cx, ones_x, 1.0), _tensor(cw, ones_w, 1.0)
    y = linear_ref(xq, wq)
    b = tolerance_bound(xq, wq, rel=1.0)
    assert y.tolist() == [[0.0, 4.0]]
    assert b.tolist() == [[4.0, 4.0]]


def test_rms_norm_vs_torch():
    x = np.random.default_rng(0).standard_normal((3, 640)) * 7.0
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (640,), eps=1e-6).numpy()
    assert np.allclose(rms_norm_rows(x), ref, rtol=1e-14, atol=0)


def test_silu_mul_vs_torch():
    gu = np.random.default_rng(1).standard_normal((2, 512)) * 4.0
    t = torch.from_numpy(gu)
    ref = (torch.nn.functional.silu(t[:, :256]) * t[:, 256:]).numpy()
    assert np.allclose(silu_mul(gu), ref, rtol=1e-14, atol=1e-300)
