"""Pins for the oracle's token entropy (closed forms, library routines,
invariances) and checks of the stated readings of the step statistics and
the temperature rule (parity unpinned: the pages give no formula).  CPU
only."""

import numpy as np
import pytest
from scipy import special, stats

from oracle import reset

V_QWEN3 = 151936          # Qwen3 vocabulary size ("Supported models": Qwen3)


def test_uniform_rows_give_log_v():
    for V in (2, 7, 1000, V_QWEN3):
        z = np.full((3, V), 1.25)
        assert np.allclose(reset.token_entropy(z), np.log(V), rtol=1e-13, atol=0)


def test_two_values_give_the_binary_entropy():
    # p = logistic(a - b); H = -p log p - (1 - p) log(1 - p)
    for a, b in [(0.0, 0.0), (2.0, -1.0), (-3.5, 4.0), (30.0, 0.0)]:
        p = 1.0 / (1.0 + np.exp(-(a - b)))
        want = -(special.xlogy(p, p) + special.xlogy(1 - p, 1 - p))
        got = reset.token_entropy(np.array([[a, b]]))[0]
        assert abs(got - want) <= 1e-13 * max(1.0, want) + 1e-300


def test_one_dominant_logit_gives_almost_zero():
    z = np.zeros((1, 4096))
    z[0, 17] = 60.0                      # every other term is e^-60 relative
    h = reset.token_entropy(z)[0]
    assert 0.0 <= h < 4096 * 61 * np.exp(-60.0) * 1.01


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_against_scipy_entropy_of_softmax(seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((4, 5000)) * (2.0 + seed)
    want = stats.entropy(special.softmax(z, axis=-1), axis=-1)
    assert np.allclose(reset.token_entropy(z), want, rtol=1e-12, atol=1e-12)


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((2, 777)) * 5
    h = reset.token_entropy(z)
    assert np.allclose(reset.token_entropy(z + 123.0), h, rtol=1e-12)
    assert np.allclose(reset.token_entropy(z[:, rng.permutation(777)]), h, rtol=1e-12)


def test_step_statistics_reading():
    # the mean over the step so far, restarting after a closed step
    s, c = np.zeros(2), np.zeros(2)
    seq = [(1.0, 0), (3.0, 0), (2.0, 1), (4.0, 0)]
    means = []
    for h, ended in seq:
        s, c, hs = reset.step_update(s, c, np.array([h, h]), np.array([ended, 0]))
        means.append(hs.tolist())
    assert [m[0] for m in means] == [1.0, 2.0, 2.0, 3.0]
    assert [m[1] for m in means] == [1.0, 2.0, 2.0, 2.5]


def test_temperature_rule_reading():
    t = reset.temperature(np.array([0.1, 0.9, 0.9, 0.9]), np.array([5.0, 0.3, 1.1, 50.0]),
                          t_low=0.1, tau0=0.55, t_base=0.6, t_max=1.5)
    assert np.allclose(t, [0.1, 0.6, 0.6 * 1.1 / 0.55, 1.5])


def test_scale_logits_is_one_division():
    z = np.array([[1.0, -3.0, 7.5]], np.float32)
    out = reset.scale_logits(z, [0.3])
    assert out.dtype == np.float32
    assert np.array_equal(out, z / np.float32(0.3))
