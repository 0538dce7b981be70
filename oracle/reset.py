"""Token entropy, step entropy and the decoding temperature of ReSET's
step-aware temperature scaling: the plain definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages say: ReSET is a logits processor ("ReSET" GitHub README,
section "Core components", item 1) that estimates the uncertainty of the
current reasoning step online and sets the decoding temperature from both a
token-level and a step-level entropy; the arXiv abstract adds why: NVFP4
quantization makes sampling go wrong more often at low-entropy (symbolic)
tokens and concentrates probability on too few tokens in uncertain steps.
The README's "Run benchmarks" command names two per-model hyper-parameters,
t_low and tau0 (0.1 and 0.5505 in its example).  No formula is given.

Readings (the plainest ones consistent with that; the aggregation and the
rule are "parity unpinned": nothing on the pages fixes them):

* token entropy: the Shannon entropy, in nats, of softmax(z) over the whole
  vocabulary row, H = log(sum_v e^(z_v - m)) - sum_v e^(z_v - m) (z_v - m)
  / sum_v e^(z_v - m) with m = max_v z_v (the definition, shifted so that no
  exponential overflows);
* step entropy: the mean token entropy over the tokens of the current
  reasoning step so far, this token included.  A step ends where the
  caller says it does (the sampled token closed a step, e.g. a blank line);
  the mean restarts at the next token;
* temperature: t_low for a token whose entropy is below tau0 (a confident,
  symbolic token is decoded almost greedily); otherwise the base
  temperature, raised in proportion to the step entropy once that exceeds
  tau0 and capped at t_max: T = min(t_max, t_base * max(1, H_step / tau0));
* the processed logits are z / T, one correctly rounded binary32 division
  per element.

Pins: token_entropy against closed forms (uniform rows give log V, two
values give the binary entropy of the logistic), against scipy's entropy of
scipy's softmax (library routines), and against invariances (a shift of all
logits, a permutation); temperature and step_update are parity unpinned.
"""

from __future__ import annotations

import numpy as np


def token_entropy(logits: np.ndarray) -> np.ndarray:
    """Entropy (nats) of softmax of each row of logits [M][V], float64."""
    z = np.asarray(logits, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    d = z - m
    e = np.exp(d)
    s = np.sum(e, axis=-1)
    t = np.sum(e * d, axis=-1)
    return np.log(s) - t / s


def step_update(state_sum: np.ndarray, state_count: np.ndarray, h_token: np.ndarray,
                step_ended: np.ndarray):
    """One token of the online step statistics, per row.  step_ended[m] != 0
    means the previous token of row m closed a step, so the running sum and
    count restart before this token is added.  Returns (new_sum, new_count,
    step_entropy) with step_entropy = new_sum / new_count (float64)."""
    s = np.where(np.asarray(step_ended) != 0, 0.0, np.asarray(state_sum, np.float64))
    c = np.where(np.asarray(step_ended) != 0, 0.0, np.asarray(state_count, np.float64))
    s = s + np.asarray(h_token, np.float64)
    c = c + 1.0
    return s, c, s / c


def temperature(h_token, h_step, t_low: float, tau0: float, t_base: float, t_max: float):
    """The reading of the temperature rule above, per row (float64)."""
    h_token = np.asarray(h_token, np.float64)
    h_step = np.asarray(h_step, np.float64)
    boost = np.minimum(t_max, t_base * np.maximum(1.0, h_step / tau0))
    return np.where(h_token < tau0, t_low, boost)


def scale_logits(logits: np.ndarray, temp) -> np.ndarray:
    """z / T per row, each a binary32 division (round to nearest)."""
    z = np.asarray(logits, dtype=np.float32)
    t = np.asarray(temp, dtype=np.float32).reshape(-1, 1)
    return (z / t).astype(np.float32)
