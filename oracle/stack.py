"""Elementwise steps between the linears of the decode layer stack.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The README's demo caption ("ReSET" GitHub README, the figure caption under
the title: Qwen3-32B, batch 1, CUDA graphs, a 1,500-token decode) times whole
decode steps through a stack of NVFP4 linears.  The pages say nothing about
what sits between the linears; the plainest stand-in for a decoder layer that
keeps values bounded over 64 layers is taken:

* an unweighted RMS normalisation of each activation row before the QKV and
  gate_up projections: h = x / sqrt(mean(x^2) + eps), eps = 1e-6;
* SwiGLU between gate_up and down: h = silu(g) * u with g the first half of
  the gate_up output and u the second half, silu(g) = g / (1 + exp(-g)).

Both are computed in float64 here.  The GPU computes them in binary32 and then
quantizes its own binary32 result, so parity is (a) the GPU's h within a few
binary32 ulp of this float64 h and (b) the GPU's codes bit-exact against
``quantize`` applied to the GPU's own h.
"""

from __future__ import annotations

import numpy as np

RMS_EPS = 1e-6


def rms_norm_rows(x: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Unweighted RMS norm of each row, float64.  Pinned against
    torch.nn.functional.rms_norm on the CPU in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu_mul(gate_up: np.ndarray) -> np.ndarray:
    """silu(first half) * (second half) of each row, float64.  Pinned
    against torch.nn.functional.silu on the CPU in float64."""
    gu = np.asarray(gate_up, dtype=np.float64)
    half = gu.shape[-1] // 2
    g, u = gu[..., :half], gu[..., half:]
    return g / (1.0 + np.exp(-g)) * u
