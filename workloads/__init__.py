"""Seeded synthetic inputs for the NVFP4 decode linear: shapes, value
distributions and bf16 rounding.  Shared by the tests, the bench and the
oracle's callers; holds none of the quantization arithmetic.

The pages run Qwen3 8B/14B/32B and DeepSeek-R1-Distill-Qwen checkpoints
("ReSET" README, "Supported models") and time a 1,500-token batch-1 decode of
Qwen3-32B (README demo caption).  No checkpoint is used here: the decode
linear's speed does not depend on weight values, so weights and activations
are drawn from fixed distributions at the real projection shapes:

* weights: 0.02 * N(0, 1), rounded to bf16 (round to nearest even);
* activations, 8B-class and tiny workloads: N(0, 1) with 1% of the channels
  (round(0.01 * K) columns, the same for every row) multiplied by 20;
* activations, 32B-class workloads: Student-t with 3 degrees of freedom.

Every array comes from ``numpy.random.default_rng([2606, cfg, lin, role])``
with role 0 = weights, 1 = activation values, 2 = outlier-channel choice.
Activations are drawn at M = 8; smaller M takes the first M rows.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_ROOT = 2606
M_MAX = 8


@dataclass(frozen=True)
class Linear:
    name: str
    N: int
    K: int


# Decoder projection shapes (hidden, heads x 128, FFN) of the two model sizes.
QWEN3_8B = (
    Linear("qkv", 6144, 4096),       # 32 q heads + 2 x 8 kv heads, x128
    Linear("o", 4096, 4096),
    Linear("gate_up", 24576, 4096),  # 2 x FFN 12288
    Linear("down", 4096, 12288),
)
QWEN3_32B = (
    Linear("qkv", 10240, 5120),      # 64 q heads + 2 x 8 kv heads, x128
    Linear("o", 5120, 8192),
    Linear("gate_up", 51200, 5120),  # 2 x FFN 25600
    Linear("down", 5120, 25600),
)
TINY = (Linear("tiny", 256, 512),)


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    linears: tuple
    ms: tuple
    act_kind: str          # "outlier" | "student_t"


WORKLOADS = {
    1: Workload(1, "tiny_linear_m1", TINY, (1,), "outlier"),
    2: Workload(2, "qwen3_8b_decode_step_m1", QWEN3_8B, (1,), "outlier"),
    3: Workload(3, "qwen3_8b_batch_sweep", QWEN3_8B, (1, 2, 4, 8), "outlier"),
    4: Workload(4, "qwen3_32b_linears", QWEN3_32B, (1, 4, 8), "student_t"),
    5: Workload(5, "qwen3_32b_64_layer_stack", QWEN3_32B, (1, 8), "outlier"),
}


def rng(cfg: int, lin: int, role: int) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, cfg, lin, role])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 patterns -> the float32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weights_bf16(cfg: int, lin: int, N: int, K: int) -> np.ndarray:
    """[N][K] bf16 patterns of 0.02 * N(0, 1)."""
    g = rng(cfg, lin, 0)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    return bf16_bits(w)


def activations_bf16(cfg: int, lin: int, M: int, K: int, kind: str = "outlier") -> np.ndarray:
    """[M][K] bf16 patterns (drawn at M = 8, first M rows returned)."""
    if not 1 <= M <= M_MAX:
        raise ValueError("M must be in [1, 8]")
    g = rng(cfg, lin, 1)
    if kind == "outlier":
        x = g.standard_normal((M_MAX, K), dtype=np.float32)
        n_out = int(round(0.01 * K))
        if n_out:
            ch = rng(cfg, lin, 2).choice(K, size=n_out, replace=False)
            x[:, ch] *= np.float32(20.0)
    elif kind == "student_t":
        x = g.standard_t(3, size=(M_MAX, K)).astype(np.float32)
    elif kind == "normal":
        x = g.standard_normal((M_MAX, K), dtype=np.float32)
    else:
        raise ValueError(kind)
    return bf16_bits(x[:M])
