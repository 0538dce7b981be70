"""Helpers for the GPU parity tests: device transfer, a test-side
implementation of the documented device-tiled weight layout (used to craft
weights directly), and case logging."""

import sys

import numpy as np

TILE_N, CHUNK_K, GROUP_K = 32, 64, 256


def note(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def pad_dims(N, K):
    return -(-N // TILE_N) * TILE_N, -(-K // GROUP_K) * GROUP_K


def tile_weight(codes_rm: np.ndarray, scales_rm: np.ndarray, N: int, K: int):
    """Canonical codes [N][K/2] and scales [N][K/16] -> the device-tiled
    byte arrays of layout version 1 (include/nvfp4.h), padding with zeros."""
    Np, Kp = pad_dims(N, K)
    c = np.zeros((Np, Kp // 2), np.uint8)
    c[:N, :K // 2] = codes_rm
    s = np.zeros((Np, Kp // 16), np.uint8)
    s[:N, :K // 16] = scales_rm
    T, KC, KG = Np // TILE_N, Kp // CHUNK_K, Kp // GROUP_K
    # codes: record (t, c) = 64 lanes x 16 B; lane l -> row l % 32, half l // 32
    cr = c.reshape(T, TILE_N, KC, 2, 16)              # [t][row][chunk][half][16 B]
    cr = cr.transpose(0, 2, 3, 1, 4)                  # [t][chunk][half][row][16 B]
    codes_t = np.ascontiguousarray(cr).reshape(-1)
    # scales: record (t, g) = 64 lanes x 8 B; lane (row, half) byte 2q + b holds
    # block 16g + 4q + 2*half + b
    sr = s.reshape(T, TILE_N, KG, 4, 2, 2)            # [t][row][g][q][half][b]
    sr = sr.transpose(0, 2, 4, 1, 3, 5)               # [t][g][half][row][q][b]
    scales_t = np.ascontiguousarray(sr).reshape(-1)
    return codes_t, scales_t
