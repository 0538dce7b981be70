"""nvfp4_quantize_linear_noalloc (for callers that cannot allocate device
memory) against nvfp4_quantize_linear with a caller workspace: the same
kernels on the library's own scratch array, so y, the quantized activation
and its tensor scale must be bit-identical.  Two calls in a row, the second
with a smaller input, for each case; the cases cover the one-kernel path,
the two-launch path whose quantizer combines its maximum through the sync
record, and split-K partial sums in the scratch."""

import ctypes

import numpy as np
import pytest

from gpu_util import note, to_dev_bf16
from workloads import activations_bf16, weights_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import nvfp4_decode_linear_amd as nv
    return nv


def _bytes(t):
    import torch
    return t.detach().cpu().contiguous().view(-1).view(torch.uint8).numpy()


def _call_pair(nv, M, N, K, seed, out_dtype):
    import torch
    w16 = weights_bf16(11, seed, N, K)
    x16 = activations_bf16(11, seed, M, K, "outlier")
    wq = nv.quantize_weight(to_dev_bf16(w16))
    x = to_dev_bf16(x16)
    # the library-scratch call, straight through the C ABI
    y1 = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    q1 = nv.empty_act(M, K)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    st = nv._lib.nvfp4_quantize_linear_noalloc(
        M, N, K, ctypes.c_void_p(x.data_ptr()), x.stride(0), ctypes.c_void_p(wq.codes.data_ptr()),
        ctypes.c_void_p(wq.scales.data_ptr()), ctypes.c_void_p(wq.gscale.data_ptr()),
        ctypes.c_void_p(y1.data_ptr()), od, ctypes.c_void_p(q1.codes.data_ptr()),
        ctypes.c_void_p(q1.scales.data_ptr()), ctypes.c_void_p(q1.gscale.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nv.OK, nv.NVFP4Error(st, "nvfp4_quantize_linear_noalloc")
    # the same call with a caller workspace
    ws = torch.empty(max(256, nv._quantize_linear_workspace_bytes(M, N, K)), dtype=torch.uint8,
                     device="cuda")
    nv.workspace_init(ws)
    y0, q0 = nv.quantize_linear(x, wq, out_dtype=out_dtype, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(y1), _bytes(y0)), "y differs"
    assert np.array_equal(_bytes(q1.codes), _bytes(q0.codes))
    assert np.array_equal(_bytes(q1.scales), _bytes(q0.scales))
    assert np.array_equal(_bytes(q1.gscale), _bytes(q0.gscale))


CASES = [  # (first call, second call), each (M, N, K)
    ((1, 6144, 4096), (1, 256, 512)),          # one kernel, then a smaller one
    ((8, 5120, 8192), (2, 1024, 4096)),        # two launches (sync record), then one kernel
    ((8, 1024, 12288), (3, 512, 2048)),        # split-K partial sums in the scratch
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_call(nv, first, second):
    import torch
    nv.set_option("half_tiles", 1)             # 32-row tiles: small N splits K
    try:
        for i, (M, N, K) in enumerate((first, second)):
            od = torch.float32 if i == 0 else torch.bfloat16
            note(f"noalloc call {i}: M={M} N={N} K={K} {od}")
            _call_pair(nv, M, N, K, seed=N % 97 + i, out_dtype=od)
    finally:
        nv.set_option("half_tiles", 0)


def test_noalloc_rejects_oversized_workspace(nv):
    import torch
    M, N, K = 8, 4096, 12288
    nv.set_option("split_k", 64)
    try:
        assert nv._quantize_linear_workspace_bytes(M, N, K) > (4 << 20)
        x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
        wq = nv.empty_weight(N, K)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        q = nv.empty_act(M, K)
        note("noalloc oversized request")
        with pytest.raises(nv.NVFP4Error) as e:
            nv.quantize_linear_noalloc(x, wq, y, q)
        assert e.value.status == nv.ERR_WORKSPACE
    finally:
        nv.set_option("split_k", 0)
