"""The C ABI library loads, exports every symbol include/nvfp4.h declares,
and rejects bad arguments on the host before any HIP call.  CPU only: no
call here reaches a kernel launch."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "nvfp4.h")
LIB = os.path.join(ROOT, "nvfp4_decode_linear_amd", "libnvfp4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libnvfp4.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.nvfp4_linear.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                               vp, sz, vp]
    L.nvfp4_quantize_act.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, sz, vp]
    L.nvfp4_act_workspace_bytes.argtypes = [ctypes.c_int, i64]
    L.nvfp4_act_workspace_bytes.restype = sz
    L.nvfp4_quantize_weight.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    L.nvfp4_unpack_weight.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.nvfp4_weight_bytes.argtypes = [i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.nvfp4_linear_workspace_bytes.argtypes = [ctypes.c_int, i64, i64]
    L.nvfp4_linear_workspace_bytes.restype = sz
    L.nvfp4_set_option.argtypes = [ctypes.c_int, i64]
    L.nvfp4_get_option.argtypes = [ctypes.c_int, ctypes.POINTER(i64)]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_workspace_init.argtypes = [vp, sz, vp]
    return L


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_versions_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == 1
    assert lib.nvfp4_layout_version() == 1
    for s in range(6):
        assert lib.nvfp4_status_string(s)
    assert lib.nvfp4_last_hip_error() == 0


def test_weight_bytes(lib):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.nvfp4_weight_bytes(4096, 4096, ctypes.byref(c), ctypes.byref(s)) == 0
    assert (c.value, s.value) == (4096 * 4096 // 2, 4096 * 4096 // 16)
    assert lib.nvfp4_weight_bytes(33, 272, ctypes.byref(c), ctypes.byref(s)) == 0
    assert (c.value, s.value) == (64 * 512 // 2, 64 * 512 // 16)      # padded to 32 x 256
    assert lib.nvfp4_weight_bytes(16, 24, ctypes.byref(c), ctypes.byref(s)) == 1
    assert lib.nvfp4_weight_bytes(0, 32, ctypes.byref(c), ctypes.byref(s)) == 1
    assert lib.nvfp4_weight_bytes(16, 32, None, ctypes.byref(s)) == 1


def test_options_roundtrip_and_validation(lib):
    v = ctypes.c_int64()
    assert lib.nvfp4_get_option(0, ctypes.byref(v)) == 0 and v.value == 0
    assert lib.nvfp4_set_option(0, 2) == 0
    assert lib.nvfp4_get_option(0, ctypes.byref(v)) == 0 and v.value == 2
    assert lib.nvfp4_set_option(0, 0) == 0
    assert lib.nvfp4_set_option(0, 9) == 1
    assert lib.nvfp4_set_option(6, -1) == 1         # spin limit
    assert lib.nvfp4_set_option(6, 1) == 0
    assert lib.nvfp4_get_option(6, ctypes.byref(v)) == 0 and v.value == 1
    assert lib.nvfp4_set_option(6, 0) == 0
    assert lib.nvfp4_set_option(9, 3) == 1          # half tiles: 0, 1 or 2
    assert lib.nvfp4_set_option(2, 6) == 1          # chunks per wave must be a multiple of 4
    assert lib.nvfp4_set_option(3, 2) == 1
    assert lib.nvfp4_set_option(99, 0) == 2
    assert lib.nvfp4_get_option(99, ctypes.byref(v)) == 2


def test_workspace_bytes(lib):
    assert lib.nvfp4_linear_workspace_bytes(9, 4096, 4096) == 0
    assert lib.nvfp4_linear_workspace_bytes(1, 4096, 24) == 0
    # The streaming kernel (the default whenever the activation fits in LDS)
    # needs no workspace unless it splits K.  With at most 128 row tiles it
    # runs on 16-row half tiles, never split; on 32-row tiles it splits only
    # below 64 tiles: N = 1024 (32 tiles), K = 4096 in 8 slices, counters
    # plus [8][M][N] partial sums.
    assert lib.nvfp4_linear_workspace_bytes(1, 24576, 4096) == 0
    assert lib.nvfp4_linear_workspace_bytes(1, 4096, 4096) == 0
    assert lib.nvfp4_linear_workspace_bytes(1, 1024, 4096) == 0
    assert lib.nvfp4_set_option(9, 1) == 0
    try:
        assert lib.nvfp4_linear_workspace_bytes(1, 1024, 4096) == 64 * 1024 + 8 * 1024 * 4
    finally:
        assert lib.nvfp4_set_option(9, 0) == 0
    assert lib.nvfp4_linear_workspace_bytes(8, 5120, 25600) == 0     # codes + f16 scales fit
    assert lib.nvfp4_linear_workspace_bytes(8, 5120, 40960) > 0      # too big for LDS: split-K
    # Forcing the split-K kernel on the 8B down projection (128 tiles) needs
    # one.
    assert lib.nvfp4_set_option(5, 2) == 0
    try:
        n = lib.nvfp4_linear_workspace_bytes(1, 4096, 12288)
        assert n > 64 * 1024 and (n - 64 * 1024) % (4096 * 4) == 0
    finally:
        assert lib.nvfp4_set_option(5, 0) == 0


FAKE = ctypes.c_void_p(0x1000)


@pytest.fixture
def no_gpu():
    """Calls below pass fake device pointers and expect a host-side error; a
    validation bug would turn one into a kernel launch, so they only run
    where no GPU is visible."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")


def test_linear_argument_errors(lib, no_gpu):
    f = lib.nvfp4_linear
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, None)
    assert f(9, 256, 512, *ok) == 2                           # M > 8: unsupported
    assert f(0, 256, 512, *ok) == 1
    assert f(1, 256, 520, *ok) == 1                           # K % 16 != 0
    assert f(1, 0, 512, *ok) == 1
    bad = list(ok)
    bad[0] = None
    assert f(1, 256, 512, *bad) == 1                          # null x_codes
    bad = list(ok)
    bad[7] = 5
    assert f(1, 256, 512, *bad) == 1                          # unknown output dtype
    # (8, 5120, 40960): the activation does not fit in LDS, so split-K with a
    # workspace
    bad = list(ok)
    bad[8] = ctypes.c_void_p(0x1001)
    assert f(8, 5120, 40960, *bad) == 1                       # misaligned workspace
    bad = list(ok)
    bad[9] = 16
    assert f(8, 5120, 40960, *bad) == 4                       # workspace too small
    bad = list(ok)
    bad[3] = ctypes.c_void_p(0x1008)
    assert f(1, 256, 512, *bad) == 1                          # misaligned tiled codes


def test_act_workspace_bytes(lib):
    assert lib.nvfp4_act_workspace_bytes(1, 4096) == 0          # 256 blocks: one workgroup
    assert lib.nvfp4_act_workspace_bytes(4, 4096) == 0          # 1024 blocks: one workgroup
    assert lib.nvfp4_act_workspace_bytes(8, 4096) == 16
    assert lib.nvfp4_act_workspace_bytes(8, 25600) == 16
    assert lib.nvfp4_act_workspace_bytes(8, 524288) == 16       # the largest tensor
    assert lib.nvfp4_act_workspace_bytes(8, 524304) == 0        # rejected: too large
    assert lib.nvfp4_act_workspace_bytes(9, 4096) == 0
    assert lib.nvfp4_act_workspace_bytes(1, 24) == 0


def test_quantize_argument_errors(lib, no_gpu):
    q = lib.nvfp4_quantize_act
    ws = (FAKE, 64, None)
    assert q(FAKE, 9, 512, 512, FAKE, FAKE, FAKE, *ws) == 2
    assert q(FAKE, 1, 520, 520, FAKE, FAKE, FAKE, *ws) == 1
    assert q(FAKE, 1, 512, 500, FAKE, FAKE, FAKE, *ws) == 1   # ldx < K
    assert q(FAKE, 1, 512, 516, FAKE, FAKE, FAKE, *ws) == 1   # ldx % 8
    assert q(None, 1, 512, 512, FAKE, FAKE, FAKE, *ws) == 1
    assert q(FAKE, 8, 524304, 524304, FAKE, FAKE, FAKE, *ws) == 1   # M * K > 2^22
    assert q(FAKE, 8, 25600, 25600, FAKE, FAKE, FAKE, None, 0, None) == 1     # needs a workspace
    assert q(FAKE, 8, 25600, 25600, FAKE, FAKE, FAKE, FAKE, 8, None) == 4     # too small
    assert q(FAKE, 8, 25600, 25600, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1008), 64, None) == 1
    assert lib.nvfp4_quantize_weight(FAKE, 256, 24, 24, FAKE, FAKE, FAKE, None) == 1
    assert lib.nvfp4_quantize_weight(FAKE, 256, 512, 256, FAKE, FAKE, FAKE, None) == 1
    assert lib.nvfp4_quantize_weight(ctypes.c_void_p(0x1002), 256, 512, 512, FAKE, FAKE, FAKE,
                                     None) == 1
    assert lib.nvfp4_unpack_weight(FAKE, FAKE, 256, 24, FAKE, FAKE, None) == 1
    assert lib.nvfp4_workspace_init(ctypes.c_void_p(0x1002), 64, None) == 1
    assert lib.nvfp4_workspace_init(None, 0, None) == 0


def test_no_device_is_reported(lib, no_gpu):
    assert lib.nvfp4_quantize_act(FAKE, 1, 512, 512, FAKE, FAKE, FAKE, None, 0, None) == 3
    assert lib.nvfp4_linear(1, 256, 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                            1 << 20, None) == 3


def test_stack_argument_errors(lib, no_gpu):
    class Cfg(ctypes.Structure):
        _fields_ = [("M", ctypes.c_int), ("layers", ctypes.c_int), ("hidden", ctypes.c_int64),
                    ("qkv_n", ctypes.c_int64), ("q_cols", ctypes.c_int64),
                    ("ffn", ctypes.c_int64), ("eps", ctypes.c_float),
                    ("gate_up_interleaved", ctypes.c_int)]

    class W(ctypes.Structure):
        _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                    ("gscale", ctypes.c_void_p)]

    vp = ctypes.c_void_p
    f = lib.nvfp4_stack_create
    f.argtypes = [ctypes.POINTER(Cfg), ctypes.POINTER(W), vp, vp, vp, ctypes.POINTER(vp)]
    ws = (W * 8)(*[W(0x1000, 0x1000, 0x1000)] * 8)
    out = vp(0x1234)
    good = Cfg(1, 2, 512, 768, 512, 1024, 1e-6)
    assert f(None, ws, FAKE, FAKE, FAKE, ctypes.byref(out)) == 1 and out.value is None
    assert f(ctypes.byref(good), ws, FAKE, FAKE, None, ctypes.byref(out)) == 1   # null stream
    assert f(ctypes.byref(good), ws, None, FAKE, FAKE, ctypes.byref(out)) == 1
    assert f(ctypes.byref(good), ws, ctypes.c_void_p(0x1008), FAKE, FAKE,
             ctypes.byref(out)) == 1                                             # x_in alignment
    for bad in (Cfg(9, 2, 512, 768, 512, 1024, 1e-6),):
        assert f(ctypes.byref(bad), ws, FAKE, FAKE, FAKE, ctypes.byref(out)) == 2
    for bad in (Cfg(0, 2, 512, 768, 512, 1024, 1e-6), Cfg(1, 0, 512, 768, 512, 1024, 1e-6),
                Cfg(1, 2, 520, 768, 512, 1024, 1e-6), Cfg(1, 2, 512, 500, 512, 1024, 1e-6),
                Cfg(1, 2, 512, 768, 512, 40000, 1e-6), Cfg(1, 2, 512, 768, 512, 1024, -1.0),
                Cfg(1, 2, 512, 768, 512, 1024, 1e-6, 2)):
        assert f(ctypes.byref(bad), ws, FAKE, FAKE, FAKE, ctypes.byref(out)) == 1
    nulls = (W * 8)(*[W(0x1000, 0x1000, 0x1000)] * 7 + [W(0x1000, 0, 0x1000)])
    assert f(ctypes.byref(good), nulls, FAKE, FAKE, FAKE, ctypes.byref(out)) == 1
    lib.nvfp4_stack_run.argtypes = [vp, ctypes.c_int, vp]
    lib.nvfp4_stack_destroy.argtypes = [vp]
    assert lib.nvfp4_stack_run(None, 1, None) == 1
    assert lib.nvfp4_stack_destroy(None) == 1


def test_fused_quantize_argument_errors(lib, no_gpu):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    r = lib.nvfp4_rmsnorm_quantize_act
    r.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.c_float, vp, vp, vp, vp, vp,
                  ctypes.c_size_t, vp]
    s = lib.nvfp4_silu_mul_quantize_act
    s.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    assert r(FAKE, 9, 512, 512, 1e-6, FAKE, FAKE, FAKE, None, FAKE, 64, None) == 2
    assert r(FAKE, 1, 40960, 40960, 1e-6, FAKE, FAKE, FAKE, None, FAKE, 64, None) == 1  # K cap
    assert r(FAKE, 1, 512, 512, -1.0, FAKE, FAKE, FAKE, None, FAKE, 64, None) == 1      # eps
    assert r(FAKE, 2, 512, 512, 1e-6, FAKE, FAKE, FAKE, None, None, 0, None) == 1      # ws
    assert r(FAKE, 2, 512, 512, 1e-6, FAKE, FAKE, FAKE, None, FAKE, 8, None) == 4
    assert r(FAKE, 1, 512, 512, 1e-6, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1004), None, 0,
             None) == 1                                                             # h_out
    assert s(FAKE, 1, 512, 1000, FAKE, FAKE, FAKE, None, None, 0, None) == 1        # ld < 2K
    assert s(FAKE, 1, 512, 1024, FAKE, FAKE, FAKE, None, None, 0, None) == 3        # no device


def test_quantize_linear_argument_errors(lib, no_gpu):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.nvfp4_quantize_linear
    f.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                  ctypes.c_size_t, vp]
    ok = (FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert f(9, 256, 512, FAKE, 512, *ok) == 2
    assert f(1, 256, 520, FAKE, 520, *ok) == 1                 # K % 16
    assert f(1, 256, 512, FAKE, 500, *ok) == 1                 # ldx < K
    assert f(1, 256, 512, ctypes.c_void_p(0x1008), 512, *ok) == 1   # x alignment
    bad = list(ok)
    bad[5] = None
    assert f(1, 256, 512, FAKE, 512, *bad) == 1                # x_codes output required
    assert f(1, 256, 512, FAKE, 512, *ok) == 3                 # no device
    lib.nvfp4_quantize_linear_workspace_bytes.argtypes = [ctypes.c_int, i64, i64]
    lib.nvfp4_quantize_linear_workspace_bytes.restype = ctypes.c_size_t
    assert lib.nvfp4_quantize_linear_workspace_bytes(8, 24576, 4096) == 16   # act sync record
    # at least the sync record for every valid shape: the unfused fallback of
    # the RMS-norm variant needs it whenever M > 1
    assert lib.nvfp4_quantize_linear_workspace_bytes(1, 24576, 4096) == 16
    assert lib.nvfp4_quantize_linear_workspace_bytes(2, 4096, 4096) == 16
    assert lib.nvfp4_quantize_linear_workspace_bytes(9, 4096, 4096) == 0
    assert lib.nvfp4_quantize_linear_workspace_bytes(1, 4096, 24) == 0


def test_static_scale_argument_errors(lib, no_gpu):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    a = lib.nvfp4_quantize_act_static
    a.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp]
    assert a(FAKE, 9, 512, 512, FAKE, FAKE, FAKE, None) == 2
    assert a(FAKE, 1, 520, 520, FAKE, FAKE, FAKE, None) == 1          # K % 16
    assert a(FAKE, 1, 512, 500, FAKE, FAKE, FAKE, None) == 1          # ldx < K
    assert a(FAKE, 1, 512, 512, None, FAKE, FAKE, None) == 1          # no scale
    assert a(FAKE, 1, 512, 512, ctypes.c_void_p(0x1002), FAKE, FAKE, None) == 1   # alignment
    assert a(FAKE, 8, 25600, 25600, FAKE, FAKE, FAKE, None) == 3      # no workspace needed
    f = lib.nvfp4_quantize_linear_static
    f.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                  ctypes.c_size_t, vp]
    ok = (FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1 << 20, None)
    assert f(9, 256, 512, FAKE, 512, FAKE, *ok) == 2
    assert f(1, 256, 512, FAKE, 512, None, *ok) == 1                  # no scale
    assert f(1, 256, 512, FAKE, 500, FAKE, *ok) == 1                  # ldx < K
    assert f(1, 256, 512, FAKE, 512, FAKE, *ok) == 3                  # no device


def test_noalloc_argument_errors_and_scratch_size(lib, no_gpu):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.nvfp4_quantize_linear_noalloc
    f.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp]
    ok = (FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None)
    assert f(9, 256, 512, FAKE, 512, *ok) == 2
    assert f(1, 256, 520, FAKE, 520, *ok) == 1
    assert f(1, 256, 512, FAKE, 500, *ok) == 1                        # ldx < K
    assert f(1, 256, 512, None, 512, *ok) == 1
    bad = list(ok)
    bad[4] = 7
    assert f(1, 256, 512, FAKE, 512, *bad) == 1                       # output dtype
    # the library's scratch: 4 MiB (the header's NVFP4_NOALLOC_SCRATCH_BYTES)
    hdr = open(HEADER).read()
    assert "#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)" in hdr
    cap = 4 << 20
    q = lib.nvfp4_quantize_linear_workspace_bytes
    q.argtypes = [ctypes.c_int, i64, i64]
    q.restype = ctypes.c_size_t
    for M in range(1, 9):
        for N in (1, 31, 256, 1024, 2016, 4096, 5120, 6144, 10240, 24576, 51200, 65536):
            for K in (16, 512, 4096, 5120, 8192, 12288, 25600, 32768):
                if M * K <= 204800:
                    assert 0 < q(M, N, K) <= cap, (M, N, K)
    # forcing many K slices exceeds the scratch: rejected before any HIP call
    assert lib.nvfp4_set_option(1, 64) == 0
    try:
        assert q(8, 65536, 32768) > cap
        assert f(8, 65536, 32768, FAKE, 32768, *ok) == 4
    finally:
        assert lib.nvfp4_set_option(1, 0) == 0


def test_reset_temperature_argument_errors(lib, no_gpu):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64

    class P(ctypes.Structure):
        _fields_ = [("t_low", ctypes.c_float), ("tau0", ctypes.c_float),
                    ("t_base", ctypes.c_float), ("t_max", ctypes.c_float)]

    w = lib.nvfp4_reset_workspace_bytes
    w.argtypes = [ctypes.c_int, i64]
    w.restype = ctypes.c_size_t
    # 1 KiB of row counters, then 16 B per (row, group of 4096 logits),
    # rounded up to 256 B: the Qwen3 vocabulary (151936) has 38 groups
    assert w(1, 151936) == 1024 + 768
    assert w(8, 151936) == 1024 + 4864
    assert w(0, 10) == 0 and w(257, 10) == 0 and w(1, 0) == 0
    assert w(1, 1 << 20) == 1024 + 4096 and w(1, (1 << 20) + 1) == 0    # at most 2^20 per row
    f = lib.nvfp4_reset_temperature
    f.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.POINTER(P), vp, vp, vp, vp, vp, i64, vp,
                  ctypes.c_size_t, vp]
    good = P(0.1, 0.5505, 0.6, 1.5)
    ok_tail = (FAKE, None, FAKE, FAKE, None, 0, FAKE, 1 << 20, None)
    assert f(FAKE, 1, 1000, 1000, ctypes.byref(good), *ok_tail) == 3          # no device
    assert f(FAKE, 0, 1000, 1000, ctypes.byref(good), *ok_tail) == 1
    assert f(FAKE, 257, 1000, 1000, ctypes.byref(good), *ok_tail) == 1
    assert f(FAKE, 1, 1000, 999, ctypes.byref(good), *ok_tail) == 1           # ldl < V
    v = (1 << 20) + 4
    assert f(FAKE, 1, v, v, ctypes.byref(good), *ok_tail) == 1                # V > 2^20
    assert f(FAKE, 1, 1000, 1002, ctypes.byref(good), *ok_tail) == 1          # ldl % 4
    assert f(ctypes.c_void_p(0x1008), 1, 1000, 1000, ctypes.byref(good), *ok_tail) == 1
    assert f(FAKE, 1, 1000, 1000, None, *ok_tail) == 1                        # no params
    for bad in (P(0.0, 0.5, 0.6, 1.5), P(0.1, -1.0, 0.6, 1.5), P(0.1, 0.5, float("nan"), 1.5),
                P(0.1, 0.5, 0.6, float("inf"))):
        assert f(FAKE, 1, 1000, 1000, ctypes.byref(bad), *ok_tail) == 1
    tail = list(ok_tail)
    tail[6] = None                                                            # no workspace
    assert f(FAKE, 1, 1000, 1000, ctypes.byref(good), *tail) == 1
    tail = list(ok_tail)
    tail[7] = 16                                                              # too small
    assert f(FAKE, 1, 1000, 1000, ctypes.byref(good), *tail) == 4
    tail = list(ok_tail)
    tail[4], tail[5] = FAKE, 1000                                             # in place, ldo == ldl
    assert f(FAKE, 1, 1000, 1000, ctypes.byref(good), *tail) == 3
    tail[5] = 1004                                                            # in place, ldo != ldl
    assert f(FAKE, 1, 1000, 1000, ctypes.byref(good), *tail) == 1


def test_silu_and_f32_argument_errors(lib, no_gpu):
    vp, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    MIS = ctypes.c_void_p(0x1004)
    g = lib.nvfp4_quantize_weight_gate_up
    g.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    assert g(FAKE, 24, 512, 512, FAKE, FAKE, FAKE, None) == 1            # F % 16
    assert g(FAKE, 64, 512, 500, FAKE, FAKE, FAKE, None) == 1            # ldw < K
    assert g(FAKE, 64, 512, 512, FAKE, FAKE, FAKE, None) == 3            # no device
    s = lib.nvfp4_quantize_linear_silu_mul
    s.argtypes = [ctypes.c_int, i64, i64, vp, i64, ctypes.c_int, f32, vp, vp, vp, vp, i64, vp,
                  vp, vp, vp, vp, vp, vp, sz, vp]

    def silu(M=1, F=1024, K=512, ldx=512, rms=1, eps=1e-6, h=FAKE, ldh=1024, amax=FAKE,
             xh=None):
        return s(M, F, K, FAKE, ldx, rms, eps, FAKE, FAKE, FAKE, h, ldh, amax, None, FAKE, FAKE,
                 FAKE, xh, FAKE, 1 << 20, None)
    assert silu(M=9) == 2
    assert silu(F=1000) == 1                                              # F % 16
    assert silu(ldh=1000) == 1                                            # ldh < F
    assert silu(ldx=500) == 1                                             # ldx < K
    assert silu(rms=2) == 1
    assert silu(rms=0, xh=FAKE) == 1                                      # xh_out needs the norm
    assert silu(eps=-1.0) == 1
    assert silu(h=None) == 1 and silu(amax=None) == 1 and silu(amax=MIS) == 1
    assert silu() == 3                                                    # no device
    a = lib.nvfp4_quantize_act_f32
    a.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    assert a(FAKE, 9, 512, 512, None, FAKE, FAKE, FAKE, FAKE, 64, None) == 2
    assert a(FAKE, 1, 512, 510, None, FAKE, FAKE, FAKE, FAKE, 64, None) == 1     # ldx
    assert a(FAKE, 1, 512, 516, MIS, FAKE, FAKE, FAKE, FAKE, 64, None) == 1      # record alignment
    # several workgroups combine their maxima in the workspace unless a record is given
    assert a(FAKE, 8, 25600, 25600, None, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert a(FAKE, 8, 25600, 25600, None, FAKE, FAKE, FAKE, FAKE, 8, None) == 4
    assert a(FAKE, 8, 25600, 25600, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 3
    q = lib.nvfp4_quantize_linear_f32
    q.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                  vp, sz, vp]
    ok = (FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1 << 24, None)
    assert q(9, 5120, 25600, FAKE, 25600, FAKE, *ok) == 2
    assert q(1, 5120, 25600, FAKE, 25599, FAKE, *ok) == 1               # ldx
    assert q(1, 5120, 25600, FAKE, 25600, MIS, *ok) == 1                 # record alignment
    assert q(1, 5120, 25600, FAKE, 25600, FAKE, *ok) == 3                # no device
    qw = lib.nvfp4_quantize_linear_f32_workspace_bytes
    qw.argtypes = [ctypes.c_int, i64, i64]
    qw.restype = sz
    lw = lib.nvfp4_linear_workspace_bytes
    # Qwen3-8B down at M = 1: the whole activation fits the prologue of a plan
    # that fills the CUs: the linear's need (none) or the sync record
    assert qw(1, 4096, 12288) == 16
    # M = 8: the two launches' need by default; with the K-slice plan allowed,
    # its split-K counters and partials
    assert qw(8, 5120, 25600) == max(16, lw(8, 5120, 25600))
    lib.nvfp4_set_option.argtypes = [ctypes.c_int, i64]
    assert lib.nvfp4_set_option(10, 1) == 0
    try:
        assert qw(8, 5120, 25600) > max(16, lw(8, 5120, 25600))
        assert qw(1, 4096, 12288) == 16                  # fits: no slices even then
    finally:
        assert lib.nvfp4_set_option(10, 0) == 0
    assert lib.nvfp4_set_option(10, 3) == 1
    assert qw(9, 5120, 25600) == 0
