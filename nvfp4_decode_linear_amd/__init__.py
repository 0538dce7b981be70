"""Python binding of libnvfp4.so, the MI355X (gfx950) small-M NVFP4 W4A4
decode linear ("ReSET" GitHub README, "Core components", item 2).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/nvfp4.h.  torch supplies device memory
and the current HIP stream.  There is no fallback: if the library is not
built, importing this package raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_WORKSPACE, ERR_HIP = range(6)
OUT_F32, OUT_BF16 = 0, 1
OPTIONS = {"gemv_max_m": 0, "split_k": 1, "chunks_per_wave": 2, "nontemporal": 3, "waves": 4,
           "kernel": 5, "spin_limit": 6, "grid": 7, "fuse_quant": 8, "half_tiles": 9,
           "f32_slices": 10}
TILE_N, CHUNK_K, GROUP_K = 32, 64, 256

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(python nvfp4_decode_linear_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_c_i64, _c_int, _c_size, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_abi_version = _sig("nvfp4_abi_version", _c_int)
_layout_version = _sig("nvfp4_layout_version", _c_int)
_status_string = _sig("nvfp4_status_string", ctypes.c_char_p, _c_int)
_last_hip_error = _sig("nvfp4_last_hip_error", _c_int)
_set_option = _sig("nvfp4_set_option", _c_int, _c_int, _c_i64)
_get_option = _sig("nvfp4_get_option", _c_int, _c_int, ctypes.POINTER(_c_i64))
_weight_bytes = _sig("nvfp4_weight_bytes", _c_int, _c_i64, _c_i64, ctypes.POINTER(_c_size),
                     ctypes.POINTER(_c_size))
_quantize_weight = _sig("nvfp4_quantize_weight", _c_int, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp,
                        _vp, _vp)
_unpack_weight = _sig("nvfp4_unpack_weight", _c_int, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp)
_quantize_act = _sig("nvfp4_quantize_act", _c_int, _vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp,
                     _vp, _c_size, _vp)
_act_workspace_bytes = _sig("nvfp4_act_workspace_bytes", _c_size, _c_int, _c_i64)
_rmsnorm_quantize_act = _sig("nvfp4_rmsnorm_quantize_act", _c_int, _vp, _c_int, _c_i64, _c_i64,
                             ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _c_size, _vp)
_silu_mul_quantize_act = _sig("nvfp4_silu_mul_quantize_act", _c_int, _vp, _c_int, _c_i64, _c_i64,
                              _vp, _vp, _vp, _vp, _vp, _c_size, _vp)
_linear_workspace_bytes = _sig("nvfp4_linear_workspace_bytes", _c_size, _c_int, _c_i64, _c_i64)
_workspace_init = _sig("nvfp4_workspace_init", _c_int, _vp, _c_size, _vp)
_selftest_e2m1 = _sig("nvfp4_selftest_e2m1", _c_int, _vp, _vp)
_linear = _sig("nvfp4_linear", _c_int, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
               _c_int, _vp, _c_size, _vp)
_quantize_linear = _sig("nvfp4_quantize_linear", _c_int, _c_int, _c_i64, _c_i64, _vp, _c_i64, _vp,
                        _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_size, _vp)
_quantize_linear_workspace_bytes = _sig("nvfp4_quantize_linear_workspace_bytes", _c_size, _c_int,
                                        _c_i64, _c_i64)
_quantize_act_static = _sig("nvfp4_quantize_act_static", _c_int, _vp, _c_int, _c_i64, _c_i64, _vp,
                           _vp, _vp, _vp)
_quantize_linear_static = _sig("nvfp4_quantize_linear_static", _c_int, _c_int, _c_i64, _c_i64, _vp,
                               _c_i64, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_size,
                               _vp)
_quantize_linear_noalloc = _sig("nvfp4_quantize_linear_noalloc", _c_int, _c_int, _c_i64, _c_i64,
                                _vp, _c_i64, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp)
_rmsnorm_quantize_linear = _sig("nvfp4_rmsnorm_quantize_linear", _c_int, _c_int, _c_i64, _c_i64, _vp,
                                _c_i64, ctypes.c_float, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp,
                                _vp, _vp, _c_size, _vp)


_quantize_weight_gate_up = _sig("nvfp4_quantize_weight_gate_up", _c_int, _vp, _c_i64, _c_i64,
                                _c_i64, _vp, _vp, _vp, _vp)
_quantize_act_f32 = _sig("nvfp4_quantize_act_f32", _c_int, _vp, _c_int, _c_i64, _c_i64, _vp, _vp,
                         _vp, _vp, _vp, _c_size, _vp)
_quantize_linear_f32 = _sig("nvfp4_quantize_linear_f32", _c_int, _c_int, _c_i64, _c_i64, _vp,
                            _c_i64, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_size,
                            _vp)
_quantize_linear_f32_workspace_bytes = _sig("nvfp4_quantize_linear_f32_workspace_bytes", _c_size,
                                            _c_int, _c_i64, _c_i64)
_quantize_linear_silu_mul = _sig("nvfp4_quantize_linear_silu_mul", _c_int, _c_int, _c_i64, _c_i64,
                                 _vp, _c_i64, _c_int, ctypes.c_float, _vp, _vp, _vp, _vp, _c_i64,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp)
AMAX_RECORD_WORDS = 256


class ResetParams(ctypes.Structure):
    """nvfp4_reset_params: t_low, tau0, t_base, t_max."""
    _fields_ = [("t_low", ctypes.c_float), ("tau0", ctypes.c_float), ("t_base", ctypes.c_float),
                ("t_max", ctypes.c_float)]


_reset_workspace_bytes = _sig("nvfp4_reset_workspace_bytes", _c_size, _c_int, _c_i64)
_reset_temperature = _sig("nvfp4_reset_temperature", _c_int, _vp, _c_int, _c_i64, _c_i64,
                          ctypes.POINTER(ResetParams), _vp, _vp, _vp, _vp, _vp, _c_i64, _vp,
                          _c_size, _vp)


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _check(status: int, where: str) -> None:
    if status != OK:
        raise NVFP4Error(status, where)


def abi_version() -> int:
    return _abi_version()


def layout_version() -> int:
    return _layout_version()


def set_option(name, value: int) -> None:
    _check(_set_option(OPTIONS.get(name, name), int(value)), "nvfp4_set_option")


def get_option(name) -> int:
    v = _c_i64()
    _check(_get_option(OPTIONS.get(name, name), ctypes.byref(v)), "nvfp4_get_option")
    return v.value


def weight_bytes(N: int, K: int):
    c, s = _c_size(), _c_size()
    _check(_weight_bytes(N, K, ctypes.byref(c), ctypes.byref(s)), "nvfp4_weight_bytes")
    return c.value, s.value


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return _linear_workspace_bytes(M, N, K)


def act_workspace_bytes(M: int, K: int) -> int:
    return _act_workspace_bytes(M, K)


# ------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class QuantWeight:
    """Device-tiled NVFP4 weight (layout version 1)."""
    codes: object      # uint8 tensor, tiled
    scales: object     # uint8 tensor, tiled
    gscale: object     # float32 tensor [1]
    N: int
    K: int
    gate_up: bool = False   # rows interleaved for the SiLU * mul epilogue


@dataclass
class QuantAct:
    """Canonical NVFP4 activation: codes [M][K/2], scales [M][K/16]."""
    codes: object
    scales: object
    gscale: object     # float32 tensor [1]
    M: int
    K: int


def empty_weight(N: int, K: int, device="cuda") -> QuantWeight:
    torch = _torch()
    cb, sb = weight_bytes(N, K)
    return QuantWeight(torch.empty(cb, dtype=torch.uint8, device=device),
                       torch.empty(sb, dtype=torch.uint8, device=device),
                       torch.empty(1, dtype=torch.float32, device=device), N, K)


def quantize_weight(w, out: QuantWeight | None = None) -> QuantWeight:
    """bf16 [N][K] (row stride >= K) -> device-tiled NVFP4 weight."""
    torch = _torch()
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D bf16 tensor with unit column stride")
    N, K = w.shape
    q = out if out is not None else empty_weight(N, K, w.device)
    _check(_quantize_weight(_ptr(w), N, K, w.stride(0), _ptr(q.codes), _ptr(q.scales),
                            _ptr(q.gscale), _stream(w)), "nvfp4_quantize_weight")
    return q


def quantize_weight_gate_up(w, out: QuantWeight | None = None) -> QuantWeight:
    """bf16 gate_up weight [2F][K] (gate rows first) -> device-tiled NVFP4
    weight in the interleaved row order of the SiLU * mul epilogue."""
    torch = _torch()
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1 or w.shape[0] % 2:
        raise ValueError("w must be a 2-D bf16 tensor [2F][K] with unit column stride")
    N, K = w.shape
    q = out if out is not None else empty_weight(N, K, w.device)
    _check(_quantize_weight_gate_up(_ptr(w), N // 2, K, w.stride(0), _ptr(q.codes),
                                    _ptr(q.scales), _ptr(q.gscale), _stream(w)),
           "nvfp4_quantize_weight_gate_up")
    return QuantWeight(q.codes, q.scales, q.gscale, N, K, True)


def selftest_e2m1(device="cuda"):
    """(mismatches, checked) of the device E2M1 encoder against its rounding
    rule over every finite binary32 pattern (nvfp4_selftest_e2m1)."""
    torch = _torch()
    out = torch.empty(2, dtype=torch.int64, device=device)
    _check(_selftest_e2m1(_ptr(out), _stream(out)), "nvfp4_selftest_e2m1")
    v = out.cpu().tolist()
    return v[0], v[1]


def unpack_weight(q: QuantWeight):
    """Device-tiled weight -> canonical (codes [N][K/2], scales [N][K/16])."""
    torch = _torch()
    c = torch.empty((q.N, q.K // 2), dtype=torch.uint8, device=q.codes.device)
    s = torch.empty((q.N, q.K // 16), dtype=torch.uint8, device=q.codes.device)
    _check(_unpack_weight(_ptr(q.codes), _ptr(q.scales), q.N, q.K, _ptr(c), _ptr(s),
                          _stream(c)), "nvfp4_unpack_weight")
    return c, s


def empty_act(M: int, K: int, device="cuda") -> QuantAct:
    torch = _torch()
    return QuantAct(torch.empty((M, K // 2), dtype=torch.uint8, device=device),
                    torch.empty((M, K // 16), dtype=torch.uint8, device=device),
                    torch.empty(1, dtype=torch.float32, device=device), M, K)


def quantize_act(x, out: QuantAct | None = None, ws=None) -> QuantAct:
    """bf16 [M][K] (row stride >= K, multiple of 8) -> canonical NVFP4 with
    one tensor scale computed on the device.  `ws` defaults to the device's
    shared workspace (stream-ordered use only)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    q = out if out is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(1, 1, 16, x.device)
    _check(_quantize_act(_ptr(x), M, K, x.stride(0), _ptr(q.codes), _ptr(q.scales),
                         _ptr(q.gscale), _ptr(ws), ws.numel(), _stream(x)), "nvfp4_quantize_act")
    return q


def quantize_act_static(x, gscale, out: QuantAct | None = None) -> QuantAct:
    """bf16 [M][K] -> canonical NVFP4 with a caller-supplied tensor scale
    (float32 device tensor [1], e.g. a calibrated static activation scale);
    the returned QuantAct's gscale is that tensor."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    if gscale.dtype != torch.float32 or gscale.numel() < 1:
        raise ValueError("gscale must be a float32 device tensor")
    M, K = x.shape
    q = out if out is not None else empty_act(M, K, x.device)
    _check(_quantize_act_static(_ptr(x), M, K, x.stride(0), _ptr(gscale), _ptr(q.codes),
                                _ptr(q.scales), _stream(x)), "nvfp4_quantize_act_static")
    return QuantAct(q.codes, q.scales, gscale, M, K)


def _nullable(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def rmsnorm_quantize_act(x, eps=1e-6, out: QuantAct | None = None, h_out=None, ws=None):
    """Unweighted per-row RMS norm of bf16 x [M][K] in binary32, then the
    activation quantizer on it; h_out (float32 [M][K]) receives h if given."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    q = out if out is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(1, 1, 16, x.device)
    _check(_rmsnorm_quantize_act(_ptr(x), M, K, x.stride(0), float(eps), _ptr(q.codes),
                                 _ptr(q.scales), _ptr(q.gscale), _nullable(h_out), _ptr(ws),
                                 ws.numel(), _stream(x)), "nvfp4_rmsnorm_quantize_act")
    return q


def silu_mul_quantize_act(gu, out: QuantAct | None = None, h_out=None, ws=None):
    """h = silu(gate) * up from bf16 gu [M][2K] (first half gate), in
    binary32, then the activation quantizer on it."""
    torch = _torch()
    if gu.dtype != torch.bfloat16 or gu.dim() != 2 or gu.stride(1) != 1 or gu.shape[1] % 2:
        raise ValueError("gu must be a 2-D bf16 tensor [M][2K] with unit column stride")
    M, K = gu.shape[0], gu.shape[1] // 2
    q = out if out is not None else empty_act(M, K, gu.device)
    if ws is None:
        ws = workspace(1, 1, 16, gu.device)
    _check(_silu_mul_quantize_act(_ptr(gu), M, K, gu.stride(0), _ptr(q.codes), _ptr(q.scales),
                                  _ptr(q.gscale), _nullable(h_out), _ptr(ws), ws.numel(),
                                  _stream(gu)), "nvfp4_silu_mul_quantize_act")
    return q


class _StackConfig(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int), ("layers", ctypes.c_int), ("hidden", ctypes.c_int64),
                ("qkv_n", ctypes.c_int64), ("q_cols", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("eps", ctypes.c_float), ("gate_up_interleaved", ctypes.c_int)]


class _Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p)]


_stack_create = _sig("nvfp4_stack_create", _c_int, ctypes.POINTER(_StackConfig),
                     ctypes.POINTER(_Weight), _vp, _vp, _vp, ctypes.POINTER(_vp))
_stack_run = _sig("nvfp4_stack_run", _c_int, _vp, _c_int, _vp)
_stack_run_eager = _sig("nvfp4_stack_run_eager", _c_int, _vp, _vp)
_stack_destroy = _sig("nvfp4_stack_destroy", _c_int, _vp)


class Stack:
    """Graph-replayed decode step of a layer stack (nvfp4_stack_*).

    layers: list of (qkv, o, gate_up, down) QuantWeight per layer.  x_in and
    y_out are bf16 [M][hidden] tensors the caller keeps alive.  The stack
    captures and replays on its own side stream; run() orders it after the
    caller's current stream and the caller's stream after it."""

    def __init__(self, M, hidden, qkv_n, q_cols, ffn, layers, x_in, y_out, eps=1e-6):
        torch = _torch()
        self._torch = torch
        self._h = None
        inter = [bool(ws4[2].gate_up) for ws4 in layers]
        if any(inter) != all(inter):
            raise ValueError("gate_up weights: all interleaved or none")
        self.cfg = _StackConfig(M, len(layers), hidden, qkv_n, q_cols, ffn, eps,
                                1 if all(inter) else 0)
        arr = (_Weight * (4 * len(layers)))()
        for l, ws4 in enumerate(layers):
            for j, w in enumerate(ws4):
                arr[4 * l + j] = _Weight(w.codes.data_ptr(), w.scales.data_ptr(),
                                         w.gscale.data_ptr())
        self._keep = (layers, x_in, y_out)
        self.device = x_in.device
        self.stream = torch.cuda.Stream(device=self.device)
        self.stream.wait_stream(torch.cuda.current_stream(self.device))
        h = _vp()
        _check(_stack_create(ctypes.byref(self.cfg), arr, _ptr(x_in), _ptr(y_out),
                             _vp(self.stream.cuda_stream), ctypes.byref(h)),
               "nvfp4_stack_create")
        self._h = h
        torch.cuda.current_stream(self.device).wait_stream(self.stream)

    def _around(self, fn):
        cur = self._torch.cuda.current_stream(self.device)
        self.stream.wait_stream(cur)
        fn()
        cur.wait_stream(self.stream)

    def run(self, steps=1):
        self._around(lambda: _check(_stack_run(self._h, int(steps), _vp(self.stream.cuda_stream)),
                                    "nvfp4_stack_run"))

    def run_eager(self):
        self._around(lambda: _check(_stack_run_eager(self._h, _vp(self.stream.cuda_stream)),
                                    "nvfp4_stack_run_eager"))

    def close(self):
        if self._h:
            self._torch.cuda.synchronize(self.device)
            _check(_stack_destroy(self._h), "nvfp4_stack_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_WS = {}


def workspace(M: int, N: int, K: int, device="cuda", need: int | None = None):
    """A per-device workspace, grown and zero-initialised on demand (need:
    bytes, default the linear's)."""
    torch = _torch()
    if need is None:
        need = linear_workspace_bytes(M, N, K)
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        workspace_init(ws)
        _WS[key] = ws
    return ws


def workspace_init(ws) -> None:
    _check(_workspace_init(_ptr(ws), ws.numel(), _stream(ws)), "nvfp4_workspace_init")


def quantize_linear(x, wq: QuantWeight, out_dtype=None, out=None, xq: QuantAct | None = None,
                    ws=None):
    """Quantize bf16 x [M][K] and apply the NVFP4 linear in one call (one
    kernel when possible); returns (y, xq), xq the quantized activation."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    if K != wq.K:
        raise ValueError("K mismatch")
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    y = out if out is not None else torch.empty((M, wq.N), dtype=out_dtype, device=x.device)
    q = xq if xq is not None else empty_act(M, K, x.device)
    if ws is None:
        need = _quantize_linear_workspace_bytes(M, wq.N, K)
        ws = workspace(M, wq.N, K, x.device)
        if ws.numel() < need:
            raise NVFP4Error(ERR_WORKSPACE, "quantize_linear workspace")
    _check(_quantize_linear(M, wq.N, K, _ptr(x), x.stride(0), _ptr(wq.codes), _ptr(wq.scales),
                            _ptr(wq.gscale), _ptr(y), od, _ptr(q.codes), _ptr(q.scales),
                            _ptr(q.gscale), _ptr(ws), ws.numel(), _stream(y)),
           "nvfp4_quantize_linear")
    return y, q


def _out_args(x, wq, out_dtype, out):
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    if x.shape[1] != wq.K:
        raise ValueError("K mismatch")
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    y = out if out is not None else torch.empty((x.shape[0], wq.N), dtype=out_dtype,
                                                device=x.device)
    return y, od


def quantize_linear_static(x, gscale, wq: QuantWeight, out_dtype=None, out=None,
                           xq: QuantAct | None = None, ws=None):
    """quantize_linear with a caller-supplied activation tensor scale
    (float32 device tensor [1]); returns (y, xq) with xq.gscale = gscale."""
    torch = _torch()
    if gscale.dtype != torch.float32 or gscale.numel() < 1:
        raise ValueError("gscale must be a float32 device tensor")
    y, od = _out_args(x, wq, out_dtype, out)
    M, K = x.shape
    q = xq if xq is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(M, wq.N, K, x.device)
    _check(_quantize_linear_static(M, wq.N, K, _ptr(x), x.stride(0), _ptr(gscale),
                                   _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), od,
                                   _ptr(q.codes), _ptr(q.scales), _ptr(ws), ws.numel(),
                                   _stream(y)), "nvfp4_quantize_linear_static")
    return y, QuantAct(q.codes, q.scales, gscale, M, K)


def quantize_linear_noalloc(x, wq: QuantWeight, out, xq: QuantAct):
    """quantize_linear on the library's own scratch workspace (no workspace
    argument, nothing allocated by the call): the caller passes the output
    and the quantized-activation buffers."""
    y, od = _out_args(x, wq, None, out)
    M, K = x.shape
    _check(_quantize_linear_noalloc(M, wq.N, K, _ptr(x), x.stride(0), _ptr(wq.codes),
                                    _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), od,
                                    _ptr(xq.codes), _ptr(xq.scales), _ptr(xq.gscale),
                                    _stream(y)), "nvfp4_quantize_linear_noalloc")
    return y, xq


def rmsnorm_quantize_linear(x, wq: QuantWeight, eps=1e-6, out_dtype=None, out=None,
                            xq: QuantAct | None = None, h_out=None, ws=None):
    """Unweighted per-row RMS norm of bf16 x [M][K], quantization and the
    NVFP4 linear in one call (one kernel when possible); returns (y, xq)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    if K != wq.K:
        raise ValueError("K mismatch")
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    y = out if out is not None else torch.empty((M, wq.N), dtype=out_dtype, device=x.device)
    q = xq if xq is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(M, wq.N, K, x.device)
    _check(_rmsnorm_quantize_linear(M, wq.N, K, _ptr(x), x.stride(0), float(eps), _ptr(wq.codes),
                                    _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), od, _ptr(q.codes),
                                    _ptr(q.scales), _ptr(q.gscale), _nullable(h_out), _ptr(ws),
                                    ws.numel(), _stream(y)), "nvfp4_rmsnorm_quantize_linear")
    return y, q


def quantize_act_f32(x, amax=None, out: QuantAct | None = None, ws=None) -> QuantAct:
    """Quantize a float32 activation [M][K] (row stride a multiple of 4);
    amax: the producer's uint32 maxima record, or None."""
    torch = _torch()
    if x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 tensor with unit column stride")
    M, K = x.shape
    q = out if out is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(M, 1, K, x.device, need=256)
    _check(_quantize_act_f32(_ptr(x), M, K, x.stride(0), _nullable(amax), _ptr(q.codes),
                             _ptr(q.scales), _ptr(q.gscale), _ptr(ws), ws.numel(), _stream(x)),
           "nvfp4_quantize_act_f32")
    return q


def quantize_linear_f32(x, wq: QuantWeight, amax=None, out_dtype=None, out=None,
                        xq: QuantAct | None = None, ws=None):
    """Quantize float32 x [M][K] and apply the NVFP4 linear (one kernel when
    possible; with the producer's maxima record `amax` also for activations
    too large for one workgroup's prologue); returns (y, xq)."""
    torch = _torch()
    if x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 tensor with unit column stride")
    M, K = x.shape
    if K != wq.K:
        raise ValueError("K mismatch")
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    y = out if out is not None else torch.empty((M, wq.N), dtype=out_dtype, device=x.device)
    q = xq if xq is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(M, wq.N, K, x.device,
                       need=_quantize_linear_f32_workspace_bytes(M, wq.N, K))
    _check(_quantize_linear_f32(M, wq.N, K, _ptr(x), x.stride(0), _nullable(amax), _ptr(wq.codes),
                                _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), od, _ptr(q.codes),
                                _ptr(q.scales), _ptr(q.gscale), _ptr(ws), ws.numel(), _stream(y)),
           "nvfp4_quantize_linear_f32")
    return y, q


def quantize_linear_silu_mul(x, wq: QuantWeight, rmsnorm=False, eps=1e-6, h=None, amax=None,
                             gu_out=None, xq: QuantAct | None = None, xh_out=None, ws=None):
    """gate_up linear of bf16 x [M][K] (RMS-normalised first with rmsnorm)
    with SiLU * mul applied in its epilogue: wq is the gate_up weight [2F][K];
    returns (h [M][F] float32, amax record [256] int32 holding uint32 words,
    xq)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    if K != wq.K or wq.N % 2 or not wq.gate_up:
        raise ValueError("wq must be a gate_up weight from quantize_weight_gate_up with K = x's")
    F = wq.N // 2
    h = h if h is not None else torch.empty((M, F), dtype=torch.float32, device=x.device)
    if h.dtype != torch.float32 or h.dim() != 2 or h.stride(1) != 1 or h.shape != (M, F):
        raise ValueError("h must be a float32 [M][F] tensor with unit column stride")
    amax = amax if amax is not None else torch.empty(AMAX_RECORD_WORDS, dtype=torch.int32,
                                                     device=x.device)
    q = xq if xq is not None else empty_act(M, K, x.device)
    if ws is None:
        ws = workspace(M, 1, K, x.device, need=256)
    _check(_quantize_linear_silu_mul(M, F, K, _ptr(x), x.stride(0), 1 if rmsnorm else 0,
                                     float(eps), _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.gscale),
                                     _ptr(h), h.stride(0), _ptr(amax), _nullable(gu_out),
                                     _ptr(q.codes), _ptr(q.scales), _ptr(q.gscale),
                                     _nullable(xh_out), _ptr(ws), ws.numel(), _stream(h)),
           "nvfp4_quantize_linear_silu_mul")
    return h, amax, q


def reset_workspace_bytes(M: int, V: int) -> int:
    return _reset_workspace_bytes(M, V)


def reset_temperature(logits, params: ResetParams, state, step_end=None, out=None, ws=None):
    """ReSET's step-aware temperature for float32 logits [M][V] (row stride
    a multiple of 4): returns (entropy [M], temperature [M], out) where out
    is logits / temperature per row (out=None: not computed; out="inplace":
    written over logits).  state is the float32 [M][2] running (sum, count)
    of each row's current step, updated in place; step_end an int32 [M]
    tensor flagging rows whose previous token closed a step."""
    torch = _torch()
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D float32 tensor with unit column stride")
    M, V = logits.shape
    ent = torch.empty(M, dtype=torch.float32, device=logits.device)
    tmp = torch.empty(M, dtype=torch.float32, device=logits.device)
    if isinstance(out, str):
        if out != "inplace":
            raise ValueError("out must be None, 'inplace' or a tensor")
        out = logits
    ldo = out.stride(0) if out is not None else 0
    if ws is None:
        need = reset_workspace_bytes(M, V)
        dev = logits.device
        key = ("reset", dev.index if dev.index is not None else torch.cuda.current_device())
        ws = _WS.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
            workspace_init(ws)
            _WS[key] = ws
    _check(_reset_temperature(_ptr(logits), M, V, logits.stride(0), ctypes.byref(params),
                              _ptr(state), _nullable(step_end), _ptr(ent), _ptr(tmp),
                              _nullable(out), ldo, _ptr(ws), ws.numel(), _stream(logits)),
           "nvfp4_reset_temperature")
    return ent, tmp, out


def linear(xq: QuantAct, wq: QuantWeight, out_dtype=None, out=None, ws=None):
    """y [M][N] = NVFP4 linear of the quantized activation and weight."""
    torch = _torch()
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    if xq.K != wq.K:
        raise ValueError("K mismatch")
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    y = out if out is not None else torch.empty((xq.M, wq.N), dtype=out_dtype,
                                                device=wq.codes.device)
    if ws is None:
        ws = workspace(xq.M, wq.N, wq.K, wq.codes.device)
    _check(_linear(xq.M, wq.N, wq.K, _ptr(xq.codes), _ptr(xq.scales), _ptr(xq.gscale),
                   _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), od, _ptr(ws),
                   ws.numel(), _stream(y)), "nvfp4_linear")
    return y
