"""ctypes binding of libmoe_fp4.so (include/moe_fp4.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory and streams.  Loading fails loudly when the
library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp4.so")

MXFP4 = 1
NVFP4 = 2
FORMATS = {"mxfp4": MXFP4, "nvfp4": NVFP4}

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or size",
          3: "buffer too small", 4: "HIP launch or runtime error"}


class MoeFp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


PATH_AUTO, PATH_DECODE, PATH_GROUPED = 0, 1, 2

ACT_BF16, ACT_MXFP8 = 0, 1
ACT_FORMATS = {"bf16": ACT_BF16, "mxfp8": ACT_MXFP8}

SCALES_PLAIN, SCALES_CSF = 0, 1
SCALE_FORMATS = {"plain": SCALES_PLAIN, "csf": SCALES_CSF}

FN_SILU, FN_GELU_TANH, FN_SWIGLUOAI, FN_RELU2 = 0, 1, 2, 3
ACT_FNS = {"silu": FN_SILU, "gelu_tanh": FN_GELU_TANH, "swigluoai": FN_SWIGLUOAI, "relu2": FN_RELU2}


class Tuning(ctypes.Structure):
    """Launch shape of the decode kernels and the execution path (0 keeps the
    built-in choice; path is PATH_AUTO, PATH_DECODE or PATH_GROUPED)."""
    _fields_ = [("fc1_chunks_per_wave", ctypes.c_int32), ("fc1_rows", ctypes.c_int32),
                ("fc2_rows", ctypes.c_int32), ("path", ctypes.c_int32)]


class _Desc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("act_format", ctypes.c_int32), ("act_fn", ctypes.c_int32),
                ("act_alpha", ctypes.c_float), ("act_beta", ctypes.c_float), ("act_limit", ctypes.c_float),
                ("scale_format", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class Desc:
    """Layer shape; `act` is "bf16" or "mxfp8" (the W4A8-MX variant of the
    grouped path, MXFP4 weights only); `fn` the activation ("silu",
    "gelu_tanh", "swigluoai" with alpha, beta and limit, or the non-gated
    "relu2", whose W13 has I rows); `scales` "plain" or "csf" (the
    compressed scale format, read by the decode path)."""
    fmt: str
    E: int
    H: int
    I: int
    k: int
    max_tokens: int
    act: str = "bf16"
    fn: str = "silu"
    alpha: float = 0.0
    beta: float = 0.0
    limit: float = 0.0
    scales: str = "plain"

    def c(self) -> _Desc:
        act = ACT_FORMATS.get(self.act, self.act) if isinstance(self.act, str) else self.act
        fn = ACT_FNS.get(self.fn, self.fn) if isinstance(self.fn, str) else self.fn
        return _Desc(FORMATS.get(self.fmt, self.fmt) if isinstance(self.fmt, str) else self.fmt,
                     self.E, self.H, self.I, self.k, self.max_tokens, act, fn,
                     self.alpha, self.beta, self.limit, SCALE_FORMATS.get(self.scales, self.scales)
                     if isinstance(self.scales, str) else self.scales)


_lib = None
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32

_SIGS = {
    "moe_fp4_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_fp4_prepared_bytes": ([ctypes.POINTER(_Desc), ctypes.POINTER(_SZ)], ctypes.c_int),
    "moe_fp4_prepare": ([ctypes.POINTER(_Desc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_fp4_unprepare": ([ctypes.POINTER(_Desc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "moe_fp4_workspace_bytes": ([ctypes.POINTER(_Desc), _I32, ctypes.POINTER(_SZ)], ctypes.c_int),
    "moe_fp4_forward": ([ctypes.POINTER(_Desc), _VP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_fp4_forward_i64": ([ctypes.POINTER(_Desc), _VP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_fp4_forward_noalloc": ([ctypes.POINTER(_Desc), _VP, _VP, _I32, _VP, _VP, _VP, _VP], ctypes.c_int),
    "moe_fp4_forward_ex": ([ctypes.POINTER(_Desc), _VP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ,
                            ctypes.POINTER(Tuning), _I32, _VP], ctypes.c_int),
    "moe_fp4_plan": ([ctypes.POINTER(_Desc), _I32, ctypes.POINTER(Tuning), ctypes.POINTER(Tuning)], ctypes.c_int),
    "moe_fp4_dequant_export": ([ctypes.POINTER(_Desc), _VP, _I32, _I32, _VP, _VP], ctypes.c_int),
    "moe_fp4_mxfp8_quantize": ([_VP, ctypes.c_int64, _I32, _VP, _VP, _VP], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """Load libmoe_fp4.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_scaled_fp4_gather_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeFp4Error(fn, status)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    assert t.is_contiguous(), "tensors must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def status_string(s: int) -> str:
    return lib().moe_fp4_status_string(s).decode()


def prepared_bytes(desc: Desc) -> int:
    n = _SZ()
    _check("moe_fp4_prepared_bytes", lib().moe_fp4_prepared_bytes(ctypes.byref(desc.c()), ctypes.byref(n)))
    return n.value


def workspace_bytes(desc: Desc, M: int) -> int:
    n = _SZ()
    _check("moe_fp4_workspace_bytes", lib().moe_fp4_workspace_bytes(ctypes.byref(desc.c()), M, ctypes.byref(n)))
    return n.value


def prepare(desc: Desc, w13_codes, w13_scales, w2_codes, w2_scales, g13, g2, prepared, stream=None):
    _check("moe_fp4_prepare", lib().moe_fp4_prepare(
        ctypes.byref(desc.c()), _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes), _ptr(w2_scales),
        _ptr(g13), _ptr(g2), _ptr(prepared), prepared.numel() * prepared.element_size(), _stream(stream)))


def unprepare(desc: Desc, prepared, w13_codes, w13_scales, w2_codes, w2_scales, g13, g2, stream=None):
    _check("moe_fp4_unprepare", lib().moe_fp4_unprepare(
        ctypes.byref(desc.c()), _ptr(prepared), _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(g13), _ptr(g2), _stream(stream)))


def forward(desc: Desc, prepared, x, ids, w, out, workspace, stream=None, tuning: Tuning | None = None,
            phases: int | None = None):
    """x bf16 [M][H], ids int32 or int64 [M][k], w fp32 [M][k], out bf16 [M][H].
    `tuning` and `phases` select the measurement hook (int32 ids only)."""
    M = x.shape[0]
    ws_n = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(desc.c()), _ptr(prepared), _ptr(x), M, _ptr(ids), _ptr(w), _ptr(out),
            _ptr(workspace), ws_n)
    if tuning is not None or phases is not None:
        assert ids.dtype == torch.int32
        tp = ctypes.byref(tuning) if tuning is not None else None
        _check("moe_fp4_forward_ex", lib().moe_fp4_forward_ex(*args, tp, 3 if phases is None else phases,
                                                               _stream(stream)))
    elif ids.dtype == torch.int64:
        _check("moe_fp4_forward_i64", lib().moe_fp4_forward_i64(*args, _stream(stream)))
    else:
        assert ids.dtype == torch.int32
        _check("moe_fp4_forward", lib().moe_fp4_forward(*args, _stream(stream)))


def forward_noalloc(desc: Desc, prepared, x, ids, w, out, stream=None):
    """moe_fp4_forward with the library's own 64 MiB workspace (int32 ids):
    the entry point for callers that cannot allocate."""
    assert ids.dtype == torch.int32
    _check("moe_fp4_forward_noalloc", lib().moe_fp4_forward_noalloc(
        ctypes.byref(desc.c()), _ptr(prepared), _ptr(x), x.shape[0], _ptr(ids), _ptr(w), _ptr(out),
        _stream(stream)))


def plan(desc: Desc, M: int, tuning: Tuning | None = None) -> Tuning:
    """The path and launch shape a forward call with M tokens takes (every
    field resolved; path is PATH_DECODE or PATH_GROUPED)."""
    out = Tuning()
    _check("moe_fp4_plan", lib().moe_fp4_plan(ctypes.byref(desc.c()), M,
                                              ctypes.byref(tuning) if tuning is not None else None,
                                              ctypes.byref(out)))
    return out


def dequant_export(desc: Desc, prepared, expert: int, which: int, out, stream=None):
    _check("moe_fp4_dequant_export", lib().moe_fp4_dequant_export(
        ctypes.byref(desc.c()), _ptr(prepared), expert, which, _ptr(out), _stream(stream)))


def mxfp8_quantize(x, codes=None, scales=None, stream=None):
    """MXFP8 codes uint8 [rows][cols] and scales uint8 [rows][cols/32] of bf16 x."""
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check("moe_fp4_mxfp8_quantize", lib().moe_fp4_mxfp8_quantize(
        _ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


class Fp4MoE:
    """Prepared weights plus a workspace on one device; call with x, ids, w."""

    def __init__(self, desc: Desc, w13_codes, w13_scales, w2_codes, w2_scales, g13=None, g2=None,
                 device="cuda", stream=None):
        self.desc = desc
        dev = torch.device(device)

        def dev_t(a, dtype):
            if a is None:
                return None
            t = a if isinstance(a, torch.Tensor) else torch.from_numpy(a)
            return t.to(device=dev, dtype=dtype).contiguous()

        tensors = [dev_t(a, torch.uint8) for a in (w13_codes, w13_scales, w2_codes, w2_scales)]
        g13 = dev_t(g13, torch.float32)
        g2 = dev_t(g2, torch.float32)
        self.prepared = torch.empty(prepared_bytes(desc), dtype=torch.uint8, device=dev)
        prepare(desc, *tensors, g13, g2, self.prepared, stream)
        del tensors
        self.workspace = torch.empty(workspace_bytes(desc, desc.max_tokens), dtype=torch.uint8, device=dev)

    def __call__(self, x, ids, w, out=None, stream=None, tuning=None, phases=None):
        if out is None:
            out = torch.empty_like(x)
        forward(self.desc, self.prepared, x, ids, w, out, self.workspace, stream, tuning, phases)
        return out
