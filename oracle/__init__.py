"""CPU oracle for the block-scaled FP4 mixture-of-experts layer (ctypes binding).

TEST INFRASTRUCTURE ONLY.  The oracle is plain single-threaded C++
(``moe_oracle.cpp``) that shares no code with the HIP library.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the library's product path never does.

Numpy arrays in the logical layout that ``block_scaled_fp4_gather_amd.synth``
produces go in; fp32 token sums and their bf16 bit patterns come out.  The
case dict may name the activation ("fn": "silu", "gelu_tanh",
"swigluoai" with "alpha", "beta", "limit", or "relu2", which is not gated:
W13 then has I rows); SiLU when absent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

FMT = {"mxfp4": 1, "nvfp4": 2}
ACT = {"silu": 0, "gelu_tanh": 1, "swigluoai": 2, "relu2": 3}


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c++17",
                               "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i = ctypes.c_int
        L.oracle_e2m1.argtypes = [ctypes.c_uint32]
        L.oracle_e2m1.restype = ctypes.c_float
        L.oracle_ue8m0.argtypes = [ctypes.c_uint32]
        L.oracle_ue8m0.restype = ctypes.c_float
        L.oracle_e4m3.argtypes = [ctypes.c_uint32]
        L.oracle_e4m3.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_dequant.argtypes = [i, u8p, u8p, ctypes.c_float, i, i, f32p]
        L.oracle_dequant.restype = i
        common = [i, i, i, i, i, i, u8p, u8p, u8p, u8p, f32p, f32p, u16p, i64p, f32p]
        actp = [i, ctypes.c_float, ctypes.c_float, ctypes.c_float]
        L.oracle_forward_f32.argtypes = common + [f32p, u16p] + actp
        L.oracle_forward_f32.restype = i
        L.oracle_forward_f64.argtypes = common + [f64p] + actp
        L.oracle_forward_f64.restype = i
        L.oracle_mxfp8_quantize.argtypes = [f32p, i, i, u8p, u8p]
        L.oracle_mxfp8_quantize.restype = i
        L.oracle_mxfp8_value.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.oracle_mxfp8_value.restype = ctypes.c_double
        L.oracle_forward_w4a8.argtypes = common + [i, f64p] + actp
        L.oracle_activation.argtypes = [i] + [ctypes.c_double] * 5
        L.oracle_activation.restype = ctypes.c_double
        L.oracle_forward_w4a8.restype = i
        L.oracle_csf_encode.argtypes = [i, u8p, i, u8p, u8p]
        L.oracle_csf_encode.restype = i
        L.oracle_csf_decode.argtypes = [i, ctypes.c_uint8, u8p, u8p, i, u8p]
        L.oracle_csf_decode.restype = i
        _lib = L
    return _lib


def _p(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctype))
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def e2m1(nibble: int) -> float:
    return lib().oracle_e2m1(nibble)


def ue8m0(b: int) -> float:
    return lib().oracle_ue8m0(b)


def e4m3(b: int) -> float:
    return lib().oracle_e4m3(b)


def f32_to_bf16(f: float) -> int:
    return lib().oracle_f32_to_bf16(f)


def bf16_to_f32(h: int) -> float:
    return lib().oracle_bf16_to_f32(h)


def dequant(fmt: str, codes: np.ndarray, scales: np.ndarray, global_scale: float = 1.0) -> np.ndarray:
    """Dequantise one [rows][cols/2] code matrix with its [rows][cols/G] scales."""
    rows, half = codes.shape
    cols = 2 * half
    out = np.empty((rows, cols), dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rc = lib().oracle_dequant(FMT[fmt], _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8),
                              float(global_scale), rows, cols, _p(out, ctypes.c_float))
    if rc:
        raise ValueError("oracle_dequant rejected its arguments")
    return out


def _act(d):
    """(kind, alpha, beta, limit) from the case dict; SiLU when absent."""
    fn = d.get("fn", "silu")
    return [ACT.get(fn, fn), float(d.get("alpha", 0.0)), float(d.get("beta", 0.0)), float(d.get("limit", 0.0))]


def activation(fn: str, gate: float, up: float, alpha: float = 0.0, beta: float = 0.0, limit: float = 0.0) -> float:
    return lib().oracle_activation(ACT[fn], alpha, beta, limit, gate, up)


def _args(fmt, d):
    E, _, Hh = d["w13_codes"].shape
    H, I = 2 * Hh, 2 * d["w2_codes"].shape[2]  # W13 has 2I rows, or I for relu2
    M, k = d["ids"].shape
    arr = {key: np.ascontiguousarray(d[key]) for key in
           ("w13_codes", "w13_scales", "w2_codes", "w2_scales", "x", "w")}
    ids = np.ascontiguousarray(d["ids"], dtype=np.int64)
    g13 = None if d.get("g13") is None else np.ascontiguousarray(d["g13"], dtype=np.float32)
    g2 = None if d.get("g2") is None else np.ascontiguousarray(d["g2"], dtype=np.float32)
    keep = (arr, ids, g13, g2)
    args = [FMT[fmt], E, H, I, M, k,
            _p(arr["w13_codes"], ctypes.c_uint8), _p(arr["w13_scales"], ctypes.c_uint8),
            _p(arr["w2_codes"], ctypes.c_uint8), _p(arr["w2_scales"], ctypes.c_uint8),
            _p(g13, ctypes.c_float), _p(g2, ctypes.c_float),
            _p(arr["x"], ctypes.c_uint16), _p(ids, ctypes.c_int64), _p(arr["w"], ctypes.c_float)]
    return args, keep, M, H


def forward_f32(fmt: str, d: dict) -> tuple[np.ndarray, np.ndarray]:
    """Returns (fp32 token sums [M][H], bf16 bit patterns [M][H])."""
    args, keep, M, H = _args(fmt, d)
    acc = np.empty((M, H), dtype=np.float32)
    out = np.empty((M, H), dtype=np.uint16)
    rc = lib().oracle_forward_f32(*args, _p(acc, ctypes.c_float), _p(out, ctypes.c_uint16), *_act(d))
    if rc:
        raise ValueError("oracle_forward_f32 rejected its arguments")
    del keep
    return acc, out


def forward_f64(fmt: str, d: dict) -> np.ndarray:
    args, keep, M, H = _args(fmt, d)
    acc = np.empty((M, H), dtype=np.float64)
    rc = lib().oracle_forward_f64(*args, _p(acc, ctypes.c_double), *_act(d))
    if rc:
        raise ValueError("oracle_forward_f64 rejected its arguments")
    del keep
    return acc


def mxfp8_quantize(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 codes [rows][cols] and UE8M0 scales [rows][cols/32] of fp32 `v`."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, cols = v.shape
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    rc = lib().oracle_mxfp8_quantize(_p(v, ctypes.c_float), rows, cols, _p(codes, ctypes.c_uint8),
                                     _p(scales, ctypes.c_uint8))
    if rc:
        raise ValueError("oracle_mxfp8_quantize rejected its arguments")
    return codes, scales


def mxfp8_value(code: int, scale: int) -> float:
    return lib().oracle_mxfp8_value(code, scale)


def forward_w4a8(fmt: str, d: dict, quant_act: bool = True) -> np.ndarray:
    """The W4A8-MX layer (MXFP4 only) in fp64: [M][H] token sums."""
    args, keep, M, H = _args(fmt, d)
    acc = np.empty((M, H), dtype=np.float64)
    rc = lib().oracle_forward_w4a8(*args, int(bool(quant_act)), _p(acc, ctypes.c_double), *_act(d))
    if rc:
        raise ValueError("oracle_forward_w4a8 rejected its arguments")
    del keep
    return acc


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (a bit shift, no rounding)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def csf_encode(fmt: str, scales: np.ndarray) -> tuple[int, np.ndarray, bool]:
    """Compressed-scale encoding of one row of scale bytes: (base byte,
    offsets one per block, compressed?); an exception row has base 255."""
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    base = np.zeros(1, dtype=np.uint8)
    off = np.zeros(sc.size, dtype=np.uint8)
    rc = lib().oracle_csf_encode(FMT[fmt], _p(sc, ctypes.c_uint8), sc.size, _p(base, ctypes.c_uint8),
                                 _p(off, ctypes.c_uint8))
    if rc < 0:
        raise ValueError("oracle_csf_encode rejected its arguments")
    return int(base[0]), off, bool(rc)


def csf_decode(fmt: str, base: int, offsets: np.ndarray, plain: np.ndarray) -> np.ndarray:
    """A row's scale bytes from its base and offsets (an exception row, base
    255, from `plain`)."""
    off = np.ascontiguousarray(offsets, dtype=np.uint8)
    pl = np.ascontiguousarray(plain, dtype=np.uint8)
    out = np.empty(off.size, dtype=np.uint8)
    rc = lib().oracle_csf_decode(FMT[fmt], base, _p(off, ctypes.c_uint8), _p(pl, ctypes.c_uint8), off.size,
                                 _p(out, ctypes.c_uint8))
    if rc:
        raise ValueError("oracle_csf_decode rejected its arguments")
    return out
