"""Test-side constructions that pin the oracle to something other than itself.

Weights are built here as *values* first (closed-form E2M1 from the code's
bit fields, UE8M0 from ldexp, E4M3 from PyTorch's float8_e4m3fn cast), then
packed into codes and scales.  The fp64 dense layer below is the textbook
two-layer gated MLP on those values, written with numpy matmuls; it never
calls the oracle's decoders.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def e2m1_closed_form(nib: np.ndarray) -> np.ndarray:
    """E2M1 from its bit fields: sign s = bit 3, exponent e = bits 2..1,
    mantissa m = bit 0; e > 0 gives 2^(e-1) * (1 + m/2), e = 0 gives m/2."""
    nib = np.asarray(nib, dtype=np.int64)
    s = (nib >> 3) & 1
    e = (nib >> 1) & 3
    m = nib & 1
    mag = np.where(e > 0, np.ldexp(1.0 + m / 2.0, e - 1), m / 2.0)
    return np.where(s == 1, -mag, mag)


def ue8m0_value(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def e4m3_value(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """Element 2b in the low nibble of byte b, element 2b+1 in the high nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def make_matrix(rng: np.random.Generator, fmt: str, shape_rows: tuple, cols: int,
                global_scale: float = 1.0, scale_bytes: np.ndarray | None = None,
                nibbles: np.ndarray | None = None):
    """Returns (codes u8[..., cols/2], scales u8[..., cols/G], values f32[..., cols])."""
    G = 32 if fmt == "mxfp4" else 16
    if nibbles is None:
        nibbles = rng.integers(0, 16, size=shape_rows + (cols,), dtype=np.uint8)
    if scale_bytes is None:
        if fmt == "mxfp4":
            scale_bytes = rng.integers(118, 127, size=shape_rows + (cols // G,), dtype=np.uint8)
        else:
            v = np.minimum(np.abs(rng.standard_normal(shape_rows + (cols // G,))) * 64, 448)
            scale_bytes = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sv = ue8m0_value(scale_bytes) if fmt == "mxfp4" else e4m3_value(scale_bytes)
    sv_full = np.repeat(sv, G, axis=-1)
    vals = (e2m1_closed_form(nibbles).astype(np.float32) * sv_full.astype(np.float32)).astype(np.float32)
    if fmt == "nvfp4":
        vals = (vals * np.float32(global_scale)).astype(np.float32)
    return pack_nibbles(nibbles), np.ascontiguousarray(scale_bytes, dtype=np.uint8), vals


def bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dense_layer_f64(w13: np.ndarray, w2: np.ndarray, x: np.ndarray, ids: np.ndarray,
                    w: np.ndarray, act=None) -> np.ndarray:
    """Textbook gated MLP per route, summed with router weights, in fp64.
    w13 [E][2I][H] (gate rows first), w2 [E][H][I], x [M][H]; `act(g, u)`
    replaces SiLU(g) * u when given."""
    E, twoI, H = w13.shape
    I = twoI // 2
    M, k = ids.shape
    out = np.zeros((M, H), dtype=np.float64)
    for t in range(M):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0 or e >= E:
                continue
            g = w13[e, :I].astype(np.float64) @ x[t].astype(np.float64)
            u = w13[e, I:].astype(np.float64) @ x[t].astype(np.float64)
            a = g / (1.0 + np.exp(-g)) * u if act is None else act(g, u)
            out[t] += float(w[t, j]) * (w2[e].astype(np.float64) @ a)
    return out


def random_case(rng: np.random.Generator, fmt: str, E: int, H: int, I: int, M: int, k: int,
                g13: float = 1.0 / 512, g2: float = 1.0 / 512):
    """A small random layer call plus its float weight values."""
    c13, s13, v13 = make_matrix(rng, fmt, (E, 2 * I), H, g13)
    c2, s2, v2 = make_matrix(rng, fmt, (E, H), I, g2)
    x = bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    w = rng.random((M, k)).astype(np.float32)
    d = dict(w13_codes=c13, w13_scales=s13, w2_codes=c2, w2_scales=s2, x=x, ids=ids, w=w,
             g13=np.full(E, g13, np.float32) if fmt == "nvfp4" else None,
             g2=np.full(E, g2, np.float32) if fmt == "nvfp4" else None)
    return d, v13, v2


def ldexp1(e: int) -> float:
    return math.ldexp(1.0, e)
