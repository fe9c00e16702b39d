"""Pins for the CPU oracle: each test checks it against something other than
itself (closed forms of the formats, PyTorch's own fp8/bf16 casts, a textbook
fp64 gated MLP on weight values built before encoding, invariants the layer's
definition implies, and hand-derived closed-form fixtures).  No GPU."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

from pins_util import (bf16_bits, bits_to_f32, dense_layer_f64, e2m1_closed_form, e4m3_value,
                       make_matrix, pack_nibbles, random_case, ue8m0_value)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- formats ---------------------------------------------------------------

def test_e2m1_all_codes_match_bit_field_closed_form(oracle_lib):
    got = np.array([oracle_lib.e2m1(c) for c in range(16)])
    want = e2m1_closed_form(np.arange(16))
    assert np.array_equal(got, want)
    # code 8 is negative zero, code 0 positive zero
    assert math.copysign(1.0, oracle_lib.e2m1(8)) == -1.0
    assert math.copysign(1.0, oracle_lib.e2m1(0)) == 1.0


def test_ue8m0_all_codes_match_ldexp_and_torch(oracle_lib):
    got = np.array([oracle_lib.ue8m0(b) for b in range(256)], dtype=np.float64)
    want = ue8m0_value(np.arange(256))
    assert np.array_equal(got[:255], want[:255])
    assert math.isnan(got[255])
    lib_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(got[:255], lib_vals[:255])


def test_e4m3_all_codes_match_torch_float8_e4m3fn(oracle_lib):
    got = np.array([oracle_lib.e4m3(b) for b in range(256)], dtype=np.float64)
    want = e4m3_value(np.arange(256, dtype=np.uint8))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros and the subnormal range are exact
    assert math.copysign(1.0, got[0x80]) == -1.0
    assert got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x7E] == 448.0


def test_bf16_rne_matches_torch(oracle_lib):
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    bits = v.view(np.uint32).copy()
    bits[:200] = (bits[:200] & 0xFFFF0000) | 0x8000  # exact ties, both parities
    bits[200:400] = (bits[200:400] & 0xFFFF0000) | 0x7FFF
    bits[400:600] = (bits[400:600] & 0xFFFF0000) | 0x8001
    v = bits.view(np.float32)
    extra = np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-45], dtype=np.float32)
    v = np.concatenate([v, extra])
    got = np.array([oracle_lib.f32_to_bf16(float(f)) for f in v], dtype=np.uint16)
    assert np.array_equal(got, bf16_bits(v))
    nanbits = oracle_lib.f32_to_bf16(float("nan"))
    assert (nanbits & 0x7F80) == 0x7F80 and (nanbits & 0x7F) != 0


# ---- dequantisation ----------------------------------------------------------

def test_nibble_order_low_first(oracle_lib):
    codes = np.array([[0x21] + [0] * 15, [0x9A] + [0] * 15], dtype=np.uint8)
    scales = np.full((2, 1), 127, dtype=np.uint8)
    d = oracle_lib.dequant("mxfp4", codes, scales)
    assert d[0, 0] == 0.5 and d[0, 1] == 1.0
    assert d[1, 0] == -1.0 and d[1, 1] == -0.5


def test_dequant_mxfp4_all_codes_times_all_scales(oracle_lib):
    # row b uses scale byte b; column c holds code c % 16
    nib = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :].repeat(256, axis=0)
    codes = pack_nibbles(nib)
    scales = np.arange(256, dtype=np.uint8)[:, None]
    d = oracle_lib.dequant("mxfp4", codes, scales)
    with np.errstate(over="ignore"):  # 3 * 2^127 and up overflow fp32 to inf
        want = (e2m1_closed_form(nib).astype(np.float32)
                * ue8m0_value(np.arange(256))[:, None].astype(np.float32))
    assert np.array_equal(d[:255], want[:255])
    assert np.isinf(d[254, 5])
    assert np.isnan(d[255]).all()


@pytest.mark.parametrize("g", [1.0 / 512, 1.0, 0.3, 3.7])
def test_dequant_nvfp4_all_codes_times_all_scales(oracle_lib, g):
    nib = np.arange(16, dtype=np.uint8)[None, :].repeat(256, axis=0)
    codes = pack_nibbles(nib)
    scales = np.arange(256, dtype=np.uint8)[:, None]
    d = oracle_lib.dequant("nvfp4", codes, scales, g)
    s = e4m3_value(np.arange(256, dtype=np.uint8))[:, None].astype(np.float32)
    want = (e2m1_closed_form(nib).astype(np.float32) * s).astype(np.float32) * np.float32(g)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], want[~nan])


def test_dequant_scale_blocks_follow_columns(oracle_lib):
    """One scale per 32 (MX) or 16 (NV) consecutive columns of a row."""
    rng = np.random.default_rng(7)
    for fmt in ("mxfp4", "nvfp4"):
        codes, scales, vals = make_matrix(rng, fmt, (24,), 128, 0.75)
        d = oracle_lib.dequant(fmt, codes, scales, 0.75)
        assert np.array_equal(d, vals)


# ---- the layer ---------------------------------------------------------------

CASES = [
    ("mxfp4", 4, 64, 32, 1, 2),
    ("mxfp4", 6, 96, 64, 3, 3),
    ("nvfp4", 5, 64, 48, 2, 4),
    ("nvfp4", 3, 32, 16, 4, 1),
]


@pytest.mark.parametrize("fmt,E,H,I,M,k", CASES)
def test_forward_f32_matches_textbook_fp64_mlp(oracle_lib, fmt, E, H, I, M, k):
    rng = np.random.default_rng(E * 1000 + H + I + M)
    d, v13, v2 = random_case(rng, fmt, E, H, I, M, k)
    d["ids"][0, 0] = -1  # an invalid route
    if M > 1 and k > 1:
        d["ids"][1, 1] = d["ids"][1, 0]  # a duplicate route
    ref = dense_layer_f64(v13, v2, bits_to_f32(d["x"]), d["ids"], d["w"])
    acc, out = oracle_lib.forward_f32(fmt, d)
    scale = np.abs(ref).max()
    assert scale > 0
    assert np.abs(acc - ref).max() <= 2e-5 * scale
    # fp64 twin agrees with the textbook up to fp64 rounding
    acc64 = oracle_lib.forward_f64(fmt, d)
    assert np.abs(acc64 - ref).max() <= 1e-12 * scale
    # the bf16 output is the RNE rounding of the fp32 sums
    assert np.array_equal(out, bf16_bits(acc))


def test_gate_and_up_are_not_interchangeable(oracle_lib):
    """Swapping the W13 halves changes the result (SiLU is applied to rows [0, I))."""
    rng = np.random.default_rng(3)
    d, v13, v2 = random_case(rng, "mxfp4", 2, 64, 32, 1, 1)
    acc, _ = oracle_lib.forward_f32("mxfp4", d)
    sw = dict(d)
    sw["w13_codes"] = np.ascontiguousarray(np.concatenate([d["w13_codes"][:, 32:], d["w13_codes"][:, :32]], 1))
    sw["w13_scales"] = np.ascontiguousarray(np.concatenate([d["w13_scales"][:, 32:], d["w13_scales"][:, :32]], 1))
    acc_sw, _ = oracle_lib.forward_f32("mxfp4", sw)
    ref_sw = dense_layer_f64(np.concatenate([v13[:, 32:], v13[:, :32]], 1), v2, bits_to_f32(d["x"]), d["ids"], d["w"])
    assert np.abs(acc_sw - ref_sw).max() <= 2e-5 * np.abs(ref_sw).max()
    assert np.abs(acc - acc_sw).max() > 1e-3 * np.abs(acc).max()


def test_invalid_ids_skip_even_with_nan_expert_zero(oracle_lib):
    rng = np.random.default_rng(11)
    for fmt, poison in (("mxfp4", 0xFF), ("nvfp4", 0x7F)):
        d, _, _ = random_case(rng, fmt, 4, 64, 32, 3, 4)
        d["ids"][:, :] = rng.integers(1, 4, size=(3, 4))
        d["w13_scales"][0] = poison
        d["w2_scales"][0] = poison
        d["ids"][:, 2] = [-1, 4, 2**31 - 1]
        acc, out = oracle_lib.forward_f32(fmt, d)
        assert np.isfinite(acc).all()
        kept = dict(d)
        kept["ids"] = np.ascontiguousarray(d["ids"][:, [0, 1, 3]])
        kept["w"] = np.ascontiguousarray(d["w"][:, [0, 1, 3]])
        acc_k, out_k = oracle_lib.forward_f32(fmt, kept)
        assert np.array_equal(acc, acc_k) and np.array_equal(out, out_k)
        # a valid route to the poisoned expert does propagate NaN
        d2 = dict(d)
        d2["ids"] = d["ids"].copy()
        d2["ids"][1, 0] = 0
        acc2, _ = oracle_lib.forward_f32(fmt, d2)
        assert np.isnan(acc2[1]).any() and np.isfinite(acc2[[0, 2]]).all()


def test_all_invalid_gives_positive_zero(oracle_lib):
    rng = np.random.default_rng(12)
    d, _, _ = random_case(rng, "nvfp4", 3, 32, 16, 2, 3)
    d["ids"][:] = np.array([[-1, 3, -7], [1 << 30, -1, 3]], dtype=np.int32)
    acc, out = oracle_lib.forward_f32("nvfp4", d)
    assert np.array_equal(out, np.zeros_like(out))
    assert np.array_equal(acc.view(np.uint32), np.zeros_like(acc).view(np.uint32))


def test_zero_router_weight_equals_route_removed(oracle_lib):
    rng = np.random.default_rng(13)
    d, _, _ = random_case(rng, "mxfp4", 5, 64, 32, 2, 3)
    d["w"][:, 1] = 0.0
    acc, _ = oracle_lib.forward_f32("mxfp4", d)
    kept = dict(d)
    kept["ids"] = np.ascontiguousarray(d["ids"][:, [0, 2]])
    kept["w"] = np.ascontiguousarray(d["w"][:, [0, 2]])
    acc_k, _ = oracle_lib.forward_f32("mxfp4", kept)
    assert np.array_equal(acc, acc_k)
    d["w"][:] = 0.0
    acc0, out0 = oracle_lib.forward_f32("mxfp4", d)
    assert not np.any(acc0) and not np.any(out0 & 0x7FFF)


def test_expert_relabeling_is_bit_identical(oracle_lib):
    rng = np.random.default_rng(14)
    d, _, _ = random_case(rng, "nvfp4", 6, 64, 32, 3, 2)
    d["g13"] = rng.random(6).astype(np.float32) + 0.5
    d["g2"] = rng.random(6).astype(np.float32) + 0.5
    acc, out = oracle_lib.forward_f32("nvfp4", d)
    perm = rng.permutation(6)  # new expert p holds old expert perm[p]
    inv = np.argsort(perm)
    r = dict(d)
    for key in ("w13_codes", "w13_scales", "w2_codes", "w2_scales", "g13", "g2"):
        r[key] = np.ascontiguousarray(d[key][perm])
    r["ids"] = inv[d["ids"]].astype(np.int32)
    acc_r, out_r = oracle_lib.forward_f32("nvfp4", r)
    assert np.array_equal(acc, acc_r) and np.array_equal(out, out_r)


def test_zero_gate_codes_give_zero(oracle_lib):
    rng = np.random.default_rng(15)
    d, _, _ = random_case(rng, "mxfp4", 3, 64, 32, 2, 2)
    d["w13_codes"][:, :32] = 0
    acc, out = oracle_lib.forward_f32("mxfp4", d)
    assert not np.any(acc) and not np.any(out & 0x7FFF)


def test_signed_unit_weights_reduce_to_signed_sums(oracle_lib):
    """Codes +-1 with unit scales: gate and up are signed sums of x."""
    rng = np.random.default_rng(16)
    H, I = 64, 32
    nib13 = np.where(rng.random((1, 2 * I, H)) < 0.5, 0x2, 0xA).astype(np.uint8)
    nib2 = np.where(rng.random((1, H, I)) < 0.5, 0x2, 0xA).astype(np.uint8)
    sign13 = np.where(nib13 == 0x2, 1.0, -1.0)[0]
    sign2 = np.where(nib2 == 0x2, 1.0, -1.0)[0]
    x = bf16_bits(rng.standard_normal((1, H)).astype(np.float32))
    xf = bits_to_f32(x)[0].astype(np.float64)
    d = dict(w13_codes=pack_nibbles(nib13), w13_scales=np.full((1, 2 * I, H // 32), 127, np.uint8),
             w2_codes=pack_nibbles(nib2), w2_scales=np.full((1, H, I // 32), 127, np.uint8),
             x=x, ids=np.zeros((1, 1), np.int32), w=np.ones((1, 1), np.float32), g13=None, g2=None)
    g = np.array([np.sum(sign13[n] * xf) for n in range(I)])
    u = np.array([np.sum(sign13[I + n] * xf) for n in range(I)])
    a = g / (1 + np.exp(-g)) * u
    y = np.array([np.sum(sign2[h] * a) for h in range(H)])
    acc, _ = oracle_lib.forward_f32("mxfp4", d)
    assert np.abs(acc[0] - y).max() <= 1e-5 * np.abs(y).max()


def _read_golden(name):
    kv = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            kv[key] = vals
    return kv


@pytest.mark.parametrize("name", ["mxfp4_uniform.txt", "nvfp4_subnormal_scale.txt"])
def test_golden_closed_form_cases(oracle_lib, name):
    kv = _read_golden(name)
    fmt = kv["format"][0]
    E, H, I = int(kv["E"][0]), int(kv["H"][0]), int(kv["I"][0])
    G = 32 if fmt == "mxfp4" else 16
    rid, rw = int(kv["route"][0]), float(kv["route"][1])

    def code_byte(c):
        c = int(c, 0)
        return c | (c << 4)

    w13c = np.full((E, 2 * I, H // 2), code_byte(kv["w13_code"][0]), np.uint8)
    w2c = np.full((E, H, I // 2), code_byte(kv["w2_code"][0]), np.uint8)
    if rid != 0:
        w13c[0] = 0xFF
        w2c[0] = 0xFF
    d = dict(w13_codes=w13c, w13_scales=np.full((E, 2 * I, H // G), int(kv["w13_scale"][0], 0), np.uint8),
             w2_codes=w2c, w2_scales=np.full((E, H, I // G), int(kv["w2_scale"][0], 0), np.uint8),
             x=np.full((1, H), int(kv["x_bf16"][0], 0), np.uint16),
             ids=np.array([[rid]], np.int32), w=np.array([[rw]], np.float32),
             g13=np.full(E, float(kv["g13"][0]), np.float32) if "g13" in kv else None,
             g2=np.full(E, float(kv["g2"][0]), np.float32) if "g2" in kv else None)
    acc, out = oracle_lib.forward_f32(fmt, d)
    want = float(kv["expected_acc"][0])
    assert np.abs(acc - want).max() <= 1e-6 * abs(want)
    assert np.all(out == int(kv["expected_bf16"][0], 0))


def test_oracle_runs_a_page_geometry_token(oracle_lib):
    """One token of the E512/H2560/I320 NVFP4 geometry finishes and is finite."""
    from block_scaled_fp4_gather_amd import synth

    wl = synth.WORKLOADS["nvfp4_decode_e512"].replace(E=16)
    d = synth.generate(wl)
    d["ids"] = d["ids"] % 16
    acc, out = oracle_lib.forward_f32("nvfp4", d)
    assert np.isfinite(acc).all() and np.abs(acc).max() > 0
