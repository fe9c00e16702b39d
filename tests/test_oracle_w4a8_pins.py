"""Pins for the oracle's W4A8-MX step (MXFP4 weights, activations quantised
to MXFP8 per 32 values): the quantiser against PyTorch's float8_e4m3fn cast
and a brute-force nearest search, its scale against the OCP MX shared-exponent
property, the special blocks, and the layer against the textbook gated MLP on
quantised activations and a closed-form case whose act quantisation is exact
in one block and flushes in the other.  No GPU."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from pins_util import bf16_bits, bits_to_f32, dense_layer_f64, e4m3_value, make_matrix, random_case, ue8m0_value

# every finite non-negative E4M3 value, ascending (codes 0x00..0x7E)
E4M3_POS = e4m3_value(np.arange(0x7F, dtype=np.uint8))


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Test-side MXFP8 decode: torch's E4M3 value times 2^(s - 127)."""
    sv = np.repeat(ue8m0_value(scales), 32, axis=-1)
    return e4m3_value(codes) * sv


def test_codes_match_torch_e4m3fn_rne_at_unit_scale(oracle_lib):
    """With 256 in the block the shared exponent is 0, so codes are the RNE
    cast of the values themselves; exact midpoints check ties-to-even."""
    rng = np.random.default_rng(5)
    mids = (E4M3_POS[1:] + E4M3_POS[:-1]) / 2
    vals = np.concatenate([E4M3_POS, mids, rng.uniform(0, 448, 2000), rng.uniform(0, 2.0 ** -5, 500)])
    vals = np.concatenate([vals, -vals])
    n = (len(vals) + 30) // 31 * 31
    vals = np.concatenate([vals, np.zeros(n - len(vals))]).reshape(-1, 31)
    block = np.concatenate([np.full((len(vals), 1), 256.0), vals], axis=1).astype(np.float32)
    assert np.array_equal(mids.astype(np.float32), mids)  # the ties are exact in fp32
    codes, scales = oracle_lib.mxfp8_quantize(block)
    assert np.all(scales == 127)
    want = torch.from_numpy(block).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)


def test_saturates_at_448(oracle_lib):
    v = np.zeros((1, 32), np.float32)
    v[0, :6] = [1.875, 1.8, 1.76, -1.99, 1.0, 0.5]  # shared exponent -8: values times 256
    codes, scales = oracle_lib.mxfp8_quantize(v)
    assert scales[0, 0] == 127 - 8
    # 480, 460.8, 450.56 and -509.44 are past 448: the largest finite code
    assert list(codes[0, :6]) == [0x7E, 0x7E, 0x7E, 0xFE, 0x78, 0x70]


def test_nearest_value_by_brute_force(oracle_lib):
    rng = np.random.default_rng(7)
    rows = 400
    v = rng.standard_normal((rows, 64)) * np.exp2(rng.integers(-40, 40, (rows, 1)))
    v *= np.exp2(rng.integers(-12, 1, (rows, 64)))  # spread within blocks, into subnormal E4M3
    v = v.astype(np.float32)
    codes, scales = oracle_lib.mxfp8_quantize(v)
    got = decode(codes, scales)
    X = np.repeat(ue8m0_value(scales), 32, axis=-1)
    t = np.abs(v.astype(np.float64)) / X
    assert np.all(t < 512)
    dist = np.abs(t[..., None] - E4M3_POS[None, None, :])
    best = dist.min(-1)
    chosen = np.abs(got) / X
    tol = 1e-12 * np.maximum(t, 1)
    sat = t > 448
    ok = np.abs(np.abs(chosen - t) - best) <= tol
    assert np.all(ok | sat)
    assert np.all(chosen[sat] == 448)
    # at a tie the even code wins
    tie = np.sum(np.abs(dist - best[..., None]) <= tol[..., None], -1) > 1
    assert np.all((codes[tie] & 1) == 0)
    # sign follows the value (zero codes keep the sign bit of the input)
    assert np.all((codes >> 7) == np.signbit(v))


def test_shared_exponent_puts_amax_in_top_binade(oracle_lib):
    """OCP MX: the scale is the power of two that brings the block maximum
    into [256, 512), the binade of E4M3's largest power of two."""
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((300, 32)) * np.exp2(rng.integers(-100, 100, (300, 1)))).astype(np.float32)
    codes, scales = oracle_lib.mxfp8_quantize(v)
    amax = np.abs(v.astype(np.float64)).max(1)
    ratio = amax / ue8m0_value(scales[:, 0])
    assert np.all((ratio >= 256) & (ratio < 512))


def test_special_blocks(oracle_lib):
    v = np.zeros((5, 32), np.float32)
    v[1, 3] = np.nan
    v[2, 0] = -np.inf
    v[2, 1] = 1.0
    v[3, :] = 2.0 ** -140            # subnormal fp32: shared exponent clamps at -127
    v[4, 0] = 3.0e38                 # floor(log2) = 127: shared 119
    codes, scales = oracle_lib.mxfp8_quantize(v)
    assert scales[0, 0] == 0 and np.all(codes[0] == 0)
    assert scales[1, 0] == 255 and np.all(codes[1] == 0x7F)
    assert scales[2, 0] == 255 and np.all(codes[2] == 0x7F)
    assert scales[3, 0] == 0
    # 2^-140 / 2^-127 = 2^-13 is below half the smallest subnormal (2^-10): zero
    assert np.all(codes[3] == 0)
    assert scales[4, 0] == 127 + 119
    assert math.isnan(oracle_lib.mxfp8_value(0x20, 255))


def test_layer_without_act_quant_is_textbook_mlp_on_mxfp8_x(oracle_lib):
    rng = np.random.default_rng(21)
    E, H, I, M, k = 5, 128, 64, 3, 3
    d, v13, v2 = random_case(rng, "mxfp4", E, H, I, M, k)
    d["ids"][0, 1] = -1
    d["ids"][2, 2] = d["ids"][2, 0]
    xc, xs = oracle_lib.mxfp8_quantize(bits_to_f32(d["x"]))
    xq = decode(xc, xs)
    assert np.mean(xq != bits_to_f32(d["x"])) > 0.5  # the quantisation does change x
    ref = dense_layer_f64(v13, v2, xq, d["ids"], d["w"])
    got = oracle_lib.forward_w4a8("mxfp4", d, quant_act=False)
    scale = np.abs(ref).max()
    # only the fp32 roundings of gate, up and the SiLU product separate them
    assert np.abs(got - ref).max() <= 1e-6 * scale


def test_act_blocks_run_along_I_closed_form(oracle_lib):
    """gate = 128 for every n (SiLU(128) = 128 exactly in fp64); up_0 = 2^13
    and up_n = 2^-6 otherwise, so a = [2^20, 2, 2, ...].  In block 0 (n < 32)
    the shared exponent is 12 and 2 / 2^12 = 2^-11 rounds to zero; block 1
    keeps its 2s exactly.  FC2 then sums exact products."""
    rng = np.random.default_rng(4)
    H = I = 64
    nib13 = np.full((1, 2 * I, H), 2, np.uint8)      # E2M1 code 2 = 1.0
    s13 = np.empty((1, 2 * I, H // 32), np.uint8)
    s13[0, :I] = 128                                 # gate: 64 * 2 = 128
    s13[0, I] = 127 + 7                              # up_0: 64 * 128 = 2^13
    s13[0, I + 1:] = 127 - 12                        # up_n: 64 * 2^-12 = 2^-6
    c13, s13, v13 = make_matrix(rng, "mxfp4", (1, 2 * I), H, scale_bytes=s13, nibbles=nib13)
    c2, sc2, v2 = make_matrix(rng, "mxfp4", (1, H), I)
    x = bf16_bits(np.ones((1, H), np.float32))
    d = dict(w13_codes=c13, w13_scales=s13, w2_codes=c2, w2_scales=sc2, x=x,
             ids=np.zeros((1, 1), np.int32), w=np.full((1, 1), 0.75, np.float32), g13=None, g2=None)
    aq = np.zeros(I)
    aq[0] = 2.0 ** 20
    aq[32:] = 2.0
    want = 0.75 * (v2[0].astype(np.float64) @ aq)
    got = oracle_lib.forward_w4a8("mxfp4", d)
    assert np.array_equal(got[0], want)
    a_plain = np.full(I, 2.0)
    a_plain[0] = 2.0 ** 20
    plain = oracle_lib.forward_w4a8("mxfp4", d, quant_act=False)
    assert np.array_equal(plain[0], 0.75 * (v2[0].astype(np.float64) @ a_plain))
    assert not np.array_equal(got, plain)


def test_w4a8_stays_close_to_the_bf16_layer(oracle_lib):
    """The pages report cos 0.9990 against an fp32 reference for the MXFP8
    path (b12x PR #22, note on activations staying bf16); on random data the
    quantised layer stays within that class."""
    rng = np.random.default_rng(33)
    d, v13, v2 = random_case(rng, "mxfp4", 6, 256, 128, 4, 4)
    a8 = oracle_lib.forward_w4a8("mxfp4", d).ravel()
    ref = oracle_lib.forward_f64("mxfp4", d).ravel()
    cos = a8 @ ref / np.linalg.norm(a8) / np.linalg.norm(ref)
    assert 0.998 <= cos < 1.0


def test_w4a8_invalid_and_nvfp4(oracle_lib):
    rng = np.random.default_rng(2)
    d, _, _ = random_case(rng, "mxfp4", 3, 64, 32, 2, 2)
    d["ids"][:] = -1
    d["w13_scales"][:] = 255  # NaN everywhere, never read
    assert np.array_equal(oracle_lib.forward_w4a8("mxfp4", d), np.zeros((2, 64)))
    dn, _, _ = random_case(rng, "nvfp4", 3, 64, 32, 2, 2)
    with pytest.raises(ValueError):
        oracle_lib.forward_w4a8("nvfp4", dn)
