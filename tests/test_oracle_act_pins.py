"""Pins for the oracle's gated activations: gelu_tanh and SiLU against
PyTorch's own functions, swigluoai against its SiLU special case and a form
built from torch's clamp and silu, the clamps' invariances and NaN
pass-through, and the layer with each activation against the textbook gated
MLP.  No GPU."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from pins_util import bits_to_f32, dense_layer_f64, random_case

PTS = np.concatenate([np.linspace(-12, 12, 241), [-80.0, -30.0, -1e-3, 0.0, 1e-3, 30.0, 80.0]])


def test_gelu_tanh_matches_torch(oracle_lib):
    got = np.array([oracle_lib.activation("gelu_tanh", g, 1.0) for g in PTS])
    want = F.gelu(torch.from_numpy(PTS), approximate="tanh").numpy()
    # far below zero 1 + tanh cancels: both sides are within an fp64 ulp of 1
    # times 0.5 |x| of the true value (about -1.8e-16 at x = -7.2)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15 * np.max(np.abs(PTS)))
    # the up factor multiplies
    assert oracle_lib.activation("gelu_tanh", 1.5, -2.0) == pytest.approx(-2.0 * oracle_lib.activation("gelu_tanh", 1.5, 1.0), rel=1e-15)


def test_silu_matches_torch(oracle_lib):
    got = np.array([oracle_lib.activation("silu", g, 0.75) for g in PTS])
    want = 0.75 * F.silu(torch.from_numpy(PTS)).numpy()
    assert np.allclose(got, want, rtol=1e-13, atol=1e-300)


def test_swigluoai_reduces_to_silu(oracle_lib):
    """alpha = 1, beta = 0 and an infinite limit leave SiLU(gate) * up."""
    for g, u in [(0.3, 2.0), (-4.0, 1.5), (9.0, -3.0), (25.0, 40.0)]:
        assert oracle_lib.activation("swigluoai", g, u, 1.0, 0.0, math.inf) == pytest.approx(
            oracle_lib.activation("silu", g, u), rel=1e-15)


@pytest.mark.parametrize("alpha,beta,limit", [(1.702, 1.0, 7.0), (0.5, -0.25, 2.0), (3.0, 0.0, 100.0)])
def test_swigluoai_against_torch_clamp_and_silu(oracle_lib, alpha, beta, limit):
    rng = np.random.default_rng(int(alpha * 1000))
    g = rng.normal(0, 6, 400)
    u = rng.normal(0, 6, 400)
    got = np.array([oracle_lib.activation("swigluoai", a, b, alpha, beta, limit) for a, b in zip(g, u)])
    gt, ut = torch.from_numpy(g), torch.from_numpy(u)
    gc = torch.clamp(gt, max=limit)
    uc = torch.clamp(ut, min=-limit, max=limit)
    want = (F.silu(alpha * gc) / alpha * (uc + beta)).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_swigluoai_clamps(oracle_lib):
    a = lambda g, u: oracle_lib.activation("swigluoai", g, u, 1.702, 1.0, 7.0)
    assert a(7.0, 2.0) == a(9.0, 2.0) == a(1e6, 2.0)          # gate clamped above only
    assert a(-9.0, 2.0) != a(-7.0, 2.0)
    assert a(3.0, 7.0) == a(3.0, 50.0) and a(3.0, -7.0) == a(3.0, -50.0)
    assert math.isnan(a(math.nan, 1.0)) and math.isnan(a(1.0, math.nan))
    assert math.isnan(oracle_lib.activation("gelu_tanh", math.nan, 1.0))


@pytest.mark.parametrize("fn,alpha,beta,limit", [("gelu_tanh", 0.0, 0.0, 0.0), ("swigluoai", 1.702, 1.0, 7.0),
                                                 ("swigluoai", 1.0, 0.5, 1.5)])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_layer_with_activation_is_textbook_mlp(oracle_lib, fn, alpha, beta, limit, fmt):
    rng = np.random.default_rng(7 + len(fn) + int(limit))
    # the layer takes its activation parameters as fp32
    alpha, beta, limit = (float(np.float32(v)) for v in (alpha, beta, limit))
    d, v13, v2 = random_case(rng, fmt, 5, 96, 64, 3, 3)
    d.update(fn=fn, alpha=alpha, beta=beta, limit=limit)
    d["ids"][0, 0] = -1
    if fn == "gelu_tanh":
        act = lambda g, u: F.gelu(torch.from_numpy(g), approximate="tanh").numpy() * u
    else:
        act = lambda g, u: (F.silu(alpha * torch.clamp(torch.from_numpy(g), max=limit)).numpy() / alpha
                            * (np.clip(u, -limit, limit) + beta))
    ref = dense_layer_f64(v13, v2, bits_to_f32(d["x"]), d["ids"], d["w"], act)
    scale = np.abs(ref).max()
    assert np.abs(oracle_lib.forward_f64(fmt, d) - ref).max() <= 1e-12 * scale
    acc, _ = oracle_lib.forward_f32(fmt, d)
    assert np.abs(acc - ref).max() <= 2e-5 * scale
    # the activation matters: SiLU gives a different layer
    silu = dict(d, fn="silu")
    assert np.abs(oracle_lib.forward_f64(fmt, silu) - ref).max() > 1e-3 * scale
    if fmt == "mxfp4":
        a8 = oracle_lib.forward_w4a8(fmt, d)
        cos = float(a8.ravel() @ ref.ravel() / np.linalg.norm(a8) / np.linalg.norm(ref))
        assert cos > 0.995


def test_unknown_activation_rejected(oracle_lib):
    rng = np.random.default_rng(1)
    d, _, _ = random_case(rng, "mxfp4", 2, 64, 32, 1, 1)
    d["fn"] = 7
    with pytest.raises(ValueError):
        oracle_lib.forward_f64("mxfp4", d)


def test_relu2_matches_torch(oracle_lib):
    got = np.array([oracle_lib.activation("relu2", g, 123.0) for g in PTS])
    want = (F.relu(torch.from_numpy(PTS)) ** 2).numpy()
    assert np.array_equal(got, want)
    assert math.isnan(oracle_lib.activation("relu2", math.nan, 0.0))


def _relu2_case(rng, fmt, E, H, I, M, k):
    """A layer whose W13 has I rows (relu2 is not gated)."""
    from pins_util import bf16_bits, make_matrix
    c13, s13, v13 = make_matrix(rng, fmt, (E, I), H, 1.0 / 512)
    c2, s2, v2 = make_matrix(rng, fmt, (E, H), I, 1.0 / 512)
    d = dict(w13_codes=c13, w13_scales=s13, w2_codes=c2, w2_scales=s2,
             x=bf16_bits(rng.standard_normal((M, H)).astype(np.float32)),
             ids=rng.integers(0, E, size=(M, k)).astype(np.int32), w=rng.random((M, k)).astype(np.float32),
             g13=np.full(E, 1.0 / 512, np.float32) if fmt == "nvfp4" else None,
             g2=np.full(E, 1.0 / 512, np.float32) if fmt == "nvfp4" else None, fn="relu2")
    return d, v13, v2


def _relu2_textbook(v13, v2, x, ids, w):
    M, k = ids.shape
    out = np.zeros((M, v2.shape[1]))
    for t in range(M):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < v13.shape[0]:
                h = v13[e].astype(np.float64) @ x[t].astype(np.float64)
                out[t] += float(w[t, j]) * (v2[e].astype(np.float64) @ (F.relu(torch.from_numpy(h)) ** 2).numpy())
    return out


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_relu2_layer_is_textbook_non_gated_mlp(oracle_lib, fmt):
    rng = np.random.default_rng(17)
    d, v13, v2 = _relu2_case(rng, fmt, 5, 96, 64, 3, 3)
    d["ids"][1, 2] = -1
    ref = _relu2_textbook(v13, v2, bits_to_f32(d["x"]), d["ids"], d["w"])
    scale = np.abs(ref).max()
    assert np.abs(oracle_lib.forward_f64(fmt, d) - ref).max() <= 1e-12 * scale
    acc, _ = oracle_lib.forward_f32(fmt, d)
    assert np.abs(acc - ref).max() <= 2e-5 * scale
    if fmt == "mxfp4":
        from test_oracle_w4a8_pins import decode
        xc, xs = oracle_lib.mxfp8_quantize(bits_to_f32(d["x"]))
        ref_q = _relu2_textbook(v13, v2, decode(xc, xs), d["ids"], d["w"])
        got = oracle_lib.forward_w4a8(fmt, d, quant_act=False)
        assert np.abs(got - ref_q).max() <= 1e-6 * np.abs(ref_q).max()
