"""NaN propagation on the bf16 paths (decode and grouped), as the interface
promises: a NaN in a token's x makes that token's whole output row NaN; a
NaN block scale in one row of a routed expert's W2 makes that output column
NaN for the tokens routed there; everything else stays finite and matches
the oracle.  NaN positions are compared exactly."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from block_scaled_fp4_gather_amd import moe
from gpu_util import compare, make_layer, run_layer, say
from pins_util import random_case

pytestmark = pytest.mark.gpu

GROUPED = moe.Tuning(0, 0, 0, moe.PATH_GROUPED)


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    yield


@pytest.mark.parametrize("fmt,nan_scale", [("mxfp4", 0xFF), ("nvfp4", 0x7F)])
@pytest.mark.parametrize("M", [3, 60])
def test_nan_propagates(fmt, nan_scale, M):
    rng = np.random.default_rng(50 + M)
    E, H, I, k = 8, 256, 96, 4
    d, _, _ = random_case(rng, fmt, E, H, I, M, k)
    d["ids"][:] = rng.integers(1, E, size=(M, k))
    d["ids"][M - 1, 0] = 0                     # only the last token routes to expert 0
    d["x"][1, 7] = 0x7FC0                      # NaN in token 1's x
    d["w2_scales"][0, 5, 0] = nan_scale        # NaN scale: expert 0, W2 row (output column) 5
    acc, _ = oracle.forward_f32(fmt, d)
    want_nan = np.isnan(acc)
    assert want_nan[1].all() and want_nan[M - 1, 5] and want_nan.sum() == H + 1 - (M - 1 == 1)
    layer = make_layer(fmt, d, k, M)
    for label, tuning in (("auto", None), ("grouped", GROUPED), ("decode", moe.Tuning(0, 0, 0, moe.PATH_DECODE))):
        got = run_layer(layer, d, tuning=tuning)
        g = oracle.bf16_bits_to_f32(got)
        assert np.array_equal(np.isnan(g), want_nan), f"{fmt} M{M} {label}: NaN positions"
        keep = ~want_nan.any(axis=1)
        compare(got[keep], acc[keep], f"{fmt} M{M} {label}, finite tokens")
        # the poisoned token's other columns stay finite
        cols = np.arange(H) != 5
        assert np.isfinite(g[M - 1, cols]).all()
