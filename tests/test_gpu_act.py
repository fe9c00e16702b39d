"""GPU parity of the gated activations (gelu_tanh, swigluoai) on every path:
decode, grouped with bf16 activations and grouped with MXFP8 activations,
each against the oracle with the same activation, to that path's bar."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from block_scaled_fp4_gather_amd import moe
from gpu_util import W4A8_MAXABS_REL_RMS, compare, make_layer, run_layer, say
from pins_util import random_case

pytestmark = pytest.mark.gpu

GROUPED = moe.Tuning(0, 0, 0, moe.PATH_GROUPED)
FNS = [("gelu_tanh", 0.0, 0.0, 0.0), ("swigluoai", 1.702, 1.0, 7.0), ("swigluoai", 1.0, 0.5, 0.75)]


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    yield


def _case(seed, fmt, E, H, I, M, k, fn, alpha, beta, limit):
    rng = np.random.default_rng(seed)
    d, _, _ = random_case(rng, fmt, E, H, I, M, k)
    d.update(fn=fn, alpha=alpha, beta=beta, limit=limit)
    d["ids"].reshape(-1)[1 % d["ids"].size] = -1
    return d


def _layer(fmt, d, k, M, act="bf16"):
    E, twoI, Hh = d["w13_codes"].shape
    desc = moe.Desc(fmt, E, 2 * Hh, twoI // 2, k, M, act, d["fn"], d["alpha"], d["beta"], d["limit"])
    from gpu_util import to_dev
    return moe.Fp4MoE(desc, to_dev(d["w13_codes"]), to_dev(d["w13_scales"]), to_dev(d["w2_codes"]),
                      to_dev(d["w2_scales"]), to_dev(d.get("g13")), to_dev(d.get("g2")))


@pytest.mark.parametrize("fn,alpha,beta,limit", FNS)
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_activation_decode_and_grouped(fmt, fn, alpha, beta, limit):
    for M, k in ((1, 8), (4, 4), (70, 4)):
        d = _case(300 + M + len(fn), fmt, 12, 512, 160, M, k, fn, alpha, beta, limit)
        acc, _ = oracle.forward_f32(fmt, d)
        layer = _layer(fmt, d, k, M)
        label = f"{fmt} {fn}({alpha},{beta},{limit}) M{M} k{k}"
        compare(run_layer(layer, d), acc, label + " auto")
        if M <= 16:
            compare(run_layer(layer, d, tuning=GROUPED), acc, label + " grouped")


@pytest.mark.parametrize("fn,alpha,beta,limit", FNS)
def test_activation_w4a8(fn, alpha, beta, limit):
    d = _case(400 + len(fn), "mxfp4", 10, 448, 224, 150, 4, fn, alpha, beta, limit)
    layer = _layer("mxfp4", d, 4, 150, act="mxfp8")
    compare(run_layer(layer, d), oracle.forward_w4a8("mxfp4", d), f"w4a8 {fn}", maxabs=W4A8_MAXABS_REL_RMS)
