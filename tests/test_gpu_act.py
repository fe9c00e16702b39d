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
        compare(run_layer(layer, d, tuning=GROUPED), acc, label + " grouped")
        # the decode path forced (M = 70: five chunks of 16 tokens)
        compare(run_layer(layer, d, tuning=moe.Tuning(0, 0, 0, moe.PATH_DECODE)), acc, label + " decode")


@pytest.mark.parametrize("fn,alpha,beta,limit", FNS)
def test_activation_w4a8(fn, alpha, beta, limit):
    d = _case(400 + len(fn), "mxfp4", 10, 448, 224, 150, 4, fn, alpha, beta, limit)
    layer = _layer("mxfp4", d, 4, 150, act="mxfp8")
    compare(run_layer(layer, d), oracle.forward_w4a8("mxfp4", d), f"w4a8 {fn}", bar=W4A8_MAXABS_REL_RMS)


def _relu2_case(seed, fmt, E, H, I, M, k):
    from pins_util import bf16_bits, make_matrix
    rng = np.random.default_rng(seed)
    c13, s13, _ = make_matrix(rng, fmt, (E, I), H, 1.0 / 512)
    c2, s2, _ = make_matrix(rng, fmt, (E, H), I, 1.0 / 512)
    d = dict(w13_codes=c13, w13_scales=s13, w2_codes=c2, w2_scales=s2,
             x=bf16_bits(rng.standard_normal((M, H)).astype(np.float32)),
             ids=rng.integers(0, E, size=(M, k)).astype(np.int32), w=rng.random((M, k)).astype(np.float32),
             g13=np.full(E, 1.0 / 512, np.float32) if fmt == "nvfp4" else None,
             g2=np.full(E, 1.0 / 512, np.float32) if fmt == "nvfp4" else None,
             fn="relu2", alpha=0.0, beta=0.0, limit=0.0)
    d["ids"].reshape(-1)[1 % d["ids"].size] = -1
    return d


def _relu2_layer(fmt, d, k, M, act="bf16"):
    E, I, Hh = d["w13_codes"].shape
    desc = moe.Desc(fmt, E, 2 * Hh, I, k, M, act, "relu2")
    from gpu_util import to_dev
    return moe.Fp4MoE(desc, to_dev(d["w13_codes"]), to_dev(d["w13_scales"]), to_dev(d["w2_codes"]),
                      to_dev(d["w2_scales"]), to_dev(d.get("g13")), to_dev(d.get("g2")))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_relu2_decode_and_grouped(fmt):
    for M, k in ((1, 8), (4, 4), (70, 4)):
        d = _relu2_case(500 + M, fmt, 12, 512, 192, M, k)
        acc, _ = oracle.forward_f32(fmt, d)
        layer = _relu2_layer(fmt, d, k, M)
        compare(run_layer(layer, d), acc, f"{fmt} relu2 M{M} k{k} auto")
        if M <= 16:
            compare(run_layer(layer, d, tuning=GROUPED), acc, f"{fmt} relu2 M{M} k{k} grouped")


def test_relu2_w4a8_and_prepare_round_trip():
    import torch
    d = _relu2_case(600, "mxfp4", 10, 448, 256, 150, 4)
    layer = _relu2_layer("mxfp4", d, 4, 150, act="mxfp8")
    compare(run_layer(layer, d), oracle.forward_w4a8("mxfp4", d), "w4a8 relu2", bar=W4A8_MAXABS_REL_RMS)
    # the prepared buffer holds exactly the I-row W13 and comes back unchanged
    from gpu_util import to_dev
    src = [to_dev(d[kk]) for kk in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")]
    back = [torch.full_like(t, 0x5C) for t in src]
    moe.unprepare(layer.desc, layer.prepared, *back, None, None)
    torch.cuda.synchronize()
    for a, b in zip(src, back):
        assert torch.equal(a, b)
    # and dequantises to the oracle's values
    out = torch.empty((256, 448), dtype=torch.float32, device="cuda")
    moe.dequant_export(layer.desc, layer.prepared, 3, 0, out)
    torch.cuda.synchronize()
    want = oracle.dequant("mxfp4", d["w13_codes"][3], d["w13_scales"][3])
    assert np.array_equal(out.cpu().numpy(), want)


def test_activations_at_full_sizes_sampled():
    """Each activation on a full-size geometry: gelu_tanh on the E512/H2560/I320
    NVFP4 decode layer (M = 1, top-10), swigluoai on the H7168/I256 MXFP4
    shard at 96 tokens through both grouped paths, checked on sampled tokens."""
    from block_scaled_fp4_gather_amd import synth
    wl = synth.WORKLOADS["nvfp4_decode_e512"]
    d = synth.generate(wl)
    d.update(fn="gelu_tanh", alpha=0.0, beta=0.0, limit=0.0)
    acc, _ = oracle.forward_f32(wl.fmt, d)
    layer = _layer(wl.fmt, d, wl.k, wl.M)
    compare(run_layer(layer, d), acc, "E512 NVFP4 decode, gelu_tanh")
    wl = synth.WORKLOADS["mxfp4_shard_e256_m4"].replace(M=96)
    d = synth.generate(wl)
    d.update(fn="swigluoai", alpha=1.702, beta=1.0, limit=7.0)
    sample = np.array([0, 17, 95])
    sub = dict(d, x=d["x"][sample], ids=d["ids"][sample], w=d["w"][sample])
    for act in ("bf16", "mxfp8"):
        layer = _layer(wl.fmt, d, wl.k, wl.M, act=act)
        got = run_layer(layer, d)[sample]
        if act == "bf16":
            compare(got, oracle.forward_f32(wl.fmt, sub)[0], "H7168/I256 M96 swigluoai, grouped bf16")
        else:
            compare(got, oracle.forward_w4a8(wl.fmt, sub), "H7168/I256 M96 swigluoai, grouped mxfp8",
                    bar=W4A8_MAXABS_REL_RMS)
