"""GPU parity of the grouped (prefill) path: routes grouped by expert, FC1 and
FC2 as grouped GEMMs on the matrix cores, per-token combine.  Compared with
the CPU oracle on the same seeded inputs, to the same bar as the decode path
(cosine >= 0.99995, max-abs beyond bf16 rounding <= 2e-2 * RMS), plus exact
properties: a token's output does not depend on the other tokens of the
batch, and repeated calls are bit-identical."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_gather_amd import moe, synth
from gpu_util import compare, make_layer, run_layer, say, to_dev
from pins_util import random_case

pytestmark = pytest.mark.gpu

GROUPED = moe.Tuning(0, 0, 0, moe.PATH_GROUPED)


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    yield


def _skew(rng, ids, E, hot, frac):
    """Send about `frac` of the routes to expert `hot` (ids stay distinct
    within a token where k allows)."""
    M, k = ids.shape
    for t in range(M):
        if rng.random() < frac and hot not in ids[t]:
            ids[t, rng.integers(0, k)] = hot
    return ids


CASES = [
    # fmt, E, H, I, M, k, seed, hot-expert fraction
    ("mxfp4", 4, 64, 32, 1, 1, 1, 0.0),       # one route; FC1 and FC2 second tiles absent
    ("mxfp4", 6, 96, 64, 3, 3, 2, 0.0),       # odd K steps in FC1; FC2 tile half padding
    # NVFP4 with 16 to 128 routes per expert: 128-row FC1 tiles, 32-row FC2 tiles (one pass)
    ("nvfp4", 5, 256, 96, 40, 4, 3, 0.0),     # I = 3 units: partial FC1 column block, odd FC2 K
    ("nvfp4", 8, 512, 128, 300, 2, 4, 0.5),   # 2 m-tiles for the hot expert
    ("mxfp4", 16, 1024, 256, 520, 4, 5, 0.9), # hot expert: 4 full m-tiles + a ragged one
    ("nvfp4", 12, 2560, 64, 200, 2, 6, 0.0),
    ("mxfp4", 3, 1536, 544, 100, 2, 7, 0.0),  # 17 FC1 tiles: last column block half empty
    ("mxfp4", 1, 64, 32, 130, 1, 8, 0.0),     # a single expert, 128 + 2 rows
    # MXFP4 with 16 to 64 routes per expert: 32-row FC1 tiles, 128-row FC2 tiles
    ("mxfp4", 8, 512, 128, 100, 4, 12, 0.5),  # hot expert: 7 FC1 tiles, 2 FC2 tiles
    # past 4096 routes (routing in several workgroups) with a tile table per GEMM
    ("mxfp4", 128, 256, 64, 1100, 4, 13, 0.0),  # 34 routes per expert
    ("nvfp4", 64, 256, 64, 1200, 4, 14, 0.3),   # 75 per expert, a hot one
    # few routes per expert (at most 16 on average): 32-row m-tiles
    ("mxfp4", 64, 512, 128, 100, 4, 9, 0.9),  # hot expert: three 32-row tiles and a ragged one
    ("nvfp4", 40, 512, 96, 120, 4, 10, 0.6),  # I = 3 units: odd FC2 K; hot expert over several tiles
    ("mxfp4", 256, 1024, 64, 60, 8, 11, 0.0), # 480 routes over 256 experts, 1-2 rows each
]


@pytest.mark.parametrize("fmt,E,H,I,M,k,seed,hot", CASES)
def test_grouped_small_shapes(fmt, E, H, I, M, k, seed, hot):
    rng = np.random.default_rng(100 + seed)
    d, _, _ = random_case(rng, fmt, E, H, I, M, k)
    if hot:
        _skew(rng, d["ids"], E, E // 2, hot)
    flat = d["ids"].reshape(-1)
    if flat.size > 2:
        flat[1] = -1                 # an invalid route
        flat[-1] = E + seed          # another, past the last expert
    if M > 1 and k > 1:
        d["ids"][1, 1] = d["ids"][1, 0]  # a duplicate within a token
    acc, _ = oracle.forward_f32(fmt, d)
    layer = make_layer(fmt, d, k, M)
    label = f"{fmt} E{E} H{H} I{I} M{M} k{k}"
    got = run_layer(layer, d, tuning=GROUPED)
    compare(got, acc, label + " grouped")
    # the automatic choice gives the same bits when it picks the grouped path
    if moe.plan(layer.desc, M).path == moe.PATH_GROUPED:
        assert np.array_equal(run_layer(layer, d), got)
        assert np.array_equal(run_layer(layer, d, ids_dtype=torch.int64), got), "int64 ids"
    # repeated calls are bit-identical
    assert np.array_equal(run_layer(layer, d, tuning=GROUPED), got)


def test_grouped_token_outputs_do_not_depend_on_the_batch():
    """Each token's output is a function of its own x, ids and w only: the
    full batch equals the same tokens run one by one (bit-exact), and
    reversing the batch reverses the output."""
    rng = np.random.default_rng(31)
    fmt, E, H, I, M, k = "nvfp4", 8, 512, 192, 200, 4
    d, _, _ = random_case(rng, fmt, E, H, I, M, k)
    _skew(rng, d["ids"], E, 2, 0.7)
    d["ids"][5, 0] = -7
    layer = make_layer(fmt, d, k, M)
    full = run_layer(layer, d, tuning=GROUPED)
    for t in (0, 5, 77, M - 1):
        one = dict(d, x=d["x"][t:t + 1], ids=d["ids"][t:t + 1], w=d["w"][t:t + 1])
        assert np.array_equal(run_layer(layer, one, tuning=GROUPED)[0], full[t]), f"token {t}"
    rev = dict(d, x=d["x"][::-1].copy(), ids=d["ids"][::-1].copy(), w=d["w"][::-1].copy())
    assert np.array_equal(run_layer(layer, rev, tuning=GROUPED), full[::-1])


def test_grouped_invalid_ids_with_nan_poisoned_expert_zero():
    for fmt, poison in (("mxfp4", 0xFF), ("nvfp4", 0x7F)):
        rng = np.random.default_rng(32)
        M = 112  # past the decode path's automatic range (6 chunks of 16 tokens)
        d, _, _ = random_case(rng, fmt, 6, 512, 64, M, 4)
        d["ids"][:] = rng.integers(1, 6, size=(M, 4))
        d["w13_scales"][0] = poison
        d["w2_scales"][0] = poison
        d["ids"][:, 2] = np.resize(np.array([-1, 6, 2**31 - 1, -(2**31)], np.int32), M)
        acc, _ = oracle.forward_f32(fmt, d)
        assert np.isfinite(acc).all()
        layer = make_layer(fmt, d, 4, M)
        assert moe.plan(layer.desc, M).path == moe.PATH_GROUPED
        compare(run_layer(layer, d), acc, f"{fmt} poisoned expert 0, grouped")
        d64 = dict(d)
        d64["ids"] = d["ids"].astype(np.int64)
        d64["ids"][:, 2] = np.resize(np.array([-(2**40), 2**40, 2**62, 6], np.int64), M)
        compare(run_layer(layer, d64, ids_dtype=torch.int64), acc, f"{fmt} int64 out-of-range ids")


def test_grouped_all_invalid_and_poisoned_workspace():
    rng = np.random.default_rng(33)
    d, _, _ = random_case(rng, "nvfp4", 4, 256, 64, 100, 2)   # 100 tokens: the grouped path
    d["ids"][:10] = np.array([-1, 4], np.int32)       # tokens 0..9: no valid route
    layer = make_layer("nvfp4", d, 2, 100)
    assert moe.plan(layer.desc, 100).path == moe.PATH_GROUPED
    acc, _ = oracle.forward_f32("nvfp4", d)
    x = to_dev(d["x"]).view(torch.bfloat16)
    ids, w = to_dev(d["ids"]), to_dev(d["w"])
    outs = []
    for rep in range(2):
        layer.workspace.fill_(0xFF)
        out = torch.full((100, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
        layer(x, ids, w, out=out)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu().numpy().view(np.uint16))
    assert not outs[0][:10].any(), "tokens without a valid route must give +0"
    compare(outs[0], acc, "poisoned workspace, grouped")
    assert np.array_equal(outs[0], outs[1])
    # every route invalid
    d["ids"][:] = -1
    out = torch.full((100, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer(x, to_dev(d["ids"]), w, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), torch.zeros_like(out.view(torch.int16)))


def test_grouped_phases_split():
    rng = np.random.default_rng(34)
    d, _, _ = random_case(rng, "mxfp4", 8, 256, 128, 64, 2)
    layer = make_layer("mxfp4", d, 2, 64)
    whole = run_layer(layer, d, tuning=GROUPED)
    x = to_dev(d["x"]).view(torch.bfloat16)
    ids, w = to_dev(d["ids"]), to_dev(d["w"])
    out = torch.empty_like(x)
    layer(x, ids, w, out=out, tuning=GROUPED, phases=1)
    layer(x, ids, w, out=out, tuning=GROUPED, phases=2)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), whole)
    # routing alone and combine alone repeat their part: the result stays the same
    out.fill_(float("nan"))
    for ph in (4, 1, 2, 8):
        layer(x, ids, w, out=out, tuning=GROUPED, phases=ph)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), whole)


def test_grouped_graph_replay_with_changing_routes():
    rng = np.random.default_rng(35)
    fmt, E, H, I, M, k = "mxfp4", 16, 512, 256, 96, 4
    d, _, _ = random_case(rng, fmt, E, H, I, M, k)
    layer = make_layer(fmt, d, k, M)
    x = to_dev(d["x"]).view(torch.bfloat16)
    ids, w = to_dev(d["ids"]), to_dev(d["w"])
    out = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(x, ids, w, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, ids, w, out=out)
    for rep in range(3):
        new_ids = rng.integers(-2, E + 2, size=(M, k)).astype(np.int32)
        new_w = rng.random((M, k)).astype(np.float32)
        ids.copy_(torch.from_numpy(new_ids))
        w.copy_(torch.from_numpy(new_w))
        g.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(out)
        layer(x, ids, w, out=eager)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        acc, _ = oracle.forward_f32(fmt, dict(d, ids=new_ids, w=new_w))
        compare(out.view(torch.int16).cpu().numpy().view(np.uint16), acc, f"replay {rep}")


def test_prefill_workload_full_size_sampled():
    """The E128/H4096/I1536 prefill with 4096 tokens, top-8, run whole on the
    GPU; the oracle checks a sample of tokens (each token's output depends
    only on its own inputs, which the batch-independence test pins)."""
    wl = synth.WORKLOADS["mxfp4_prefill_e128"]
    say("  generate mxfp4_prefill_e128")
    d = synth.generate(wl)
    layer = make_layer(wl.fmt, d, wl.k, wl.M)
    say("  run")
    got = run_layer(layer, d)
    assert np.array_equal(run_layer(layer, d), got), "not bit-reproducible"
    rng = np.random.default_rng(36)
    sample = np.unique(np.concatenate([[0, 1, wl.M - 1], rng.integers(0, wl.M, 5)]))
    sub = dict(d, x=d["x"][sample], ids=d["ids"][sample], w=d["w"][sample])
    say(f"  oracle on tokens {sample.tolist()}")
    acc, _ = oracle.forward_f32(wl.fmt, sub)
    compare(got[sample], acc, f"{wl.name} sampled")
    # expert load of this routing: every expert holds rows, several m-tiles each
    counts = np.bincount(d["ids"].ravel(), minlength=wl.E)
    say(f"  rows per expert: min {counts.min()} mean {counts.mean():.0f} max {counts.max()}")


@pytest.mark.parametrize("fmt,k", [("mxfp4", 4), ("nvfp4", 8)])
def test_band_edge_both_paths(fmt, k):
    """Around the edges of one decode launch pair (M = min(16, 64/k)) and of
    the decode path's automatic range (6 such chunks), the automatic path,
    the forced decode path (in chunks past one) and the forced grouped path
    all match the oracle."""
    edge = min(16, 64 // k)
    for E, M in ((16, edge), (16, edge + 1), (16, 2 * edge + 1), (256, 3 * edge), (256, 6 * edge),
                 (256, 6 * edge + 1)):
        rng = np.random.default_rng(40 + M + E)
        d, _, _ = random_case(rng, fmt, E, 256, 128, M, k)
        d["ids"][0, 0] = -1
        d["ids"][-1, -1] = E + 3
        acc, _ = oracle.forward_f32(fmt, d)
        layer = make_layer(fmt, d, k, M)
        # up to 2 chunks: decode; up to 6 chunks with fewer route slots than E: decode; else grouped
        few = -(-M // edge) * edge * k < E
        want = moe.PATH_DECODE if M <= 2 * edge or (M <= 6 * edge and few) else moe.PATH_GROUPED
        assert moe.plan(layer.desc, M).path == want
        compare(run_layer(layer, d), acc, f"{fmt} E{E} k{k} M{M} auto")
        compare(run_layer(layer, d, tuning=GROUPED), acc, f"{fmt} E{E} k{k} M{M} grouped")
        compare(run_layer(layer, d, tuning=moe.Tuning(0, 0, 0, moe.PATH_DECODE)), acc, f"{fmt} E{E} k{k} M{M} decode")


def test_grouped_nvfp4_decode_geometry_many_tokens():
    """The E512/H2560/I320 NVFP4 geometry (64 of its experts) at 512 tokens,
    top-10: E4M3 scales and globals through the grouped GEMMs, checked on a
    sample of tokens."""
    wl = synth.WORKLOADS["nvfp4_decode_e512"].replace(E=64, M=512)
    d = synth.generate(wl)
    layer = make_layer(wl.fmt, d, wl.k, wl.M)
    got = run_layer(layer, d)
    sample = np.array([0, 1, 100, 257, 511])
    acc, _ = oracle.forward_f32(wl.fmt, dict(d, x=d["x"][sample], ids=d["ids"][sample], w=d["w"][sample]))
    compare(got[sample], acc, "nvfp4 E64/H2560/I320 M512 k10 sampled")


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_grouped_at_the_route_limit(act):
    """Exactly 2^22 routes (2^20 tokens, top-4), the most the grouped path
    takes: grouped-row indexes and workspace offsets at their largest.
    Sampled tokens against the oracle, including the last one."""
    rng = np.random.default_rng(37)
    E, H, I, M, k = 16, 64, 32, 1 << 20, 4
    d, _, _ = random_case(rng, "mxfp4", E, H, I, 8, k)   # weights; tokens drawn below
    d["x"] = rng.integers(0, 1 << 16, size=(M, H), dtype=np.uint16)
    d["x"][(d["x"] & 0x7F80) == 0x7F80] = 0x3F80           # no Inf/NaN bit patterns
    d["x"] = (d["x"] & 0x3FFF) | (d["x"] & 0x8000)         # |x| < 2
    d["ids"] = rng.integers(-1, E, size=(M, k)).astype(np.int32)
    d["w"] = rng.random((M, k)).astype(np.float32)
    layer = make_layer("mxfp4", d, k, M, act=act)
    got = run_layer(layer, d)
    sample = np.array([0, 1, 777777, M - 2, M - 1])
    sub = dict(d, x=d["x"][sample], ids=d["ids"][sample], w=d["w"][sample])
    if act == "bf16":
        compare(got[sample], oracle.forward_f32("mxfp4", sub)[0], "2^22 routes, bf16")
    else:
        from gpu_util import W4A8_MAXABS_REL_RMS
        compare(got[sample], oracle.forward_w4a8("mxfp4", sub), "2^22 routes, mxfp8", bar=W4A8_MAXABS_REL_RMS)


def test_grouped_with_8192_experts():
    """The most experts the grouping's LDS histogram holds, with routes
    spread over all of them (most experts get one or two rows)."""
    rng = np.random.default_rng(38)
    E, H, I, M, k = 8192, 64, 32, 2048, 8
    d, _, _ = random_case(rng, "nvfp4", E, H, I, M, k)
    d["ids"][:, 0] = np.arange(M) % E                 # experts 0 and 8191 both used
    d["ids"][-1, -1] = E - 1
    layer = make_layer("nvfp4", d, k, M)
    got = run_layer(layer, d)
    sample = np.array([0, 5, 1000, M - 1])
    acc, _ = oracle.forward_f32("nvfp4", dict(d, x=d["x"][sample], ids=d["ids"][sample], w=d["w"][sample]))
    compare(got[sample], acc, "E8192 grouped")
