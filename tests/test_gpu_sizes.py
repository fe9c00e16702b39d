"""One layer called at many token counts from 1 to 1024, in an order that
puts small calls after large ones, on both activation formats: each call
runs eager and as a captured graph replayed twice, with the workspace and
the output poisoned (0xFF bytes, NaN) before every run; replays are
bit-identical to the eager call, sampled tokens match the oracle, and the
inputs (x, ids, weights, prepared buffer) are unchanged afterwards."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import W4A8_MAXABS_REL_RMS, compare, make_layer, say, to_dev
from pins_util import bf16_bits, random_case

pytestmark = pytest.mark.gpu

SIZES = [1, 2, 3, 7, 16, 17, 64, 255, 1024, 1, 300, 2]


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    yield


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_sizes_eager_and_graph_with_poison(act):
    rng = np.random.default_rng(60)
    E, H, I, k, cap = 16, 256, 128, 4, 1024
    d, _, _ = random_case(rng, "mxfp4", E, H, I, 1, k)
    layer = make_layer("mxfp4", d, k, cap, act=act)
    prep0 = layer.prepared.clone()
    for it, M in enumerate(SIZES):
        x_bits = bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
        ids_np = rng.integers(-1, E + 1, size=(M, k)).astype(np.int32)
        w_np = rng.random((M, k)).astype(np.float32)
        x = to_dev(x_bits).view(torch.bfloat16)
        ids, w = to_dev(ids_np), to_dev(w_np)
        snap = [t.clone() for t in (x, ids, w)]
        out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")

        def poison():
            layer.workspace.fill_(0xFF)
            out.fill_(float("nan"))

        poison()
        layer(x, ids, w, out=out)
        torch.cuda.synchronize()
        eager = out.view(torch.int16).clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            layer(x, ids, w, out=out)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer(x, ids, w, out=out)
        for rep in range(2):
            poison()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager), f"{act} M{M}: replay {rep} differs from eager"
        for a, b in zip(snap, (x, ids, w)):
            assert torch.equal(a, b), f"{act} M{M}: an input was written"
        sample = np.unique(np.array([0, M // 2, M - 1]))
        sub = dict(d, x=x_bits[sample], ids=ids_np[sample], w=w_np[sample])
        got = eager.cpu().numpy().view(np.uint16)[sample]
        grouped = M > min(16, 64 // k)
        if act == "mxfp8" and grouped:
            compare(got, oracle.forward_w4a8("mxfp4", sub), f"{act} M{M}", bar=W4A8_MAXABS_REL_RMS)
        else:
            compare(got, oracle.forward_f32("mxfp4", sub)[0], f"{act} M{M}")
        del g
    assert torch.equal(layer.prepared, prep0), "the prepared buffer was written"
