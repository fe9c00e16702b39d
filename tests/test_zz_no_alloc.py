"""The entry point for callers that cannot allocate (moe_fp4_forward_noalloc,
the library's own workspace) against moe_fp4_forward with a caller's
workspace: two calls in a row, the second with fewer tokens, on both
paths; bit-identical outputs, and each within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_gather_amd import moe, synth
from gpu_util import compare, make_layer, say, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(layer, d):
    x = to_dev(d["x"]).view(torch.bfloat16)
    ids = torch.from_numpy(np.ascontiguousarray(d["ids"])).to(torch.int32).cuda()
    w = to_dev(d["w"])
    out = torch.full((x.shape[0], x.shape[1]), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.forward_noalloc(layer.desc, layer.prepared, x, ids, w, out)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def _with_workspace(layer, d):
    x = to_dev(d["x"]).view(torch.bfloat16)
    ids = torch.from_numpy(np.ascontiguousarray(d["ids"])).to(torch.int32).cuda()
    w = to_dev(d["w"])
    layer.workspace.fill_(0xFF)
    out = layer(x, ids, w)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,M1,M2", [("tiny_mxfp4", 5, 2),        # decode path
                                        ("tiny_mxfp4", 120, 40),     # grouped path, then a smaller call
                                        ("nvfp4_decode_e512", 3, 1),
                                        ("mxfp4_shard_e256_m1", 2, 1)])
def test_noalloc_matches_forward(name, M1, M2):
    wl = synth.WORKLOADS[name].replace(M=M1)
    d = synth.generate(wl)
    d["ids"].reshape(-1)[1] = -1  # an invalid route
    layer = make_layer(wl.fmt, d, wl.k, M1)
    assert moe.workspace_bytes(layer.desc, M1) <= 64 << 20
    for M in (M1, M2):
        dm = dict(d, x=d["x"][:M], ids=d["ids"][:M], w=d["w"][:M])
        say(f"  {name} M={M} path {moe.plan(layer.desc, M).path}")
        got = _noalloc(layer, dm)
        ref = _with_workspace(layer, dm)
        assert np.array_equal(got, ref), f"{name} M={M}: differs from moe_fp4_forward"
        acc, _ = oracle.forward_f32(wl.fmt, dm)
        compare(got, acc, f"{name} M={M} noalloc")
