"""Guard bands: every buffer the library writes (the output, the workspace,
the quantiser's codes and scales) sits inside a larger allocation whose
bytes before and after are filled with a pattern; after the call the bands
must be untouched.  An out-of-bounds write on the GPU shows up here even
without a device-side sanitizer."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_scaled_fp4_gather_amd import moe
from gpu_util import make_layer, say, to_dev
from pins_util import bf16_bits, random_case

pytestmark = pytest.mark.gpu

BAND = 4096  # bytes of guard on each side (a multiple of 256 keeps alignment)


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    yield


def _banded(nbytes, fill):
    big = torch.full((BAND + nbytes + BAND,), fill, dtype=torch.uint8, device="cuda")
    return big, big[BAND:BAND + nbytes]


def _bands_intact(big, nbytes, fill):
    torch.cuda.synchronize()
    lo, hi = big[:BAND], big[BAND + nbytes:]
    return bool((lo == fill).all()) and bool((hi == fill).all())


@pytest.mark.parametrize("fmt,act,M", [("mxfp4", "bf16", 2), ("nvfp4", "bf16", 3), ("mxfp4", "bf16", 300),
                                       ("nvfp4", "bf16", 130), ("mxfp4", "mxfp8", 300), ("mxfp4", "mxfp8", 37),
                                       ("nvfp4", "bf16", 40), ("mxfp4", "bf16", 96)])
def test_layer_writes_stay_inside_out_and_workspace(fmt, act, M):
    rng = np.random.default_rng(70 + M)
    E, H, I, k = 12, 288, 96, 4
    d, _, _ = random_case(rng, fmt, E, H, I, M, k)
    d["ids"][0, 0] = -1
    layer = make_layer(fmt, d, k, M, act=act)
    ws_n = moe.workspace_bytes(layer.desc, M)
    wbig, ws = _banded(ws_n, 0xA5)
    obig, ob = _banded(M * H * 2, 0x5A)
    out = ob.view(torch.bfloat16).view(M, H)
    x = to_dev(d["x"]).view(torch.bfloat16)
    ids, w = to_dev(d["ids"]), to_dev(d["w"])
    # the automatic path, then the grouped and the decode path forced (the
    # decode path in chunks of 16 tokens past M = 16)
    for tuning in (None, moe.Tuning(0, 0, 0, moe.PATH_GROUPED), moe.Tuning(0, 0, 0, moe.PATH_DECODE)):
        moe.forward(layer.desc, layer.prepared, x, ids, w, out, ws, tuning=tuning)
        assert _bands_intact(wbig, ws_n, 0xA5), f"{fmt} {act} M{M}: write outside the workspace"
        assert _bands_intact(obig, M * H * 2, 0x5A), f"{fmt} {act} M{M}: write outside the output"
        assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (300, 4096)])
def test_quantiser_writes_stay_inside_codes_and_scales(rows, cols):
    rng = np.random.default_rng(rows + cols)
    x = to_dev(bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))).view(torch.bfloat16)
    cbig, cb = _banded(rows * cols, 0x3C)
    sbig, sb = _banded(rows * (cols // 32), 0xC3)
    moe.mxfp8_quantize(x, cb.view(rows, cols), sb.view(rows, cols // 32))
    assert _bands_intact(cbig, rows * cols, 0x3C)
    assert _bands_intact(sbig, rows * (cols // 32), 0xC3)
