"""The compressed scale format (CSF; b12x PR #459, "Reduce NVFP4-CSF scale
reconstruction overhead", commit messages: one-bit MXFP4 and four-bit NVFP4
offsets from a row base byte) on the GPU: the CSF blocks that preparation
writes equal the oracle's encoding byte for byte (unpacked by the layout's
documented order); dequantisation from them is bit-exact; and the layer's
output is bit-identical to the same layer with plain scales, and within the
parity bar of the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_gather_amd import moe, synth
from gpu_util import compare, run_layer, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    yield


def _csf_weights(fmt, E, H, I, seed):
    """Weights whose scales mostly fit the format, with exception rows (1 in
    64, plus rows made to span too far), a row whose bytes are all 255, and a
    compressible row holding 255 (MXFP4: 254/255; NVFP4: 0x70/0x7F)."""
    wl = synth.Workload("csf_case", fmt, E, H, I, 1, 1, seed, scales="csf")
    d = synth.weights(wl)
    s13, s2 = d["w13_scales"], d["w2_scales"]
    s13[0, 3, :] = 255
    s13[0, 5, 0] = s13[0, 5].min() + (3 if fmt == "mxfp4" else 20)
    if fmt == "mxfp4":
        s2[-1, 1, :] = 254
        s2[-1, 1, 0] = 255
    else:
        s2[-1, 1, :] = 0x70
        s2[-1, 1, 0] = 0x7F
    return wl, d


def _desc(fmt, E, H, I, k, M, scales):
    return moe.Desc(fmt, E, H, I, k, M, scales=scales)


def _prepare(desc, d):
    prep = torch.full((moe.prepared_bytes(desc),), 0xAB, dtype=torch.uint8, device="cuda")
    moe.prepare(desc, *[to_dev(d[k]) for k in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")],
                to_dev(d.get("g13")), to_dev(d.get("g2")), prep)
    torch.cuda.synchronize()
    return prep


def _block_offsets(fmt, E, H, I):
    """Byte offsets (in the prepared buffer) of every tile's CSF block, and
    each tile's logical rows per lane, from the documented layout: globals
    header (NVFP4), then per expert [FC1 tiles][FC2 tiles]; a tile is nC
    KiB of codes, nQ 256-byte scale words, then the CSF block."""
    G = 32 if fmt == "mxfp4" else 16
    nC1, nC2 = H // 32, I // 32
    nQ1, nQ2 = -(-(H // G) // 4), -(-(I // G) // 4)

    def block(nC):  # one 256-byte group of 64 words per 24 (MXFP4) or 3 (NVFP4) chunks
        return 256 * -(-nC // (24 if fmt == "mxfp4" else 3))
    t1 = nC1 * 1024 + nQ1 * 256 + block(nC1)
    t2 = nC2 * 1024 + nQ2 * 256 + block(nC2)
    nB1, nB2 = I // 32, -(-H // 64)
    expert = -(-(t1 * nB1 + t2 * nB2) // 256) * 256
    glob = -(-8 * E // 256) * 256 if fmt == "nvfp4" else 0
    out = []
    for e in range(E):
        for b in range(nB1):
            rows = [32 * b + l if l < 32 else I + 32 * b + l - 32 for l in range(64)]
            out.append((e, "w13", glob + e * expert + b * t1 + nC1 * 1024 + nQ1 * 256, nC1, rows))
        for hb in range(nB2):
            rows = [64 * hb + l for l in range(64)]
            out.append((e, "w2", glob + e * expert + nB1 * t1 + hb * t2 + nC2 * 1024 + nQ2 * 256, nC2, rows))
    return out


def _unpack(fmt, buf, at, nC, lane):
    """A row's base byte and offsets from the documented word layout: one word
    per group of 24 (MXFP4) or 3 (NVFP4) chunks, byte 0 the base (the same
    in every word of the row), then bit 8+j (MXFP4) or byte 1+j (NVFP4)."""
    cw = 24 if fmt == "mxfp4" else 3
    words = [int.from_bytes(bytes(buf[at + 256 * g + 4 * lane: at + 256 * g + 4 * lane + 4]), "little")
             for g in range(-(-nC // cw))]
    bases = {w & 0xFF for w in words}
    assert len(bases) == 1
    off = []
    for c in range(nC):
        w = words[c // cw]
        if fmt == "mxfp4":
            off.append((w >> (8 + c % cw)) & 1)
        else:
            b = (w >> (8 + 8 * (c % cw))) & 0xFF
            off += [b & 15, b >> 4]
    return bases.pop(), np.array(off, np.uint8)


@pytest.mark.parametrize("fmt,E,H,I", [("mxfp4", 3, 96, 64), ("nvfp4", 3, 96, 64),
                                       ("mxfp4", 2, 1024, 288), ("nvfp4", 2, 2560, 320)])
def test_csf_blocks_equal_the_oracle_encoding(fmt, E, H, I):
    wl, d = _csf_weights(fmt, E, H, I, 31 + H)
    desc = _desc(fmt, E, H, I, 2, 1, "csf")
    buf = _prepare(desc, d).cpu().numpy()
    n_exc = n_rows = 0
    for e, which, at, nC, rows in _block_offsets(fmt, E, H, I):
        sc = d[f"{which}_scales"][e]
        for lane, row in enumerate(rows):
            base, off = _unpack(fmt, buf, at, nC, lane)
            if row >= sc.shape[0]:  # padding rows of the last W2 tile
                assert base == 0 and not off.any()
                continue
            want_base, want_off, comp = oracle.csf_encode(fmt, sc[row])
            assert base == want_base, (e, which, row)
            assert np.array_equal(off, want_off), (e, which, row)
            n_rows += 1
            n_exc += not comp
    say(f"  {n_rows} rows, {n_exc} exceptions")
    assert 0 < n_exc < n_rows
    # the plain scales stay in place: the inverse preparation gives the bytes back
    src = [to_dev(d[k]) for k in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")]
    back = [torch.zeros_like(t) for t in src]
    g = [to_dev(d.get("g13")), to_dev(d.get("g2"))]
    gb = [torch.zeros_like(t) if t is not None else None for t in g]
    moe.unprepare(desc, torch.from_numpy(buf).cuda(), *back, *gb)
    torch.cuda.synchronize()
    for a, b in zip(src, back):
        assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_csf_dequant_export_bit_exact(fmt):
    E, H, I = 3, 512, 160
    wl, d = _csf_weights(fmt, E, H, I, 7)
    desc = _desc(fmt, E, H, I, 2, 1, "csf")
    prep = _prepare(desc, d)
    for e in range(E):
        for which, rows, cols, c, s, gl in ((0, 2 * I, H, "w13_codes", "w13_scales", d.get("g13")),
                                            (1, H, I, "w2_codes", "w2_scales", d.get("g2"))):
            out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
            moe.dequant_export(desc, prep, e, which, out)
            got = out.cpu().numpy()
            want = oracle.dequant(fmt, d[c][e], d[s][e], 1.0 if gl is None else float(gl[e]))
            nan = np.isnan(want)
            assert np.array_equal(np.isnan(got), nan)
            assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _layer(fmt, d, k, M, scales):
    E, twoI, Hh = d["w13_codes"].shape
    desc = _desc(fmt, E, 2 * Hh, twoI // 2, k, M, scales)
    return moe.Fp4MoE(desc, to_dev(d["w13_codes"]), to_dev(d["w13_scales"]), to_dev(d["w2_codes"]),
                      to_dev(d["w2_scales"]), to_dev(d.get("g13")), to_dev(d.get("g2")))


CASES = [
    # fmt, E, H, I, M, k
    ("mxfp4", 6, 96, 64, 3, 3),       # ragged last W2 tile
    ("nvfp4", 5, 256, 96, 2, 4),
    ("mxfp4", 16, 1024, 256, 8, 4),
    ("nvfp4", 12, 2560, 320, 4, 6),   # FC2 in two chunk groups
    ("mxfp4", 4, 512, 544, 2, 2),     # I = 17 chunks: FC2 over two passes
]


@pytest.mark.parametrize("fmt,E,H,I,M,k", CASES)
def test_csf_layer_bit_identical_to_plain(fmt, E, H, I, M, k):
    wl, d = _csf_weights(fmt, E, H, I, 100 + E)
    wl = wl.replace(M=M, k=k)
    d["x"] = synth.activations(wl, 5 + M)
    d["ids"], d["w"] = synth.routing(wl, 5 + M)
    d["ids"].reshape(-1)[1] = -1
    d["ids"][0, 0] = 0  # the expert with the 255 rows, routed by token 0 only
    d["ids"][1:][d["ids"][1:] == 0] = -1
    acc, _ = oracle.forward_f32(fmt, d)
    plain, csf = _layer(fmt, d, k, M, "plain"), _layer(fmt, d, k, M, "csf")
    shapes = [None] + [moe.Tuning(kl1, r1, r2, moe.PATH_DECODE) for kl1 in (4, 8) for r1 in (16, 32)
                       for r2 in (16, 32)]
    for t in shapes:
        if t is not None and t.fc2_rows * (4 if I <= 128 else (8 if I <= 512 else 16)) < 64:
            continue
        try:
            moe.plan(csf.desc, M, t)
        except moe.MoeFp4Error:
            continue  # a shape the compressed scales do not run (tests/test_abi.py)
        got = run_layer(csf, d, tuning=t)
        ref = run_layer(plain, d, tuning=t)
        assert np.array_equal(got, ref), f"{fmt} E{E} H{H} I{I}: csf differs from plain"
        # token 0 routes to the expert with an all-255 (NaN) scale row: NaN
        # where the oracle has NaN, the finite tokens within the bar
        keep = np.isfinite(acc)
        assert not keep[0].any() and keep.any()
        assert np.array_equal(np.isnan(oracle.bf16_bits_to_f32(got)), np.isnan(acc))
        compare(got[keep], acc[keep], f"{fmt} E{E} H{H} I{I} M{M} k{k} csf "
                f"{t and (t.fc1_chunks_per_wave, t.fc1_rows, t.fc2_rows)}, finite values")
    # the grouped path reads the plain scales of the same buffer
    g = run_layer(csf, d, tuning=moe.Tuning(0, 0, 0, moe.PATH_GROUPED))
    assert np.array_equal(g, run_layer(plain, d, tuning=moe.Tuning(0, 0, 0, moe.PATH_GROUPED)))


@pytest.mark.parametrize("name", ["mxfp4_csf_shard_e256_m1", "nvfp4_csf_decode_e512"])
def test_csf_workloads_full_size(name):
    wl = synth.WORKLOADS[name]
    d = synth.generate(wl)
    acc, _ = oracle.forward_f32(wl.fmt, d)
    got = run_layer(_layer(wl.fmt, d, wl.k, wl.M, "csf"), d)
    compare(got, acc, name)
    assert np.array_equal(got, run_layer(_layer(wl.fmt, d, wl.k, wl.M, "plain"), d))
