"""Pins of the oracle's compressed-scale (CSF) encoding and decoding
(b12x PR #459, "Reduce NVFP4-CSF scale reconstruction overhead", commit
messages: one-bit MXFP4 and four-bit NVFP4 offsets from a row base byte).
Each check is against something other than the oracle: hand-derived rows,
closed-form counts over every two-block row, and the lossless round trip
with garbage in the uncompressed bytes of compressible rows."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "csf_rows.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, sc, base, off, comp = [f.strip() for f in line.split("|")]
        rows.append((fmt, np.array([int(v, 16) for v in sc.split()], np.uint8), int(base, 16),
                     np.array([int(v) for v in off.split()], np.uint8), comp == "1"))
    return rows


def test_golden_rows():
    rows = _golden()
    assert len(rows) == 11
    for fmt, sc, base, off, comp in rows:
        b, o, c = oracle.csf_encode(fmt, sc)
        assert (b, c) == (base, comp), (fmt, sc)
        assert np.array_equal(o, off), (fmt, sc)
        # the decode gives the bytes back; exceptions from the plain bytes
        assert np.array_equal(oracle.csf_decode(fmt, b, o, sc), sc)


@pytest.mark.parametrize("fmt,expected", [
    # every ordered pair (a, b) of bytes: compressible iff |a - b| <= reach
    # and min(a, b) < 255.  MXFP4 (reach 1): 255 equal pairs below 255, plus
    # 255 pairs (a, a+1) and 255 pairs (a+1, a): 765.  NVFP4 (reach 15):
    # 255 equal pairs, plus 2 * (256 - d) ordered pairs at each distance
    # d = 1..15: 255 + 2 * (15 * 256 - 120) = 7695.
    ("mxfp4", 765), ("nvfp4", 7695)])
def test_compressible_two_block_rows_count(fmt, expected):
    n = 0
    garbage = np.array([0x5A, 0xA5], np.uint8)
    for a in range(256):
        for b in range(256):
            sc = np.array([a, b], np.uint8)
            base, off, comp = oracle.csf_encode(fmt, sc)
            if comp:
                n += 1
                assert base == min(a, b) and off.max() <= (1 if fmt == "mxfp4" else 15)
                # compressible rows never read their uncompressed bytes
                assert np.array_equal(oracle.csf_decode(fmt, base, off, garbage), sc)
            else:
                assert base == 255 and not off.any()
                assert np.array_equal(oracle.csf_decode(fmt, base, off, sc), sc)
    assert n == expected


def test_lossless_on_long_random_rows():
    rng = np.random.default_rng(459)
    for fmt, reach in (("mxfp4", 1), ("nvfp4", 15)):
        for trial in range(300):
            n = int(rng.integers(1, 400))
            lo = int(rng.integers(0, 256))
            span = int(rng.integers(0, 2 * reach + 2))
            sc = np.clip(lo + rng.integers(0, span + 1, n), 0, 255).astype(np.uint8)
            base, off, comp = oracle.csf_encode(fmt, sc)
            plain = sc if not comp else rng.integers(0, 256, n).astype(np.uint8)
            assert np.array_equal(oracle.csf_decode(fmt, base, off, plain), sc)
            # dequantised weights are unchanged by the round trip
            codes = rng.integers(0, 256, (1, n * (16 if fmt == "mxfp4" else 8))).astype(np.uint8)
            back = oracle.csf_decode(fmt, base, off, plain).reshape(1, n)
            np.testing.assert_array_equal(oracle.dequant(fmt, codes, back), oracle.dequant(fmt, codes, sc.reshape(1, n)))


def test_decode_rejects_offsets_past_the_reach():
    with pytest.raises(ValueError):
        oracle.csf_decode("mxfp4", 100, np.array([2], np.uint8), np.array([0], np.uint8))
    with pytest.raises(ValueError):
        oracle.csf_decode("nvfp4", 100, np.array([16], np.uint8), np.array([0], np.uint8))
