"""The GPU tests' comparator on the CPU: a localised error the cosine lets
through must fail the max-abs bar, and a difference within the output's own
bf16 rounding must pass."""
import numpy as np
import pytest

import oracle
import gpu_util
from gpu_util import COS_MIN, MAXABS_REL_RMS, W4A8_MAXABS_REL_RMS, compare


@pytest.fixture(autouse=True)
def _keep_records_clean():
    """These comparisons are planted; keep them out of the suite's table."""
    n = len(gpu_util.RECORDS)
    yield
    del gpu_util.RECORDS[n:]


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    return np.array([oracle.lib().oracle_f32_to_bf16(float(a)) for a in v.ravel()], dtype=np.uint16)


@pytest.fixture(scope="module")
def ref():
    rng = np.random.default_rng(7)
    return rng.standard_normal(4096).astype(np.float32)


def test_correctly_rounded_output_passes(ref):
    rec = compare(_bf16_bits(ref), ref, "rounded only")
    assert rec["cos"] > COS_MIN and rec["excess_rel"] <= 0.0


def test_single_large_error_fails_maxabs_even_when_cosine_passes(ref):
    bad = ref.copy()
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    bad[123] += 0.5 * rms
    g = oracle.bf16_bits_to_f32(_bf16_bits(bad)).astype(np.float64)
    cos = float(g @ ref / (np.linalg.norm(g) * np.linalg.norm(ref)))
    assert cos >= COS_MIN  # the cosine alone would pass this output
    with pytest.raises(AssertionError, match="max-abs"):
        compare(_bf16_bits(bad), ref, "one 0.5 RMS error")


def test_error_just_past_the_bar_fails_and_just_inside_passes(ref):
    # a value on an exact bf16 grid point, so rounding adds nothing to the error
    ref2 = oracle.bf16_bits_to_f32(_bf16_bits(ref)).astype(np.float32)
    rms = float(np.sqrt(np.mean(ref2.astype(np.float64) ** 2)))
    i = int(np.argmin(np.abs(ref2 - 1.0)))
    for factor, ok in ((0.5, True), (2.0, False)):
        bad = ref2.copy()
        bad[i] = np.float32(ref2[i] + factor * MAXABS_REL_RMS * rms)
        bits = _bf16_bits(bad)
        if ok:
            compare(bits, ref2, "inside")
        else:
            with pytest.raises(AssertionError, match="max-abs"):
                compare(bits, ref2, "outside")


def test_w4a8_bar_is_wider(ref):
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    bad = ref.copy()
    bad[5] += 0.05 * rms
    with pytest.raises(AssertionError):
        compare(_bf16_bits(bad), ref, "bf16 bar")
    compare(_bf16_bits(bad), ref, "w4a8 bar", bar=W4A8_MAXABS_REL_RMS)


def test_all_zero_reference_needs_exact_zero():
    z = np.zeros(64, dtype=np.float32)
    compare(np.zeros(64, dtype=np.uint16), z, "zeros")
    with pytest.raises(AssertionError):
        compare(np.full(64, 0x3F80, dtype=np.uint16), z, "ones")
