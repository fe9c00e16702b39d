"""Helpers for GPU tests: move seeded inputs to the device, run the layer
through the C-ABI, and compare with the CPU oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from block_scaled_fp4_gather_amd import moe, synth

# Parity bar for the layer output (fp64 over all M x H values): cosine >=
# 0.99995 against the oracle's fp32 sums, and |gpu - oracle| <= 2e-2 * RMS
# plus half a bf16 ulp of the oracle value.  The half ulp is the output's own
# rounding: the oracle's correctly rounded bf16 output alone reaches 0.0218 *
# RMS on heavy-tailed outputs (max |v| = 8.7 RMS), so the bar is read as
# bounding the error beyond that unavoidable rounding.
COS_MIN = 0.99995
MAXABS_REL_RMS = 2e-2

# The W4A8-MX variant against the oracle's W4A8 layer: the same cosine, and
# max-abs beyond bf16 rounding <= 0.1 * RMS.  Its activations are quantised
# to E4M3 from fp32 FC1 results that GPU and oracle sum in different orders,
# so an activation on a rounding midpoint can take the adjacent code (the
# identity-projection test measures 1.7e-4 of the codes flipping, every one
# to a neighbour).  One flip moves a route's output by one E4M3 step of that
# activation (at most |a| / 8) times the W2 column: for a route's largest
# activation on these heavy-tailed rows, a few percent of the output RMS.
W4A8_MAXABS_REL_RMS = 0.1


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits)."""
    _, e = np.frexp(np.abs(v))
    return np.where(v == 0, 0.0, np.ldexp(1.0, e - 9))


def say(*a):
    print(*a, file=sys.stdout, flush=True)


def to_dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def make_layer(fmt: str, d: dict, k: int, max_tokens: int, act: str = "bf16") -> moe.Fp4MoE:
    E, twoI, Hh = d["w13_codes"].shape
    desc = moe.Desc(fmt, E, 2 * Hh, twoI // 2, k, max_tokens, act)
    return moe.Fp4MoE(desc, to_dev(d["w13_codes"]), to_dev(d["w13_scales"]), to_dev(d["w2_codes"]),
                      to_dev(d["w2_scales"]), to_dev(d.get("g13")), to_dev(d.get("g2")))


def run_layer(layer: moe.Fp4MoE, d: dict, ids_dtype=torch.int32, **kw) -> np.ndarray:
    x = to_dev(d["x"]).view(torch.bfloat16)  # bf16 bit patterns
    ids = torch.from_numpy(np.ascontiguousarray(d["ids"])).to(ids_dtype).cuda()
    w = to_dev(d["w"])
    out = layer(x, ids, w, **kw)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(bits).astype(np.float64)


# Every compare() call of the session, for the summary table the suite prints
# at its end (tests/conftest.py).
RECORDS: list[dict] = []


def compare(gpu_bits: np.ndarray, acc: np.ndarray, label: str = "", bar: float = MAXABS_REL_RMS) -> dict:
    """Checks a bf16 layer output against the oracle's fp32 sums: cosine >=
    COS_MIN and max |gpu - oracle| beyond half a bf16 ulp of the oracle value
    <= bar * RMS(oracle), both in fp64 over every value."""
    g = bf16_to_f64(gpu_bits).ravel()
    r = acc.astype(np.float64).ravel()
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    if rms == 0.0:
        assert np.array_equal(gpu_bits, np.zeros_like(gpu_bits)), f"{label}: expected +0 everywhere"
        rec = dict(test=test, label=label, n=int(r.size), cos=1.0, maxabs_rel=0.0, excess_rel=0.0, bar=bar)
        RECORDS.append(rec)
        return rec
    assert np.isfinite(g).all(), f"{label}: non-finite GPU output"
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r)))
    err = np.abs(g - r)
    maxabs_rel = float(err.max()) / rms
    excess_rel = float(np.max(err - bf16_half_ulp(r))) / rms
    say(f"  {label}: cos={cos:.8f} maxabs/rms={maxabs_rel:.3e} beyond-rounding/rms={excess_rel:.3e} (bar {bar})")
    rec = dict(test=test, label=label, n=int(r.size), cos=cos, maxabs_rel=maxabs_rel, excess_rel=excess_rel, bar=bar)
    RECORDS.append(rec)
    assert cos >= COS_MIN, f"{label}: cosine {cos} < {COS_MIN}"
    assert excess_rel <= bar, f"{label}: max-abs/RMS beyond bf16 rounding {excess_rel} > {bar}"
    return rec


def workload_inputs(name: str, seed=None) -> tuple[synth.Workload, dict]:
    wl = synth.WORKLOADS[name]
    return wl, synth.generate(wl, seed)
