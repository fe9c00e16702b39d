"""Seeded synthetic inputs for the block-scaled FP4 mixture-of-experts layer.

This module is the one piece shared by the CPU oracle's tests and the HIP
path's tests and benchmark.  It draws random numbers and packs them into the
layer's input formats; it holds none of the layer's arithmetic (no decode, no
dequantisation, no GEMV, no activation, no combine).  Float-to-bf16 and
float-to-E4M3 encodings of *inputs* are delegated to PyTorch's CPU casts, so
no format arithmetic is written here either.

Generator (counter based, so any slice of a stream is reproducible):
  * SplitMix64 finaliser applied to key + (i+1)*0x9E3779B97F4A7C15, where the
    key is the finaliser of seed XOR finaliser(stream_id + 1);
  * uniform in [0, 1) from the top 53 bits;
  * normal from Box-Muller, cos branch only, one normal per pair of uniforms.

Workloads follow the geometries the pages measure on: the E512/H2560/I320
and E288/H4096/I512 rows of the decoder-only cold-L2 table (b12x PR #459,
"Reduce NVFP4-CSF scale reconstruction overhead", PR body table), the
M=1 tiny-decode band of b12x PR #22 ("rp-native tiny-decode kernel for
w4a8_mx (M=1)", Notes), a one-GPU shard of an E256/H7168 layer at M=1,2,4,
and an E128/H4096/I1536 prefill with 4096 tokens.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

SEED_BASE = 0x4D4F454600000000


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_scalar(v: int) -> int:
    return int(_mix64(np.array([v & (2**64 - 1)], dtype=np.uint64))[0])


class Stream:
    """One independent counter-based SplitMix64 stream."""

    def __init__(self, seed: int, stream_id: int):
        self.key = np.uint64(_mix64_scalar(seed ^ _mix64_scalar(stream_id + 1)))
        self.ctr = 0

    def u64(self, n: int) -> np.ndarray:
        out = np.empty(n, dtype=np.uint64)
        with np.errstate(over="ignore"):
            for s in range(0, n, _CHUNK):
                e = min(n, s + _CHUNK)
                i = np.arange(self.ctr + s + 1, self.ctr + e + 1, dtype=np.uint64)
                out[s:e] = _mix64(self.key + i * _GAMMA)
        self.ctr += n
        return out

    def uniform(self, n: int) -> np.ndarray:
        return (self.u64(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def normal(self, n: int) -> np.ndarray:
        u = self.uniform(2 * n)
        u1 = 1.0 - u[0::2]  # (0, 1]
        u2 = u[1::2]
        return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)

    def bytes(self, n: int) -> np.ndarray:
        return self.u64((n + 7) // 8).view(np.uint8)[:n].copy()

    def integers(self, lo: int, hi: int, n: int) -> np.ndarray:
        """Integers uniform in [lo, hi] (inclusive); modulo bias < 2^-50."""
        span = np.uint64(hi - lo + 1)
        return (self.u64(n) % span).astype(np.int64) + lo


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str  # "mxfp4" or "nvfp4"
    E: int
    H: int
    I: int
    M: int
    k: int
    seed: int
    n_invalid: int = 0  # route slots overwritten with out-of-range ids
    description: str = ""
    scales: str = "plain"  # "csf": rows whose scales fit the compressed scale format, 1 in csf_plain_rows not
    csf_plain_rows: int = 64  # with scales="csf": 1 in this many rows drawn plain (0: none)

    @property
    def G(self) -> int:
        return 32 if self.fmt == "mxfp4" else 16

    @property
    def format_code(self) -> int:
        return 1 if self.fmt == "mxfp4" else 2

    def expert_bytes(self) -> int:
        """Codes + block scales of one expert (W13 and W2)."""
        w13 = 2 * self.I * (self.H // 2 + self.H // self.G)
        w2 = self.H * (self.I // 2 + self.I // self.G)
        return w13 + w2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_mxfp4": Workload(
        "tiny_mxfp4", "mxfp4", E=8, H=256, I=128, M=1, k=2, seed=SEED_BASE + 0,
        description="MXFP4 E8/H256/I128, M=1, top-2"),
    "nvfp4_decode_e512": Workload(
        "nvfp4_decode_e512", "nvfp4", E=512, H=2560, I=320, M=1, k=10, seed=SEED_BASE + 1,
        description="NVFP4 decode E512/H2560/I320, M=1, top-10"),
    "nvfp4_multi_e288": Workload(
        "nvfp4_multi_e288", "nvfp4", E=288, H=4096, I=512, M=5, k=8, seed=SEED_BASE + 2,
        n_invalid=2, description="NVFP4 multi-token decode E288/H4096/I512, M=5, top-8, 2 of 40 ids invalid"),
    "mxfp4_shard_e256_m1": Workload(
        "mxfp4_shard_e256_m1", "mxfp4", E=256, H=7168, I=256, M=1, k=8, seed=SEED_BASE + 3 + 1,
        description="MXFP4 one-GPU shard E256/H7168/I256, M=1, top-8"),
    "mxfp4_shard_e256_m2": Workload(
        "mxfp4_shard_e256_m2", "mxfp4", E=256, H=7168, I=256, M=2, k=8, seed=SEED_BASE + 3 + 2,
        description="MXFP4 one-GPU shard E256/H7168/I256, M=2, top-8"),
    "mxfp4_shard_e256_m4": Workload(
        "mxfp4_shard_e256_m4", "mxfp4", E=256, H=7168, I=256, M=4, k=8, seed=SEED_BASE + 3 + 4,
        description="MXFP4 one-GPU shard E256/H7168/I256, M=4, top-8"),
    "mxfp4_prefill_e128": Workload(
        "mxfp4_prefill_e128", "mxfp4", E=128, H=4096, I=1536, M=4096, k=8, seed=SEED_BASE + 4,
        description="MXFP4 prefill E128/H4096/I1536, M=4096, top-8"),
    # Extra sweep points (not configurations): the decoder-only geometries at
    # the other routed-row counts of the pages' table (b12x #459, PR body:
    # 10, 40 and 63 routed rows), as M tokens x top-k routes.
    "nvfp4_e512_routed40": Workload(
        "nvfp4_e512_routed40", "nvfp4", E=512, H=2560, I=320, M=4, k=10, seed=SEED_BASE + 100,
        description="NVFP4 E512/H2560/I320, M=4, top-10 (40 routes)"),
    "nvfp4_e512_routed63": Workload(
        "nvfp4_e512_routed63", "nvfp4", E=512, H=2560, I=320, M=7, k=9, seed=SEED_BASE + 101,
        description="NVFP4 E512/H2560/I320, M=7, top-9 (63 routes)"),
    "nvfp4_e288_routed10": Workload(
        "nvfp4_e288_routed10", "nvfp4", E=288, H=4096, I=512, M=1, k=10, seed=SEED_BASE + 102,
        description="NVFP4 E288/H4096/I512, M=1, top-10 (10 routes)"),
    # The compressed-scale format (b12x #459: one-bit MXFP4 and four-bit
    # NVFP4 offsets from a row base byte) on the M = 1 geometries of the
    # metric and of the E512 decoder table row, with scales drawn so that
    # rows fit it (1 in 64 rows does not).
    "mxfp4_csf_shard_e256_m1": Workload(
        "mxfp4_csf_shard_e256_m1", "mxfp4", E=256, H=7168, I=256, M=1, k=8, seed=SEED_BASE + 200,
        scales="csf", description="MXFP4 shard E256/H7168/I256, M=1, top-8, compressed scales"),
    "nvfp4_csf_decode_e512": Workload(
        "nvfp4_csf_decode_e512", "nvfp4", E=512, H=2560, I=320, M=1, k=10, seed=SEED_BASE + 201,
        scales="csf", description="NVFP4 decode E512/H2560/I320, M=1, top-10, compressed scales"),
    "nvfp4_e288_routed63": Workload(
        "nvfp4_e288_routed63", "nvfp4", E=288, H=4096, I=512, M=7, k=9, seed=SEED_BASE + 103,
        description="NVFP4 E288/H4096/I512, M=7, top-9 (63 routes)"),
}

# Stream ids: one per drawn tensor, so that changing one shape leaves the
# other tensors' draws unchanged.
_S_W13C, _S_W13S, _S_W2C, _S_W2S, _S_X, _S_LOGIT, _S_INVALID = range(7)


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _e4m3_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def scales(wl: Workload, stream: Stream, n: int) -> np.ndarray:
    """Block-scale bytes: UE8M0 exponent uniform in [118, 126] (MXFP4), or
    E4M3 of min(|N(0,1)| * 64, 448) (NVFP4)."""
    if wl.fmt == "mxfp4":
        return stream.integers(118, 126, n).astype(np.uint8)
    v = np.minimum(np.abs(stream.normal(n)) * 64.0, 448.0)
    return _e4m3_bits(v.astype(np.float32))


def csf_scales(wl: Workload, stream: Stream, rows: int, n: int) -> np.ndarray:
    """Block-scale bytes [rows][n] whose rows mostly fit the compressed scale
    format: per row a base byte and an offset per block, the byte being
    base + offset (MXFP4: base uniform in [118, 125], offset 0 or 1, so the
    bytes stay in [118, 126]; NVFP4: base the E4M3 code of min(|N(0,1)| * 64,
    448) capped at 0x6F, offset uniform in [0, 15], so codes stay at or
    below 0x7E = 448).  One row in wl.csf_plain_rows (uniformly chosen) is
    drawn by the plain recipe instead and mostly does not fit."""
    if wl.fmt == "mxfp4":
        base = stream.integers(118, 125, rows).astype(np.int64)
        off = stream.integers(0, 1, rows * n).reshape(rows, n)
    else:
        b = _e4m3_bits(np.minimum(np.abs(stream.normal(rows)) * 64.0, 448.0).astype(np.float32))
        base = np.minimum(b.astype(np.int64), 0x6F)
        off = stream.integers(0, 15, rows * n).reshape(rows, n)
    out = (base[:, None] + off).astype(np.uint8)
    plain = stream.uniform(rows) < (1.0 / wl.csf_plain_rows if wl.csf_plain_rows else 0.0)
    if plain.any():
        out[plain] = scales(wl, stream, int(plain.sum()) * n).reshape(-1, n)
    return out


def weights(wl: Workload) -> dict:
    """Expert weights in the logical layout: W13 codes [E][2I][H/2], W13
    scales [E][2I][H/G], W2 codes [E][H][I/2], W2 scales [E][H][I/G]; the
    element at column c of a row sits in byte c/2, low nibble for even c."""
    E, H, I, G = wl.E, wl.H, wl.I, wl.G
    w13c = Stream(wl.seed, _S_W13C).bytes(E * 2 * I * H // 2).reshape(E, 2 * I, H // 2)
    w2c = Stream(wl.seed, _S_W2C).bytes(E * H * I // 2).reshape(E, H, I // 2)
    if wl.scales == "csf":
        w13s = csf_scales(wl, Stream(wl.seed, _S_W13S), E * 2 * I, H // G).reshape(E, 2 * I, H // G)
        w2s = csf_scales(wl, Stream(wl.seed, _S_W2S), E * H, I // G).reshape(E, H, I // G)
    else:
        w13s = scales(wl, Stream(wl.seed, _S_W13S), E * 2 * I * H // G).reshape(E, 2 * I, H // G)
        w2s = scales(wl, Stream(wl.seed, _S_W2S), E * H * I // G).reshape(E, H, I // G)
    if wl.fmt == "nvfp4":
        g13 = np.full(E, 1.0 / 512.0, dtype=np.float32)
        g2 = np.full(E, 1.0 / 512.0, dtype=np.float32)
    else:
        g13 = g2 = None
    return dict(w13_codes=w13c, w13_scales=w13s, w2_codes=w2c, w2_scales=w2s, g13=g13, g2=g2)


def activations(wl: Workload, seed: int | None = None, M: int | None = None) -> np.ndarray:
    """bf16 bit patterns of x ~ N(0, 1), shape [M][H]."""
    seed = wl.seed if seed is None else seed
    M = wl.M if M is None else M
    return _bf16_bits(Stream(seed, _S_X).normal(M * wl.H).astype(np.float32)).reshape(M, wl.H)


def routing(wl: Workload, seed: int | None = None, M: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Top-k ids (int32 [M][k]) and weights (fp32 [M][k]) from N(0,1) logits:
    softmax over all E, top-k (ties to the lower index), renormalised to sum 1.
    If the workload asks for invalid ids, that many distinct slots are chosen
    uniformly; the first becomes -1, the others an id >= E drawn from
    {E, E+1, 2^31-1}.  Their weights stay as drawn (nonzero)."""
    seed = wl.seed if seed is None else seed
    M = wl.M if M is None else M
    E, k = wl.E, wl.k
    logits = Stream(seed, _S_LOGIT).normal(M * E).reshape(M, E)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, ids, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = ids.astype(np.int32)
    if wl.n_invalid:
        st = Stream(seed, _S_INVALID)
        slots: list[int] = []
        while len(slots) < min(wl.n_invalid, M * k):
            s = int(st.integers(0, M * k - 1, 1)[0])
            if s not in slots:
                slots.append(s)
        flat = ids.reshape(-1)
        for i, s in enumerate(slots):
            if i == 0:
                flat[s] = -1
            else:
                flat[s] = [E, E + 1, 2**31 - 1][int(st.integers(0, 2, 1)[0])]
    return ids, w


def generate(wl: Workload, seed: int | None = None) -> dict:
    """All inputs of one layer call."""
    d = weights(wl)
    d["x"] = activations(wl, seed)
    d["ids"], d["w"] = routing(wl, seed)
    return d


def random_codes(stream: Stream, shape) -> np.ndarray:
    """Uniform code bytes of a given shape (helper for tests)."""
    n = int(np.prod(shape))
    return stream.bytes(n).reshape(shape)
