"""The C-ABI library on the host: it loads, exports every entry point the
header declares, and rejects bad arguments before any HIP call (so these run
without a GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from block_scaled_fp4_gather_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_fp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from block_scaled_fp4_gather_amd import build
        build.build()
    return moe.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) >= set(moe._SIGS)


def test_status_strings(L):
    for s, text in moe.STATUS.items():
        assert moe.status_string(s) == text
    assert moe.status_string(99) == "unknown status"


def test_prepared_bytes_counts_every_byte_once(L):
    """The resident buffer holds the logical bytes plus tile padding only."""
    for fmt, G in (("mxfp4", 32), ("nvfp4", 16)):
        for E, H, I in ((8, 256, 128), (512, 2560, 320), (3, 96, 64)):
            d = moe.Desc(fmt, E, H, I, 2, 1)
            n = moe.prepared_bytes(d)
            logical = E * (2 * I * (H // 2 + H // G) + H * (I // 2 + I // G))
            if fmt == "nvfp4":
                logical += 8 * E
            assert n >= logical
            # padding is bounded: whole 64-row FC2 tiles, 4-byte scale words,
            # 256-byte expert alignment and the globals header
            slack = E * (64 * (I // 2 + I // G + 4) + 2 * I * 4 + 64 * 4 + 256) + 256
            assert n - logical <= slack


def test_descriptor_validation(L):
    def status(desc):
        n = ctypes.c_size_t()
        return L.moe_fp4_prepared_bytes(ctypes.byref(desc.c()), ctypes.byref(n))

    assert status(moe.Desc("mxfp4", 8, 256, 128, 2, 1)) == 0
    assert status(moe.Desc(3, 8, 256, 128, 2, 1)) == 1          # unknown format
    assert status(moe.Desc("mxfp4", 0, 256, 128, 2, 1)) == 1    # no experts
    assert status(moe.Desc("mxfp4", 8, 240, 128, 2, 1)) == 1    # H not whole MX blocks
    assert status(moe.Desc("nvfp4", 8, 240, 128, 2, 1)) == 2    # whole NV blocks, not whole units
    assert status(moe.Desc("mxfp4", 8, 256, 128, 0, 1)) == 1    # k = 0
    assert L.moe_fp4_prepared_bytes(None, None) == 1


def _forward_status(L, desc, M=1, prepared=256, x=16, ids=4, w=4, out=16, ws=256, ws_bytes=1 << 30):
    # fake device addresses: validation must reject before any dereference
    return L.moe_fp4_forward(ctypes.byref(desc.c()), prepared, x, M, ids, w, out, ws, ws_bytes, None)


def test_forward_rejects_before_launch(L):
    d = moe.Desc("nvfp4", 512, 2560, 320, 10, 4)
    assert _forward_status(L, d, M=5) == 1                     # M > max_tokens
    assert _forward_status(L, d, M=-1) == 1
    assert _forward_status(L, d, prepared=None) == 1
    assert _forward_status(L, d, x=None) == 1
    assert _forward_status(L, d, prepared=256 + 16) == 1       # misaligned prepared buffer
    assert _forward_status(L, d, x=18) == 1                    # misaligned activations
    assert _forward_status(L, d, ws_bytes=1024) == 3           # workspace too small
    assert _forward_status(L, d, M=0, prepared=None) == 0      # nothing to do
    huge = moe.Desc("mxfp4", 8, 256, 128, 8, 1 << 20)
    assert _forward_status(L, huge, M=1) == 2                  # 2^23 routes of capacity > 2^22


def test_prepare_rejects_mismatched_globals(L):
    d = moe.Desc("mxfp4", 8, 256, 128, 2, 1).c()
    n = moe.prepared_bytes(moe.Desc("mxfp4", 8, 256, 128, 2, 1))
    # MXFP4 with a global pointer, and NVFP4 without one
    assert L.moe_fp4_prepare(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 256, n, None) == 1
    dn = moe.Desc("nvfp4", 8, 256, 128, 2, 1).c()
    assert L.moe_fp4_prepare(ctypes.byref(dn), 16, 16, 16, 16, None, None, 256, n, None) == 1
    assert L.moe_fp4_prepare(ctypes.byref(d), 16, 16, 16, 16, None, None, 256, 10, None) == 3


def test_tuning_hook_rejects_bad_shapes(L):
    d = moe.Desc("mxfp4", 8, 256, 128, 2, 1)   # I = 128: FC2 uses 4 chunk lanes
    def status(t, phases=3):
        return L.moe_fp4_forward_ex(ctypes.byref(d.c()), 256, 16, 1, 4, 4, 16, 256, 1 << 30,
                                    ctypes.byref(t) if t is not None else None, phases, None)
    assert status(moe.Tuning(3, 0, 0, 0)) == 1      # chunks per wave not 4/8/16
    assert status(moe.Tuning(0, 24, 0, 0)) == 1     # FC1 rows not 16/32
    assert status(moe.Tuning(0, 0, 8, 0)) == 1      # 8 FC2 rows x 4 lanes < 64
    assert status(moe.Tuning(0, 0, 0, 3)) == 1      # no such path
    assert status(moe.Tuning(0, 0, 0, -1)) == 1
    assert status(None, phases=0) == 1
    assert status(None, phases=5) == 1
    assert status(None, phases=4) == 1  # M = 1 takes the decode path: no routing-only phase


def test_decode_path_past_one_launch_pair(L):
    # past M * k = 64 route slots or M = 16 the decode path runs in chunks
    # (chosen automatically with bf16 activations up to 2 chunks, and up to 6
    # when the chunks' route slots number fewer than E)
    wide = moe.Desc("nvfp4", 512, 2560, 320, 10, 64)     # 6 tokens per chunk
    t = moe.Tuning(0, 0, 0, moe.PATH_DECODE)
    assert _plan(wide, 7, t)[0] == moe.PATH_DECODE
    assert _plan(wide, 36)[0] == moe.PATH_DECODE         # 6 chunks
    assert _plan(wide, 37)[0] == moe.PATH_GROUPED        # 7
    assert _plan(wide, 64, t)[0] == moe.PATH_DECODE
    # MXFP8 activations: the decode path only within one chunk by default
    a8 = moe.Desc("mxfp4", 256, 2048, 256, 8, 64, "mxfp8")
    assert _plan(a8, 8)[0] == moe.PATH_DECODE
    assert _plan(a8, 9)[0] == moe.PATH_GROUPED
    assert _plan(moe.Desc("mxfp4", 256, 2048, 256, 8, 64), 9)[0] == moe.PATH_DECODE
    small_e = moe.Desc("mxfp4", 64, 1024, 256, 8, 64)   # routes shared by few experts
    assert _plan(small_e, 16)[0] == moe.PATH_DECODE     # two chunks
    assert _plan(small_e, 17)[0] == moe.PATH_GROUPED    # three, 136 routes > E
    big_e = moe.Desc("mxfp4", 256, 2048, 256, 8, 64)
    assert _plan(big_e, 24)[0] == moe.PATH_DECODE       # three chunks, 192 slots < E
    assert _plan(big_e, 25)[0] == moe.PATH_GROUPED      # four, 256 slots
    # the grouped path's expert grouping holds at most 8192 experts; past it
    # the decode path takes every M
    wide_e = moe.Desc("mxfp4", 9000, 64, 32, 8, 64)
    assert _plan(wide_e, 64)[0] == moe.PATH_DECODE
    with pytest.raises(moe.MoeFp4Error) as ei:
        moe.plan(wide_e, 64, moe.Tuning(0, 0, 0, moe.PATH_GROUPED))
    assert ei.value.status == 2
    many = moe.Desc("mxfp4", 8, 256, 128, 1, 32)          # 16 tokens per chunk
    assert _plan(many, 17, t)[0] == moe.PATH_DECODE
    # the decode launches' second grid dimension holds at most 65535 chunks or groups
    huge_m = moe.Desc("mxfp4", 9000, 64, 32, 1, 70000)
    assert _plan(huge_m, 65535)[0] == moe.PATH_DECODE
    for bad in (None, t):
        with pytest.raises(moe.MoeFp4Error) as ei:
            moe.plan(huge_m, 65536, bad)
        assert ei.value.status == 2


def test_workspace_sizes_do_not_depend_on_m(L):
    d = moe.Desc("nvfp4", 288, 4096, 512, 8, 8)
    sizes = {moe.workspace_bytes(d, m) for m in (1, 2, 5, 8)}
    assert len(sizes) == 1
    size = sizes.pop()
    routes, H, I = 8 * 8, 4096, 512
    # decode: two bf16 activation planes per route slot; grouped: two bf16
    # activation rows and an fp32 output row per route, plus routing tables
    assert size >= 2 * 2 * routes * I
    assert routes * (4 * I + 4 * H) <= size <= routes * (4 * I + 4 * H) + 64 * 1024


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()


def test_activation_format_validation(L):
    def status(desc):
        n = ctypes.c_size_t()
        return L.moe_fp4_workspace_bytes(ctypes.byref(desc.c()), 1, ctypes.byref(n))

    assert status(moe.Desc("mxfp4", 8, 256, 128, 2, 4, "mxfp8")) == 0
    assert status(moe.Desc("nvfp4", 8, 256, 128, 2, 4, "mxfp8")) == 2   # E8M0 scales only
    assert status(moe.Desc("mxfp4", 8, 256, 128, 2, 4, 2)) == 1         # no such format
    assert status(moe.Desc("mxfp4", 8, 256, 128, 2, 4, -1)) == 1
    d = moe.Desc("nvfp4", 8, 256, 128, 2, 4, "mxfp8")
    assert _forward_status(L, d, M=1) == 2


def test_mxfp8_workspace_size(L):
    M, k, H, I = 300, 4, 1024, 256
    d = moe.Desc("mxfp4", 16, H, I, k, M, "mxfp8")
    size = moe.workspace_bytes(d, 1)
    routes = M * k
    # grouped: x codes + scales per token; act codes + scales and an fp32
    # output row per route; routing tables (5 int32 arrays) in between
    need = M * (H + H // 32) + routes * (I + I // 32 + 4 * H)
    assert need <= size <= need + 8 * 4 * routes + 64 * 1024
    assert size < moe.workspace_bytes(moe.Desc("mxfp4", 16, H, I, k, M), 1)


def test_mxfp8_quantize_rejects_before_launch(L):
    q = L.moe_fp4_mxfp8_quantize
    assert q(16, 4, 48, 16, 16, None) == 1      # cols not a multiple of 32
    assert q(16, -1, 64, 16, 16, None) == 1
    assert q(None, 4, 64, 16, 16, None) == 1
    assert q(18, 4, 64, 16, 16, None) == 1      # misaligned input
    assert q(16, 4, 64, 12, 16, None) == 1      # misaligned codes
    assert q(None, 0, 64, None, None, None) == 0  # nothing to do


def test_activation_function_validation(L):
    def status(**kw):
        n = ctypes.c_size_t()
        d = moe.Desc("mxfp4", 8, 256, 128, 2, 4, **kw)
        return L.moe_fp4_workspace_bytes(ctypes.byref(d.c()), 1, ctypes.byref(n))

    assert status(fn="silu") == 0
    assert status(fn="gelu_tanh") == 0
    assert status(fn="swigluoai", alpha=1.702, beta=1.0, limit=7.0) == 0
    assert status(fn="swigluoai", alpha=1.702, beta=1.0, limit=float("inf")) == 0
    assert status(fn=4) == 1                                                # no such activation
    assert status(fn=-1) == 1
    assert status(fn="swigluoai", alpha=1.702, beta=1.0, limit=0.0) == 1       # limit must be > 0
    assert status(fn="swigluoai", alpha=float("nan"), beta=1.0, limit=7.0) == 1
    assert status(fn="swigluoai", alpha=1.0, beta=float("inf"), limit=7.0) == 1
    assert status(fn="swigluoai", alpha=1.0, beta=0.0, limit=float("nan")) == 1


def test_relu2_layout_and_validation(L):
    def status(I):
        n = ctypes.c_size_t()
        return L.moe_fp4_prepared_bytes(ctypes.byref(moe.Desc("mxfp4", 8, 256, I, 2, 4, fn="relu2").c()),
                                        ctypes.byref(n))
    assert status(128) == 0
    assert status(96) == 2     # I must hold two 32-row halves per FC1 tile
    gated = moe.prepared_bytes(moe.Desc("mxfp4", 8, 256, 128, 2, 4))
    non_gated = moe.prepared_bytes(moe.Desc("mxfp4", 8, 256, 128, 2, 4, fn="relu2"))
    # W13 holds I rows instead of 2I: the FC1 part of every expert halves
    E, H, I = 8, 256, 128
    fc1_gated = 2 * I * (H // 2 + H // 32)
    assert gated - non_gated == E * fc1_gated // 2


def _plan(desc, M, tuning=None):
    p = moe.plan(desc, M, tuning)
    return p.path, p.fc1_chunks_per_wave, p.fc1_rows, p.fc2_rows


def test_plan_resolves_path_and_shape(L):
    # the decode band with its built-in launch shape, the grouped path past it
    e512 = moe.Desc("nvfp4", 512, 2560, 320, 10, 1)
    assert _plan(e512, 1) == (moe.PATH_DECODE, 4, 32, 16)
    assert _plan(moe.Desc("mxfp4", 8, 256, 128, 2, 1), 1) == (moe.PATH_DECODE, 4, 16, 32)
    shard = moe.Desc("mxfp4", 256, 7168, 256, 8, 4)
    assert _plan(shard, 1) == (moe.PATH_DECODE, 8, 16, 32)
    assert _plan(shard, 4) == (moe.PATH_DECODE, 4, 32, 32)
    assert _plan(moe.Desc("nvfp4", 288, 4096, 512, 8, 5), 5) == (moe.PATH_DECODE, 4, 32, 16)
    assert _plan(moe.Desc("mxfp4", 128, 4096, 1536, 8, 4096), 4096) == (moe.PATH_GROUPED, 0, 0, 0)
    # explicit fields are kept, the rest resolved; the grouped path at any M
    assert _plan(e512, 1, moe.Tuning(16, 16, 0, 0)) == (moe.PATH_DECODE, 16, 16, 16)
    assert _plan(e512, 1, moe.Tuning(0, 0, 0, moe.PATH_GROUPED)) == (moe.PATH_GROUPED, 0, 0, 0)
    # rejected requests: the same status moe_fp4_forward_ex gives
    for bad in (moe.Tuning(3, 0, 0, 0), moe.Tuning(0, 0, 0, 3)):
        with pytest.raises(moe.MoeFp4Error) as ei:
            moe.plan(e512, 1, bad)
        assert ei.value.status == 1
    with pytest.raises(moe.MoeFp4Error) as ei:
        moe.plan(moe.Desc("nvfp4", 512, 2560, 320, 65, 8), 1, moe.Tuning(0, 0, 0, moe.PATH_DECODE))
    assert ei.value.status == 2  # k = 65: more route slots than one wave holds
    with pytest.raises(moe.MoeFp4Error):
        moe.plan(e512, 2)  # M past max_tokens


def test_plan_rejects_decode_past_the_lds_limit(L):
    """FC1 of the decode path stages a token's H activations in LDS; a layer
    whose staging exceeds what a workgroup may allocate takes the grouped
    path by default and is rejected on the decode path before any launch."""
    wide = moe.Desc("mxfp4", 8, 131072, 32, 2, 1)
    assert _plan(wide, 1)[0] == moe.PATH_GROUPED
    with pytest.raises(moe.MoeFp4Error) as ei:
        moe.plan(wide, 1, moe.Tuning(0, 0, 0, moe.PATH_DECODE))
    assert ei.value.status == 2
    # the widest H whose staging still fits keeps the decode path
    assert _plan(moe.Desc("mxfp4", 8, 16384, 32, 2, 1), 1)[0] == moe.PATH_DECODE


def test_noalloc_forward_rejects_before_any_hip_call(L):
    """moe_fp4_forward_noalloc checks its arguments and the workspace the
    descriptor needs (at most the library's 64 MiB) before any HIP call."""
    fn = L.moe_fp4_forward_noalloc
    small = moe.Desc("mxfp4", 8, 256, 128, 2, 4)
    assert moe.workspace_bytes(small, 4) <= 64 << 20
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below is rejected or has M = 0
    args = lambda d, M, p=fake: (ctypes.byref(d.c()), p, p, M, p, p, p, None)
    assert fn(*args(small, 0)) == 0             # M = 0: nothing to do
    assert fn(*args(small, 1, nul)) == 1        # null pointers
    assert fn(*args(small, 5)) == 1             # M past max_tokens
    big = moe.Desc("mxfp4", 128, 4096, 1536, 8, 4096)  # the prefill layer needs ~700 MiB of workspace
    assert moe.workspace_bytes(big, 1) > 64 << 20
    assert fn(*args(big, 1)) == 3               # MOE_FP4_EWORKSPACE
    assert fn(*args(moe.Desc("mxfp4", 8, 250, 128, 2, 4), 1)) == 1  # H not whole scale blocks


def test_csf_prepared_bytes_and_validation(L):
    """The compressed scale format adds one CSF block per tile (a 256-byte
    group of one word per row for every 24 (MXFP4) or 3 (NVFP4) chunks) to the
    plain layout; any other scale format is rejected."""
    for fmt, G in (("mxfp4", 32), ("nvfp4", 16)):
        for E, H, I in ((8, 256, 128), (256, 7168, 256), (512, 2560, 320), (3, 96, 64)):
            plain = moe.prepared_bytes(moe.Desc(fmt, E, H, I, 2, 1))
            csf = moe.prepared_bytes(moe.Desc(fmt, E, H, I, 2, 1, scales="csf"))
            nC1, nC2 = H // 32, I // 32

            def block(nC):  # 256 bytes per group of 24 (MXFP4) or 3 (NVFP4) chunks
                return 256 * -(-nC // (24 if fmt == "mxfp4" else 3))
            tiles1, tiles2 = (2 * I) // 64, -(-H // 64)
            grow = E * (tiles1 * block(nC1) + tiles2 * block(nC2))
            # the expert stride stays a multiple of 256 bytes, so the growth is exact
            assert csf - plain == grow, (fmt, E, H, I)
    bad = moe.Desc("mxfp4", 8, 256, 128, 2, 1, scales=2)
    with pytest.raises(moe.MoeFp4Error) as ei:
        moe.prepared_bytes(bad)
    assert ei.value.status == 1


def test_csf_rejects_the_shapes_it_does_not_run(L):
    """With compressed scales the decode kernels keep each row's base byte
    and offsets in registers; the two launch shapes that would spill are
    rejected before any launch."""
    desc = moe.Desc("mxfp4", 4, 512, 320, 2, 1, scales="csf")
    assert _plan(desc, 1)[0] == moe.PATH_DECODE
    for t in (moe.Tuning(16, 32, 0, moe.PATH_DECODE),   # 8 FC1 rows per lane
              moe.Tuning(0, 0, 32, moe.PATH_DECODE)):   # 32 FC2 rows over two chunk groups (I = 320)
        with pytest.raises(moe.MoeFp4Error) as ei:
            moe.plan(desc, 1, t)
        assert ei.value.status == 1
    plain = moe.Desc("mxfp4", 4, 512, 320, 2, 1)
    assert _plan(plain, 1, moe.Tuning(16, 32, 32, moe.PATH_DECODE))[0] == moe.PATH_DECODE
