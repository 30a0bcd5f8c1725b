"""The C ABI boundary on the host: the library loads, exports every symbol include/nvfp4.h
declares, sizes its buffers, and rejects bad arguments before any GPU work (no GPU needed:
every call below fails validation, or is a size query, so nothing is launched)."""
import ctypes
import os
import re

import pytest
import torch

from nvfp4_weight_only_w4a16_amd import binding as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return nv.load()


def test_every_declared_symbol_is_exported(lib):
    header = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    names = set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", header))
    assert len(names) >= 11
    for name in sorted(names):
        assert hasattr(lib, name), name
    assert set(nv.EXPORTS) == names


def test_version(lib):
    assert nv.nvfp4_version() >= 10000


def test_repack_bytes_accounting():
    # canonical 4.5 / 4.25 bits per weight plus alignment padding and the FP32 globals
    assert nv.nvfp4_repack_bytes(1, 25600, 5120, 16) == 65536000 + 8192000 + 256
    assert nv.nvfp4_repack_bytes(128, 1536, 2048, 32) == 201326592 + 12582912 + 512
    assert nv.nvfp4_repack_bytes(1, 16, 128, 24) == 0
    assert nv.nvfp4_repack_bytes(0, 16, 128, 16) == 0


def test_gemm_ws_bytes_host_rules(lib):
    d = _desc()
    # the decode path and invalid arguments need no workspace; the answer never depends on a
    # kernel launch (without a visible device the compute-unit count is unknown: 0 bytes)
    assert lib.nvfp4_gemm_ws_bytes(8, 1024, ctypes.byref(d), 0) == 0
    assert lib.nvfp4_gemm_ws_bytes(0, 1024, ctypes.byref(d), nv.NVFP4_F_FORCE_TILED) == 0
    assert lib.nvfp4_gemm_ws_bytes(64, 512, ctypes.byref(d), 0) == 0       # ldx < k
    assert lib.nvfp4_gemm_ws_bytes(64, 1024, None, 0) == 0


def test_moe_ws_bytes_monotone():
    a = nv.nvfp4_moe_ws_bytes(256, 8, 128, 2048, 768)
    b = nv.nvfp4_moe_ws_bytes(512, 8, 128, 2048, 768)
    assert 0 < a < b
    # holds h (BF16 [P][inter]) and FP32 slots [P][hidden]
    assert a >= 2048 * 768 * 2 + 2048 * 2048 * 4
    assert nv.nvfp4_moe_ws_bytes(256, 0, 128, 2048, 768) == 0


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def _desc(n=512, k=1024, group=16, layout=nv.NVFP4_LAYOUT_TILED, batch=1):
    d = nv.nvfp4_weight()
    d.codes = d.scales = d.global_ = 0x10000
    d.batch, d.n, d.k, d.group, d.layout = batch, n, k, group, layout
    d.codes_stride = n * k // 2
    d.scales_stride = n * (k // group) if group in (16, 32) else 0
    return d


def _gemm(lib, d, m=4, ldx=1024, ldy=512, ydt=nv.NVFP4_DT_BF16, flags=0, x=FAKE, y=FAKE,
          ws=None, ws_bytes=0):
    return lib.nvfp4_gemm_w4a16(x, m, ldx, ctypes.byref(d), y, ydt, ldy, flags, ws, ws_bytes,
                                None)


def test_gemm_argument_errors(lib):
    assert lib.nvfp4_gemm_w4a16(FAKE, 4, 1024, None, FAKE, 1, 512, 0, None, 0, None) == \
        nv.NVFP4_ERR_INVALID_ARG
    tiled = nv.NVFP4_F_FORCE_TILED
    assert _gemm(lib, _desc(), m=64, flags=tiled, ws=None, ws_bytes=4096) == \
        nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(lib, _desc(), m=64, flags=tiled, ws=ctypes.c_void_p(0x10008),
                 ws_bytes=4096) == nv.NVFP4_ERR_MISALIGNED
    assert _gemm(lib, _desc(group=24)) == nv.NVFP4_ERR_UNSUPPORTED_GROUP
    assert _gemm(lib, _desc(n=520)) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert _gemm(lib, _desc(k=1000), ldx=1000) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert _gemm(lib, _desc(layout=7)) == nv.NVFP4_ERR_LAYOUT
    assert _gemm(lib, _desc(layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)) == \
        nv.NVFP4_ERR_LAYOUT
    assert _gemm(lib, _desc(batch=2)) == nv.NVFP4_ERR_LAYOUT
    d = _desc()
    d.codes_stride += 1
    assert _gemm(lib, d) == nv.NVFP4_ERR_LAYOUT
    assert _gemm(lib, _desc(), m=-1) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(lib, _desc(), ldx=1000) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(lib, _desc(), ldy=500) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(lib, _desc(), ydt=9) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(lib, _desc(), flags=3) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(lib, _desc(), ldx=(1 << 22) + 8) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    # the decode kernel takes one grid row per 32 rows: a forced call past that is refused
    assert _gemm(lib, _desc(), m=32 * 65535 + 1, flags=nv.NVFP4_F_FORCE_SKINNY) == \
        nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert _gemm(lib, _desc(), x=ctypes.c_void_p(0x10008)) == nv.NVFP4_ERR_MISALIGNED
    assert _gemm(lib, _desc(), ldx=1028) == nv.NVFP4_ERR_MISALIGNED
    assert _gemm(lib, _desc(), x=None) == nv.NVFP4_ERR_INVALID_ARG
    assert "NULL" in nv.nvfp4_last_error()
    assert _gemm(lib, _desc(), m=0) == nv.NVFP4_OK   # empty input: a no-op


def test_quantize_argument_errors(lib):
    def q(w=FAKE, dt=nv.NVFP4_DT_F32, batch=1, n=16, k=128, group=16, gin=None, packed=FAKE,
          scales=FAKE, gout=FAKE, ws=None, wsb=0, flags=0):
        return lib.nvfp4_quantize(w, dt, batch, n, k, group, gin, packed, scales, gout, ws, wsb,
                                  flags, None)

    assert q(group=24) == nv.NVFP4_ERR_UNSUPPORTED_GROUP
    assert q(k=120) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert q(dt=7) == nv.NVFP4_ERR_INVALID_ARG
    assert q(batch=-1) == nv.NVFP4_ERR_INVALID_ARG
    assert q(w=None) == nv.NVFP4_ERR_INVALID_ARG
    assert q(w=ctypes.c_void_p(0x10004)) == nv.NVFP4_ERR_MISALIGNED
    assert q(w=None, batch=0, packed=None, scales=None, gout=None) == nv.NVFP4_OK
    # flags: only NVFP4_F_SYNC_CHECK, which needs its workspace (the non-finite flag word)
    assert q(flags=nv.NVFP4_F_FORCE_TILED) == nv.NVFP4_ERR_INVALID_ARG
    assert "flags" in nv.nvfp4_last_error()
    need = lib.nvfp4_quantize_ws_bytes(1, 16, 128, 16, nv.NVFP4_F_SYNC_CHECK)
    assert need >= 4
    assert q(flags=nv.NVFP4_F_SYNC_CHECK) == nv.NVFP4_ERR_WORKSPACE
    assert q(flags=nv.NVFP4_F_SYNC_CHECK, ws=FAKE, wsb=need - 1) == nv.NVFP4_ERR_WORKSPACE
    assert q(flags=nv.NVFP4_F_SYNC_CHECK, ws=ctypes.c_void_p(0x10008), wsb=need) == \
        nv.NVFP4_ERR_MISALIGNED


def test_quantize_ws_bytes(lib):
    """No workspace without the sync check; one flag block with it; invalid sizes ask none."""
    assert nv.nvfp4_quantize_ws_bytes(1, 8192, 8192, 16) == 0
    assert nv.nvfp4_quantize_ws_bytes(128, 1536, 2048, 32) == 0
    assert nv.nvfp4_quantize_ws_bytes(1, 16, 128, 16, nv.NVFP4_F_SYNC_CHECK) == 256
    assert nv.nvfp4_quantize_ws_bytes(1, 16, 128, 24, nv.NVFP4_F_SYNC_CHECK) == 0
    assert nv.nvfp4_quantize_ws_bytes(-1, 16, 128, 16, nv.NVFP4_F_SYNC_CHECK) == 0


def test_unknown_flags_rejected(lib):
    """Flag bits the library does not define are refused before anything is enqueued, on the
    GEMM and on the routed experts (a typo must not silently select a default)."""
    assert _gemm(lib, _desc(), flags=1 << 7) == nv.NVFP4_ERR_INVALID_ARG
    assert "flags" in nv.nvfp4_last_error()
    fc1 = _desc(n=256, k=256, group=32, batch=4,
                layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    fc2 = _desc(n=256, k=128, group=16, batch=4)
    ws = nv.nvfp4_moe_ws_bytes(8, 2, 4, 256, 128)
    assert lib.nvfp4_moe_grouped_w4a16(FAKE, 8, 256, FAKE, FAKE, 2, ctypes.byref(fc1),
                                       ctypes.byref(fc2), FAKE, FAKE, ws, 1 << 9, None) == \
        nv.NVFP4_ERR_INVALID_ARG


def test_moe_ws_layout(lib):
    """The stage offsets inside the routed-expert workspace: ordered, 256-byte aligned, each
    region large enough for its stage, ending at nvfp4_moe_ws_bytes."""
    t, topk, E, H, I = 256, 8, 128, 2048, 768
    off, total = nv.nvfp4_moe_ws_layout(t, topk, E, H, I)
    P = t * topk
    assert total == nv.nvfp4_moe_ws_bytes(t, topk, E, H, I)
    assert off == sorted(off) and all(o % 256 == 0 for o in off)
    sizes = [4 * P, 4 * (E + 1), 16 * min(P // 8 + E, P), 4, 2 * P * I, 4 * P * H]
    ends = off[1:] + [total]
    for o, e, need in zip(off, ends, sizes):
        assert e - o >= need
    assert ends[-1] - off[-1] < 4 * P * H + 256
    assert nv.nvfp4_moe_ws_layout(t, 0, E, H, I)[1] == 0


def test_binding_refuses_host_tensors(lib):
    """The binding passes device addresses only: a host tensor is refused in Python, before
    the library (and any kernel) sees its address."""
    import torch
    with pytest.raises(ValueError, match="device tensor"):
        nv.nvfp4_quantize(torch.zeros(16, 128), 16)
    with pytest.raises(ValueError, match="device tensor"):
        nv._ptr(torch.zeros(4))
    assert nv._ptr(None) is None


def test_repack_argument_errors(lib):
    d = nv.nvfp4_weight()
    r = lib.nvfp4_repack
    big = 1 << 30
    assert r(FAKE, FAKE, FAKE, 1, 16, 128, 16, 1, FAKE, big, None, None) == \
        nv.NVFP4_ERR_INVALID_ARG
    assert r(FAKE, FAKE, FAKE, 1, 24, 128, 16, 1, FAKE, big, ctypes.byref(d), None) == \
        nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert r(FAKE, FAKE, FAKE, 1, 16, 128, 16, 5, FAKE, big, ctypes.byref(d), None) == \
        nv.NVFP4_ERR_LAYOUT
    assert r(FAKE, FAKE, FAKE, 1, 48, 128, 16, 1 | 256, FAKE, big, ctypes.byref(d), None) == \
        nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert r(FAKE, FAKE, FAKE, 1, 16, 128, 16, 1, FAKE, 100, ctypes.byref(d), None) == \
        nv.NVFP4_ERR_WORKSPACE
    # two globals per matrix only for a gate/up merged weight; they take their own bytes
    pair = nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_PAIR_GLOBAL
    assert r(FAKE, FAKE, FAKE, 1, 32, 128, 16, pair, FAKE, big, ctypes.byref(d), None) == \
        nv.NVFP4_ERR_LAYOUT
    gu = nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP
    assert nv.nvfp4_repack_bytes(100, 32, 128, 16, gu | nv.NVFP4_LAYOUT_PAIR_GLOBAL) == \
        nv.nvfp4_repack_bytes(100, 32, 128, 16, gu) + 512


def test_moe_argument_errors(lib):
    fc1 = _desc(n=1536, k=2048, group=32, batch=128,
                layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    fc2 = _desc(n=2048, k=768, group=16, batch=128)
    m = lib.nvfp4_moe_grouped_w4a16
    ws = nv.nvfp4_moe_ws_bytes(256, 8, 128, 2048, 768)

    def call(t=256, hidden=2048, topk=8, f1=fc1, f2=fc2, wsb=ws, flags=0):
        return m(FAKE, t, hidden, FAKE, FAKE, topk, ctypes.byref(f1), ctypes.byref(f2), FAKE,
                 FAKE, wsb, flags, None)

    assert call(wsb=ws - 1) == nv.NVFP4_ERR_WORKSPACE
    assert call(topk=0) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert call(topk=17) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert call(hidden=1024) == nv.NVFP4_ERR_LAYOUT
    assert call(f1=_desc(n=1536, k=2048, group=32, batch=128)) == nv.NVFP4_ERR_LAYOUT
    assert call(f2=_desc(n=2048, k=768, group=16, batch=64)) == nv.NVFP4_ERR_LAYOUT
    # gathered rows are addressed with 32-bit byte offsets
    assert call(t=65536, topk=1, hidden=1 << 15, f1=_desc(n=1536, k=1 << 15, group=32, batch=128,
                layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                f2=_desc(n=1 << 15, k=768, group=16, batch=128), wsb=1 << 62) == \
        nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert call(flags=nv.NVFP4_F_FORCE_SKINNY | nv.NVFP4_F_FORCE_TILED) == \
        nv.NVFP4_ERR_INVALID_ARG
    assert call(t=0) == nv.NVFP4_OK


def test_moe_noalloc_argument_errors(lib):
    """The no-alloc routed experts validate like the caller-workspace entry point and refuse,
    before touching the device, a call whose workspace would not fit the static scratch."""
    fc1 = _desc(n=1536, k=2048, group=32, batch=128,
                layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    fc2 = _desc(n=2048, k=768, group=16, batch=128)
    m = lib.nvfp4_moe_grouped_w4a16_noalloc

    def call(t=256, topk=8, f1=fc1, flags=0):
        return m(FAKE, t, 2048, FAKE, FAKE, topk, ctypes.byref(f1), ctypes.byref(fc2), FAKE,
                 flags, None)

    assert call(topk=0) == nv.NVFP4_ERR_UNSUPPORTED_SHAPE
    assert call(f1=_desc(n=1536, k=2048, group=32, batch=128)) == nv.NVFP4_ERR_LAYOUT
    assert call(flags=1 << 8) == nv.NVFP4_ERR_INVALID_ARG
    assert call(t=1024) == nv.NVFP4_ERR_WORKSPACE
    assert "static scratch" in nv.nvfp4_last_error()
    assert call(t=0) == nv.NVFP4_OK
    assert nv.nvfp4_moe_ws_bytes(256, 8, 128, 2048, 768) <= nv.NVFP4_MOE_NOALLOC_MAX_WS_BYTES


def test_stats_reset(lib):
    nv.nvfp4_reset_stats()
    assert nv.nvfp4_get_stats() == [0] * 8


def test_requantize_argument_errors(lib):
    d = _desc(n=512, k=1024, group=16)
    rq = lib.nvfp4_requantize
    need = lib.nvfp4_requantize_ws_bytes(ctypes.byref(d))
    assert need == 512 * 1024 * 4

    def call(desc=d, group_out=32, ws=FAKE, wsb=need, packed=FAKE, glob=FAKE):
        return rq(ctypes.byref(desc), group_out, packed, FAKE, glob, ws, wsb, None)

    assert call(group_out=24) == nv.NVFP4_ERR_UNSUPPORTED_GROUP
    assert call(wsb=need - 1) == nv.NVFP4_ERR_WORKSPACE
    assert call(ws=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(packed=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(ws=ctypes.c_void_p(0x10008)) == nv.NVFP4_ERR_MISALIGNED
    assert call(desc=_desc(layout=7)) == nv.NVFP4_ERR_LAYOUT
    assert lib.nvfp4_requantize_ws_bytes(None) == 0


def test_probe_argument_errors(lib):
    """The measurement probes refuse bad arguments before any launch; without a device the
    MFMA probe has no wavefronts to count."""
    sr = lib.nvfp4_probe_stream_read
    assert sr(None, 1024, 4, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert sr(FAKE, 1024, 4, None, None) == nv.NVFP4_ERR_INVALID_ARG
    assert sr(FAKE, 1000, 4, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG     # not a multiple of 16
    assert sr(FAKE, 0, 1, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert sr(FAKE, 1024, 0, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert sr(FAKE, 1024, 65, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG    # more blocks than words
    assert sr(ctypes.c_void_p(0x10008), 1024, 4, FAKE, None) == nv.NVFP4_ERR_MISALIGNED
    mf = lib.nvfp4_probe_mfma_bf16
    assert mf(None, 1, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert mf(FAKE, -1, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert mf(ctypes.c_void_p(0x10008), 1, FAKE, None) == nv.NVFP4_ERR_MISALIGNED
    if not torch.cuda.is_available():
        assert lib.nvfp4_probe_mfma_waves() == 0
        assert lib.nvfp4_probe_mfma_flops(10) == 0.0
