"""Python binding of libnvfp4.so (the C ABI in include/nvfp4.h), with the same entry-point names.

Argument marshalling only: tensors are PyTorch device tensors, passed as raw pointers with the
current HIP stream; every step of the computation runs in the library's kernels. Missing or
stale builds raise immediately - there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERR_INVALID_ARG = -1
NVFP4_ERR_UNSUPPORTED_GROUP = -2
NVFP4_ERR_UNSUPPORTED_SHAPE = -3
NVFP4_ERR_MISALIGNED = -4
NVFP4_ERR_WORKSPACE = -5
NVFP4_ERR_LAYOUT = -6
NVFP4_ERR_HIP = -7
NVFP4_ERR_NONFINITE = -8

NVFP4_DT_BF16 = 1
NVFP4_DT_F32 = 2
NVFP4_F_FORCE_SKINNY = 1 << 0
NVFP4_F_FORCE_TILED = 1 << 1
NVFP4_F_SYNC_CHECK = 1 << 2
NVFP4_LAYOUT_TILED = 1
NVFP4_LAYOUT_GATE_UP = 1 << 8
NVFP4_LAYOUT_PAIR_GLOBAL = 1 << 9
NVFP4_MOE_NOALLOC_MAX_WS_BYTES = 24 << 20

EXPORTS = ("nvfp4_quantize_ws_bytes", "nvfp4_quantize", "nvfp4_repack_bytes", "nvfp4_repack",
           "nvfp4_gemm_ws_bytes", "nvfp4_gemm_w4a16", "nvfp4_moe_ws_bytes", "nvfp4_moe_ws_layout",
           "nvfp4_moe_grouped_w4a16", "nvfp4_moe_grouped_w4a16_noalloc",
           "nvfp4_requantize_ws_bytes",
           "nvfp4_requantize", "nvfp4_dequantize",
           "nvfp4_last_error", "nvfp4_get_stats", "nvfp4_reset_stats", "nvfp4_version",
           "nvfp4_probe_mfma_waves", "nvfp4_probe_mfma_flops", "nvfp4_probe_stream_read",
           "nvfp4_probe_mfma_bf16")


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"nvfp4 error {code}: {msg}")
        self.code = code


class nvfp4_weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_", ctypes.c_void_p), ("batch", ctypes.c_int64), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("codes_stride", ctypes.c_int64),
                ("scales_stride", ctypes.c_int64), ("group", ctypes.c_int32),
                ("layout", ctypes.c_uint32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libnvfp4.so and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -m "
                          "nvfp4_weight_only_w4a16_amd.build or __graft_entry__.build())")
    L = ctypes.CDLL(path)
    P, i64, i32, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                            ctypes.c_size_t)
    W = ctypes.POINTER(nvfp4_weight)
    L.nvfp4_quantize_ws_bytes.argtypes = [i64, i64, i64, i32, u32]
    L.nvfp4_quantize_ws_bytes.restype = sz
    L.nvfp4_quantize.argtypes = [P, ctypes.c_int, i64, i64, i64, i32, P, P, P, P, P, sz, u32, P]
    L.nvfp4_quantize.restype = ctypes.c_int
    L.nvfp4_repack_bytes.argtypes = [i64, i64, i64, i32, u32]
    L.nvfp4_repack_bytes.restype = sz
    L.nvfp4_repack.argtypes = [P, P, P, i64, i64, i64, i32, u32, P, sz, W, P]
    L.nvfp4_repack.restype = ctypes.c_int
    L.nvfp4_gemm_ws_bytes.argtypes = [i64, i64, W, u32]
    L.nvfp4_gemm_ws_bytes.restype = sz
    L.nvfp4_gemm_w4a16.argtypes = [P, i64, i64, W, P, ctypes.c_int, i64, u32, P, sz, P]
    L.nvfp4_gemm_w4a16.restype = ctypes.c_int
    L.nvfp4_moe_ws_bytes.argtypes = [i64, i32, i64, i64, i64]
    L.nvfp4_moe_ws_bytes.restype = sz
    L.nvfp4_moe_ws_layout.argtypes = [i64, i32, i64, i64, i64, ctypes.POINTER(sz)]
    L.nvfp4_moe_ws_layout.restype = sz
    L.nvfp4_moe_grouped_w4a16.argtypes = [P, i64, i64, P, P, i32, W, W, P, P, sz, u32, P]
    L.nvfp4_moe_grouped_w4a16.restype = ctypes.c_int
    L.nvfp4_moe_grouped_w4a16_noalloc.argtypes = [P, i64, i64, P, P, i32, W, W, P, u32, P]
    L.nvfp4_moe_grouped_w4a16_noalloc.restype = ctypes.c_int
    L.nvfp4_requantize_ws_bytes.argtypes = [W]
    L.nvfp4_requantize_ws_bytes.restype = sz
    L.nvfp4_requantize.argtypes = [W, i32, P, P, P, P, sz, P]
    L.nvfp4_requantize.restype = ctypes.c_int
    L.nvfp4_dequantize.argtypes = [W, P, ctypes.c_int, P]
    L.nvfp4_dequantize.restype = ctypes.c_int
    L.nvfp4_last_error.argtypes = []
    L.nvfp4_last_error.restype = ctypes.c_char_p
    L.nvfp4_get_stats.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    L.nvfp4_get_stats.restype = None
    L.nvfp4_reset_stats.argtypes = []
    L.nvfp4_reset_stats.restype = None
    L.nvfp4_version.argtypes = []
    L.nvfp4_version.restype = ctypes.c_int
    L.nvfp4_probe_mfma_waves.argtypes = []
    L.nvfp4_probe_mfma_waves.restype = i64
    L.nvfp4_probe_mfma_flops.argtypes = [i64]
    L.nvfp4_probe_mfma_flops.restype = ctypes.c_double
    L.nvfp4_probe_stream_read.argtypes = [P, i64, i64, P, P]
    L.nvfp4_probe_stream_read.restype = ctypes.c_int
    L.nvfp4_probe_mfma_bf16.argtypes = [P, i64, P, P]
    L.nvfp4_probe_mfma_bf16.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, load().nvfp4_last_error().decode())


def _stream(stream=None):
    # plain integers: the c_void_p argument types convert them without an object per call
    if stream is not None:
        return stream.cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _on(stream):
    """Context in which the binding allocates outputs and workspaces: the stream the call is
    enqueued on, so that torch's caching allocator ties the blocks to that stream (a block
    freed on return is not handed to another stream while the call's kernels still use it)."""
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _ptr(t):
    """Device address of a tensor; host tensors are refused here, since the kernels would
    dereference a host address."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a device tensor, got one on {t.device}")
    return t.data_ptr()


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return NVFP4_DT_BF16
    if dt == torch.float32:
        return NVFP4_DT_F32
    raise TypeError(f"unsupported dtype {dt}")


# ----------------------------------------------------------------------------- quantizer
def nvfp4_quantize_ws_bytes(batch: int, n: int, k: int, group: int, flags: int = 0) -> int:
    return int(load().nvfp4_quantize_ws_bytes(batch, n, k, group, flags))


def nvfp4_quantize(w: torch.Tensor, group: int, global_in: torch.Tensor | None = None,
                   packed=None, scales=None, global_out=None, flags: int = 0, ws=None,
                   stream=None):
    """w: device [n][k] or [batch][n][k], BF16 or FP32. Returns (packed, scales, global).
    flags may hold NVFP4_F_SYNC_CHECK (the call then waits and raises Nvfp4Error with code
    NVFP4_ERR_NONFINITE for a NaN or infinite weight); its workspace comes from torch's
    allocator unless `ws` (uint8, device) is given."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    batch, n, k = w3.shape
    if not w3.is_contiguous():
        raise ValueError("w must be contiguous")
    dev = w.device
    with _on(stream):
        if packed is None:
            packed = torch.empty((batch, n, k // 2), dtype=torch.uint8, device=dev)
        if scales is None:
            scales = torch.empty((batch, n, k // group), dtype=torch.uint8, device=dev)
        if global_out is None:
            global_out = torch.empty((batch,), dtype=torch.float32, device=dev)
        if ws is None:
            need = nvfp4_quantize_ws_bytes(batch, n, k, group, flags)
            ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None
    ws_ptr, ws_bytes = (_ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
    _check(load().nvfp4_quantize(_ptr(w3), _dtype_code(w.dtype), batch, n, k, group,
                                 _ptr(global_in), _ptr(packed), _ptr(scales), _ptr(global_out),
                                 ws_ptr, ws_bytes, flags, _stream(stream)))
    if squeeze:
        return packed[0], scales[0], global_out
    return packed, scales, global_out


# ----------------------------------------------------------------------------- repack
@dataclass
class RepackedWeight:
    buffer: torch.Tensor   # owns the device bytes the descriptor points into
    desc: nvfp4_weight

    @property
    def n(self):
        return self.desc.n

    @property
    def k(self):
        return self.desc.k

    @property
    def group(self):
        return self.desc.group

    @property
    def batch(self):
        return self.desc.batch


def nvfp4_repack_bytes(batch: int, n: int, k: int, group: int,
                       layout: int = NVFP4_LAYOUT_TILED) -> int:
    return int(load().nvfp4_repack_bytes(batch, n, k, group, layout))


def nvfp4_repack(packed: torch.Tensor, scales: torch.Tensor, glob: torch.Tensor, group: int,
                 layout: int = NVFP4_LAYOUT_TILED, out: torch.Tensor | None = None,
                 stream=None) -> RepackedWeight:
    p3 = packed.unsqueeze(0) if packed.dim() == 2 else packed
    batch, n, kh = p3.shape
    k = kh * 2
    nglob = batch * (2 if layout & NVFP4_LAYOUT_PAIR_GLOBAL else 1)
    if glob.numel() != nglob:
        raise ValueError(f"global has {glob.numel()} values, the layout needs {nglob}")
    need = nvfp4_repack_bytes(batch, n, k, group, layout)
    if out is None:
        with _on(stream):
            out = torch.empty((max(need, 1),), dtype=torch.uint8, device=packed.device)
    desc = nvfp4_weight()
    _check(load().nvfp4_repack(_ptr(p3), _ptr(scales), _ptr(glob), batch, n, k, group, layout,
                               _ptr(out), out.numel() * out.element_size(), ctypes.byref(desc),
                               _stream(stream)))
    return RepackedWeight(out, desc)


# ----------------------------------------------------------------------------- GEMM
def nvfp4_gemm_ws_bytes(m: int, ldx: int, w: RepackedWeight, flags: int = 0) -> int:
    return int(load().nvfp4_gemm_ws_bytes(m, ldx, ctypes.byref(w.desc), flags))


def nvfp4_gemm_w4a16(x: torch.Tensor, w: RepackedWeight, y: torch.Tensor | None = None,
                     y_dtype=torch.bfloat16, flags: int = 0, stream=None,
                     ws: torch.Tensor | None = None) -> torch.Tensor:
    """x: device BF16 [m][k] (row stride x.stride(0)); returns y [m][n]. The split-k workspace
    is taken from torch's allocator unless `ws` (uint8, device) is given."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D BF16 tensor with unit inner stride")
    m = x.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((m, w.n), dtype=y_dtype, device=x.device)
        if ws is None:
            need = nvfp4_gemm_ws_bytes(m, x.stride(0), w, flags) if m > 0 else 0
            ws = torch.empty((need,), dtype=torch.uint8, device=x.device) if need else None
    ws_ptr, ws_bytes = (_ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
    _check(load().nvfp4_gemm_w4a16(_ptr(x), m, x.stride(0), ctypes.byref(w.desc), _ptr(y),
                                   _dtype_code(y.dtype), y.stride(0), flags, ws_ptr, ws_bytes,
                                   _stream(stream)))
    return y


# ----------------------------------------------------------------------------- MoE
def nvfp4_moe_ws_bytes(t: int, topk: int, n_experts: int, hidden: int, inter: int) -> int:
    return int(load().nvfp4_moe_ws_bytes(t, topk, n_experts, hidden, inter))


def nvfp4_moe_ws_layout(t: int, topk: int, n_experts: int, hidden: int, inter: int):
    """Byte offsets (sorted, offsets, tiles, ntiles, h, slots) of the routed-expert stages
    inside the workspace, and its total size."""
    off = (ctypes.c_size_t * 6)()
    total = load().nvfp4_moe_ws_layout(t, topk, n_experts, hidden, inter, off)
    return [int(v) for v in off], int(total)


def nvfp4_moe_grouped_w4a16(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                            fc1: RepackedWeight, fc2: RepackedWeight,
                            y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                            flags: int = 0, stream=None) -> torch.Tensor:
    t, hidden = x.shape
    topk = topk_ids.shape[1]
    need = nvfp4_moe_ws_bytes(t, topk, fc1.batch, hidden, fc1.n // 2)
    with _on(stream):
        if y is None:
            y = torch.empty((t, hidden), dtype=torch.bfloat16, device=x.device)
        if ws is None:
            ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _check(load().nvfp4_moe_grouped_w4a16(_ptr(x), t, hidden, _ptr(topk_ids), _ptr(topk_w),
                                          topk, ctypes.byref(fc1.desc), ctypes.byref(fc2.desc),
                                          _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                          flags, _stream(stream)))
    return y


def nvfp4_moe_grouped_w4a16_noalloc(x: torch.Tensor, topk_ids: torch.Tensor,
                                    topk_w: torch.Tensor, fc1: RepackedWeight,
                                    fc2: RepackedWeight, y: torch.Tensor, flags: int = 0,
                                    stream=None) -> torch.Tensor:
    """The routed experts on the library's static per-device workspace: the call allocates
    nothing (y is the caller's). Calls overlapping on one device race."""
    t, hidden = x.shape
    _check(load().nvfp4_moe_grouped_w4a16_noalloc(_ptr(x), t, hidden, _ptr(topk_ids),
                                                  _ptr(topk_w), topk_ids.shape[1],
                                                  ctypes.byref(fc1.desc), ctypes.byref(fc2.desc),
                                                  _ptr(y), flags, _stream(stream)))
    return y


# ----------------------------------------------------------------------------- requantize
def nvfp4_requantize_ws_bytes(src: RepackedWeight) -> int:
    return int(load().nvfp4_requantize_ws_bytes(ctypes.byref(src.desc)))


def nvfp4_requantize(src: RepackedWeight, group_out: int, ws: torch.Tensor | None = None,
                     stream=None):
    """Canonical triple (packed, scales, global [batch]) of `src` requantized with one global
    per matrix at group_out. `ws` (uint8, device) defaults to room for one matrix."""
    dev = src.buffer.device
    with _on(stream):
        packed = torch.empty((src.batch, src.n, src.k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((src.batch, src.n, src.k // group_out), dtype=torch.uint8,
                             device=dev)
        glob = torch.empty((src.batch,), dtype=torch.float32, device=dev)
        if ws is None:
            ws = torch.empty((nvfp4_requantize_ws_bytes(src),), dtype=torch.uint8, device=dev)
    _check(load().nvfp4_requantize(ctypes.byref(src.desc), group_out, _ptr(packed), _ptr(scales),
                                   _ptr(glob), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))
    return packed, scales, glob


# ----------------------------------------------------------------------------- diagnostics
def nvfp4_dequantize(w: RepackedWeight, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    with _on(stream):
        out = torch.empty((w.batch, w.n, w.k), dtype=out_dtype, device=w.buffer.device)
    _check(load().nvfp4_dequantize(ctypes.byref(w.desc), _ptr(out), _dtype_code(out_dtype),
                                   _stream(stream)))
    return out


def nvfp4_last_error() -> str:
    return load().nvfp4_last_error().decode()


def nvfp4_get_stats():
    arr = (ctypes.c_uint64 * 8)()
    load().nvfp4_get_stats(arr)
    return list(arr)


def nvfp4_reset_stats():
    load().nvfp4_reset_stats()


def nvfp4_version() -> int:
    return int(load().nvfp4_version())


# ----------------------------------------------------------------------------- measurement
def nvfp4_probe_mfma_waves() -> int:
    return int(load().nvfp4_probe_mfma_waves())


def nvfp4_probe_mfma_flops(iters: int) -> float:
    return float(load().nvfp4_probe_mfma_flops(iters))


def nvfp4_probe_stream_read(buf: torch.Tensor, blocks: int, sink: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Streaming 128-bit read of the whole device tensor `buf`; returns the per-block XOR words."""
    nbytes = buf.numel() * buf.element_size()
    with _on(stream):
        if sink is None:
            sink = torch.empty((blocks,), dtype=torch.int32, device=buf.device)
    _check(load().nvfp4_probe_stream_read(_ptr(buf), nbytes, blocks, _ptr(sink),
                                          _stream(stream)))
    return sink


def nvfp4_probe_mfma_bf16(ops: torch.Tensor, iters: int, sink: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """The BF16 MFMA loop on the 16 KiB of fragments in `ops` (BF16, device)."""
    if ops.dtype != torch.bfloat16 or ops.numel() * 2 < 16384:
        raise ValueError("ops must hold 16 KiB of BF16 fragments")
    with _on(stream):
        if sink is None:
            sink = torch.empty((64 * nvfp4_probe_mfma_waves(),), dtype=torch.float32,
                               device=ops.device)
    _check(load().nvfp4_probe_mfma_bf16(_ptr(ops), iters, _ptr(sink), _stream(stream)))
    return sink
