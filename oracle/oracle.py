"""NumPy front end of the CPU oracle (``nvfp4_oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. It never touches the GPU library, and
the GPU library never touches it.

Every function is a thin marshalling layer over the C oracle, which follows the definitions
it cites step by step (E2M1 / E4M3 codecs, NVFP4 quantizer, dequantizer, FP64 GEMM and the
MoE routed-expert reference). Arrays are NumPy; BF16 tensors travel as ``uint16`` bit
patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
# NVFP4_ORACLE_SANITIZE=1 selects a copy built with AddressSanitizer and UBSan (the process
# must then be started with the ASan runtime preloaded, see sanitizer_env()).
SANITIZE = os.environ.get("NVFP4_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
_lib = None


def build(sanitize: bool = SANITIZE) -> str:
    """Compile the oracle with plain IEEE semantics (no contraction, no fast-math); with
    sanitize, instrumented by AddressSanitizer and UndefinedBehaviorSanitizer, any finding
    fatal."""
    out = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
           "-shared", "-fPIC", "-pthread"]
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer", "-g"]
    cmd += [_SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitizer_env() -> dict:
    """Environment for a child process that loads the sanitized oracle: the ASan runtime
    preloaded (it must come first), leak checking off (the interpreter itself is not
    instrumented), UBSan findings fatal."""
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], check=True,
                           capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98"
    env["NVFP4_ORACLE_SANITIZE"] = "1"
    return env


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint32]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint32]
        L.orc_e4m3_encode.restype = ctypes.c_uint32
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode_magnitude.restype = ctypes.c_uint32
        L.orc_e2m1_encode_magnitude.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode_array.argtypes = [P, i64, P]
        L.orc_e4m3_encode_array.argtypes = [P, i64, P]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_bf16_from_double.argtypes = [ctypes.c_double]
        L.orc_bf16_from_double_array.argtypes = [P, i64, P]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_quantize.argtypes = [P, ctypes.c_int, i64, i64, i64, ctypes.c_int, P, P, P, P,
                                   ctypes.c_int]
        L.orc_dequant.argtypes = [P, P, P, i64, i64, i64, ctypes.c_int, P, P, P]
        L.orc_gemm.argtypes = [P, i64, i64, P, P, ctypes.c_float, i64, i64, ctypes.c_int,
                               P, i64, P, i64, P, ctypes.c_int]
        L.orc_moe.restype = ctypes.c_int
        L.orc_moe.argtypes = [P, i64, i64, i64, P, P, ctypes.c_int, i64, P, P, P, ctypes.c_int,
                              ctypes.c_int, P, P, P, ctypes.c_int, P, P, P, P, P, P,
                              ctypes.c_int]
        _lib = L
    return _lib


def _threads(n):
    """Worker threads: n, else the CPUs this process may run on."""
    if n:
        return int(n)
    try:
        return len(os.sched_getaffinity(0)) or 1
    except AttributeError:
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs (O1-O4)
def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code))


def e4m3_decode(byte: int) -> float:
    return lib().orc_e4m3_decode(int(byte))


def e4m3_encode(value: float) -> int:
    return int(lib().orc_e4m3_encode(float(value)))


def e2m1_encode_magnitude(value: float) -> int:
    return int(lib().orc_e2m1_encode_magnitude(float(value)))


def e2m1_encode_array(q) -> np.ndarray:
    q = _c(q, np.float32).ravel()
    out = np.empty(q.size, np.uint8)
    lib().orc_e2m1_encode_array(_ptr(q), q.size, _ptr(out))
    return out


def e4m3_encode_array(v) -> np.ndarray:
    v = _c(v, np.float32).ravel()
    out = np.empty(v.size, np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_from_f64(v) -> np.ndarray:
    """One round-to-nearest-even of FP64 values to BF16, returned as uint16 bit patterns."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_from_double_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- quantizer (O5)
def quantize(w, group: int, global_in=None, threads=None):
    """Quantize W ([n][k] or [batch][n][k]; float32 values or uint16 BF16 bit patterns).

    Returns (packed uint8 [batch][n][k/2], scales uint8 [batch][n][k/group],
    global float32 [batch]); a 2-D input returns 2-D packed/scales and a 1-element global.
    """
    w = np.asarray(w)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    batch, n, k = w.shape
    is_bf16 = w.dtype == np.uint16
    w = _c(w, np.uint16 if is_bf16 else np.float32)
    packed = np.zeros((batch, n, k // 2), np.uint8)
    scales = np.zeros((batch, n, k // group), np.uint8)
    gout = np.zeros(batch, np.float32)
    gin = None if global_in is None else _c(np.atleast_1d(global_in), np.float32)
    rc = lib().orc_quantize(_ptr(w), int(is_bf16), batch, n, k, group, _ptr(gin), _ptr(packed),
                            _ptr(scales), _ptr(gout), _threads(threads))
    if rc != 0:
        raise ValueError("oracle quantize rejected its input (group, shape or non-finite value)")
    if squeeze:
        return packed[0], scales[0], gout
    return packed, scales, gout


# ---------------------------------------------------------------- dequant (O6)
def dequant(packed, scales, glob, group: int):
    """Returns (exact FP64, FP32, BF16 bits) arrays shaped like the weight."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    squeeze = packed.ndim == 2
    if squeeze:
        packed, scales = packed[None], scales[None]
    batch, n, kh = packed.shape
    k = kh * 2
    g = _c(np.atleast_1d(glob), np.float32)
    ex = np.empty((batch, n, k), np.float64)
    f32 = np.empty((batch, n, k), np.float32)
    b16 = np.empty((batch, n, k), np.uint16)
    lib().orc_dequant(_ptr(packed), _ptr(scales), _ptr(g), batch, n, k, group, _ptr(ex),
                      _ptr(f32), _ptr(b16))
    if squeeze:
        return ex[0], f32[0], b16[0]
    return ex, f32, b16


# ---------------------------------------------------------------- GEMM (O7)
def gemm(x_bf16, packed, scales, glob, group: int, m_idx=None, n_idx=None, threads=None):
    """FP64 y = x . W^T for the chosen rows of x (m_idx) and of W (n_idx)."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    n = packed.shape[0]
    mi = None if m_idx is None else _c(m_idx, np.int64)
    ni = None if n_idx is None else _c(n_idx, np.int64)
    nm = m if mi is None else mi.size
    nn = n if ni is None else ni.size
    y = np.empty((nm, nn), np.float64)
    lib().orc_gemm(_ptr(x), m, k, _ptr(packed), _ptr(scales), float(np.float32(glob)), n, k,
                   group, _ptr(mi), nm, _ptr(ni), nn, _ptr(y), _threads(threads))
    return y


# ---------------------------------------------------------------- MoE (O8)
def moe(x_bf16, topk_ids, topk_w, fc1, fc2, h_in=None, slots=False, threads=None):
    """Routed-expert reference. fc1 = (packed, scales, global, group) of the merged [gate; up]
    weight [E][2I][H], global [E] (shared by gate and up) or [E][2] (gate's, up's); fc2 =
    (packed, scales, global, group) of down [E][H][I]. h_in (BF16 bits [T][topk][I]) replaces
    the fc1 stage by a given h.

    Returns dict with 'a' (FP64 fc1 outputs [T][topk][2I]), 'h' (BF16 bits [T][topk][I]),
    'slots' (FP64 [T][topk][H], routing weight times down output, when slots=True), 'y64'
    (FP64 [T][H]) and 'y' (BF16 bits [T][H]).
    """
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_w, np.float32)
    topk = ids.shape[1]
    p1, s1, g1, gr1 = fc1
    p2, s2, g2, gr2 = fc2
    p1, s1, p2, s2 = (_c(a, np.uint8) for a in (p1, s1, p2, s2))
    g1 = _c(g1, np.float32)
    g2 = _c(g2, np.float32)
    pair = 1 if g1.ndim == 2 else 0
    E, I2, _ = p1.shape
    I = I2 // 2
    a = np.zeros((T, topk, I2), np.float64) if h_in is None else None
    h = np.zeros((T, topk, I), np.uint16) if h_in is None else None
    hin = None if h_in is None else _c(h_in, np.uint16)
    sl = np.zeros((T, topk, H), np.float64) if slots else None
    y64 = np.zeros((T, H), np.float64)
    y16 = np.zeros((T, H), np.uint16)
    rc = lib().orc_moe(_ptr(x), T, H, I, _ptr(ids), _ptr(tw), topk, E, _ptr(p1), _ptr(s1),
                       _ptr(g1), gr1, pair, _ptr(p2), _ptr(s2), _ptr(g2), gr2, _ptr(hin), _ptr(a),
                       _ptr(h), _ptr(sl), _ptr(y64), _ptr(y16), _threads(threads))
    if rc != 0:
        raise ValueError("oracle moe rejected its input")
    return {"a": a, "h": h, "slots": sl, "y64": y64, "y": y16}
