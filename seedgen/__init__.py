"""Seeded synthetic attention inputs, shared by the fp64 oracle and the GPU library.

This package produces input bytes only (i.i.d. N(0,1) values rounded to bf16, and seeded
row samples); it contains none of the attention arithmetic. The generator definition is in
``seedgen.c``: counter-based splitmix64 feeding Box-Muller, fp64 -> fp32 -> bf16 with
round-to-nearest-even, so any element can be regenerated from (seed, tensor id, index).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "seedgen.c")
_LIB_PATH = os.path.join(_HERE, "libseedgen.so")

# Stream ids of the generator: one independent stream per tensor.
TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4, "sample": 5}

_lib = None


def build() -> str:
    """Compile libseedgen.so in-tree with gcc (host code only)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, u32, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32
    lib.seedgen_sm64.restype = u64
    lib.seedgen_sm64.argtypes = [u64]
    lib.seedgen_stream_key.restype = u64
    lib.seedgen_stream_key.argtypes = [u64, u32]
    lib.seedgen_f32_to_bf16.restype = ctypes.c_uint16
    lib.seedgen_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.seedgen_normal_f64.restype = ctypes.c_double
    lib.seedgen_normal_f64.argtypes = [u64, u64]
    lib.seedgen_normal_bf16.restype = ctypes.c_int
    lib.seedgen_normal_bf16.argtypes = [u64, u32, u64, u64, ctypes.c_void_p, ctypes.c_int]
    lib.seedgen_f64_to_e4m3.restype = ctypes.c_uint8
    lib.seedgen_f64_to_e4m3.argtypes = [ctypes.c_double]
    lib.seedgen_normal_e4m3.restype = ctypes.c_int
    lib.seedgen_normal_e4m3.argtypes = [u64, u32, u64, u64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
    lib.seedgen_sample_rows.restype = ctypes.c_int
    lib.seedgen_sample_rows.argtypes = [u64, u64, i32, i32, ctypes.c_void_p]
    _lib = lib
    return lib


def host_threads() -> int:
    """Threads for host-side generation: the process affinity mask, capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def config_seed(index: int) -> int:
    """Seed of workload number ``index`` (0-based): 0x5EED0000 + index + 1."""
    return 0x5EED0000 + index + 1


def sm64(x: int) -> int:
    return int(_load().seedgen_sm64(x & 0xFFFFFFFFFFFFFFFF))


def stream_key(seed: int, tensor: str | int) -> int:
    t = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    return int(_load().seedgen_stream_key(seed & 0xFFFFFFFFFFFFFFFF, t))


def f32_to_bf16_bits(x: float) -> int:
    return int(_load().seedgen_f32_to_bf16(float(x)))


def normal_bf16(seed: int, tensor: str | int, shape, start: int = 0, threads: int | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of the seeded N(0,1) stream, row-major over ``shape``."""
    t = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    shape = tuple(int(s) for s in shape)
    count = int(np.prod(shape)) if shape else 1
    out = np.empty(count, dtype=np.uint16)
    if count:
        _load().seedgen_normal_bf16(seed & 0xFFFFFFFFFFFFFFFF, t, start, count,
                                    out.ctypes.data, threads or host_threads())
    return out.reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (bit shift, no rounding)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def f64_to_e4m3(x: float) -> int:
    """OCP FP8 E4M3FN code of x: round to nearest even, saturating to +-448 (seedgen.c)."""
    return int(_load().seedgen_f64_to_e4m3(float(x)))


def normal_e4m3(seed: int, tensor: str | int, shape, inv_scale: float, start: int = 0,
                threads: int | None = None) -> np.ndarray:
    """FP8 E4M3FN codes (uint8) of the seeded N(0,1) stream times ``inv_scale``; the values
    they stand for are code_value * (1 / inv_scale)."""
    t = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    shape = tuple(int(s) for s in shape)
    count = int(np.prod(shape)) if shape else 1
    out = np.empty(count, dtype=np.uint8)
    if count:
        _load().seedgen_normal_e4m3(seed & 0xFFFFFFFFFFFFFFFF, t, start, count, float(inv_scale),
                                    out.ctypes.data, threads or host_threads())
    return out.reshape(shape)


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes, from the format's definition (bias 7, subnormals
    m/8 * 2^-6, 0x7F and 0xFF NaN)."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sgn = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sgn * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = sgn * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_VALUES = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 values of FP8 E4M3FN codes."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def fp8_attention_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, scale: float = 1.0 / 32):
    """Q [B,Hq,N,d], K/V [B,Hkv,N,d] as FP8 E4M3FN codes of the seeded N(0,1) streams divided by
    ``scale`` (each tensor stands for codes * scale)."""
    inv = 1.0 / scale
    return (normal_e4m3(seed, "q", (B, Hq, N, d), inv), normal_e4m3(seed, "k", (B, Hkv, N, d), inv),
            normal_e4m3(seed, "v", (B, Hkv, N, d), inv))


def sample_rows(seed: int, slice_index: int, N: int, count: int) -> np.ndarray:
    """Seeded sorted row sample of one (batch, head) slice (see seedgen.c)."""
    out = np.empty(max(count, 0) if count < N else N, dtype=np.int32)
    n = _load().seedgen_sample_rows(seed & 0xFFFFFFFFFFFFFFFF, slice_index, N, count, out.ctypes.data)
    return out[:n]


def sample_rows_all(seed: int, nslices: int, N: int, count: int) -> np.ndarray:
    """[nslices, k] row samples, k = min(count, N), one seeded sample per slice."""
    k = min(count, N)
    out = np.empty((nslices, k), dtype=np.int32)
    for s in range(nslices):
        r = sample_rows(seed, s, N, count)
        assert r.shape[0] == k
        out[s] = r
    return out


def attention_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, with_do: bool = False):
    """Q [B,Hq,N,d], K/V [B,Hkv,N,d] (and dO [B,Hq,N,d]) as bf16 bit patterns."""
    q = normal_bf16(seed, "q", (B, Hq, N, d))
    k = normal_bf16(seed, "k", (B, Hkv, N, d))
    v = normal_bf16(seed, "v", (B, Hkv, N, d))
    if with_do:
        return q, k, v, normal_bf16(seed, "do", (B, Hq, N, d))
    return q, k, v
