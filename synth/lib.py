"""ctypes wrapper of the counter-based normal generator in ``csrc/synth.c``."""
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth.c")
_SO = os.path.join(_HERE, "libsynth.so")
_LOCK = threading.Lock()
_LIB = None

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def build(force=False):
    """Compile libsynth.so with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(_SO):
                build()
            L = ctypes.CDLL(_SO)
            u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            L.synth_mix64.argtypes = [u64]
            L.synth_mix64.restype = u64
            L.synth_normal_f64.argtypes = [u64, u64, i64, vp]
            L.synth_normal_f32.argtypes = [u64, u64, i64, dbl, vp]
            L.synth_normal_bf16.argtypes = [u64, u64, i64, dbl, vp]
            L.synth_blocks_bf16.argtypes = [vp, i64, i64, dbl, vp]
            L.synth_blocks_f32.argtypes = [vp, i64, i64, dbl, vp]
            _LIB = L
    return _LIB


def mix64(z):
    """SplitMix64 finaliser (Python reference of the C one)."""
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def key_of(*tags):
    """Stream key derived from a tuple of non-negative integer tags."""
    k = 0x5EED5EED5EED5EED
    for t in tags:
        k = mix64((k ^ (int(t) & M64)) + GOLDEN)
    return k


def normal_f64(key, count, start=0):
    out = np.empty(int(count), np.float64)
    _lib().synth_normal_f64(key, start, out.size, out.ctypes.data)
    return out


def normal_f32(key, count, sigma=1.0, start=0):
    out = np.empty(int(count), np.float32)
    _lib().synth_normal_f32(key, start, out.size, float(sigma), out.ctypes.data)
    return out


def normal_bf16(key, count, sigma=1.0, start=0):
    """bf16 bit patterns (uint16)."""
    out = np.empty(int(count), np.uint16)
    _lib().synth_normal_bf16(key, start, out.size, float(sigma), out.ctypes.data)
    return out


def blocks(keys, block, sigma, dtype, out=None):
    """Concatenation of elements [0, block) of each stream in `keys`."""
    keys = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
    npdt = np.uint16 if dtype == "bf16" else np.float32
    if out is None:
        out = np.empty(keys.size * int(block), npdt)
    assert out.dtype == npdt and out.size == keys.size * int(block) and out.flags.c_contiguous
    fn = _lib().synth_blocks_bf16 if dtype == "bf16" else _lib().synth_blocks_f32
    fn(keys.ctypes.data, keys.size, int(block), float(sigma), out.ctypes.data)
    return out


def bf16_to_f32(u16):
    """Exact decode of bf16 bit patterns to fp32."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f32):
    """Round-to-nearest-even of fp32 values to bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
