"""Loads (building on first use) the C draw kernels of gen.c."""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth_gen.so")
_lib = None


def build(force=False):
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        l = ctypes.CDLL(_LIB)
        l.synth_normal_f64.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        l.synth_normal_f64.restype = None
        l.synth_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        l.synth_f32_to_bf16.restype = None
        _lib = l
    return _lib


def normal_f64(seed, n, std=1.0):
    out = np.empty(n, dtype=np.float64)
    if n:
        lib().synth_normal_f64(seed, n, float(std), out.ctypes.data)
    return out


def f32_to_bf16(x):
    f = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    if f.size:
        lib().synth_f32_to_bf16(f.ctypes.data, f.size, out.ctypes.data)
    return out
