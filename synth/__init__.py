"""Seeded synthetic inputs (Philox4x32-10 + Box-Muller) for the offloaded MoE step.

Only input generation lives here: expert weight records, router weights and
biases, and token hidden states.  Both the CPU oracle and the GPU library read
the bytes these functions write; this module contains none of the layer's own
arithmetic.  Every value is a pure function of (seed, stream, index).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "_build", "libsynth.so")
_lib = None

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3


def build():
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i32, f32, f64, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
        L.syn_philox4x32_10.argtypes = [vp, vp, vp]
        L.syn_normal_f32.argtypes = [u64, u64, u64, u64, f32, vp]
        L.syn_normal_bf16.argtypes = [u64, u64, u64, u64, f32, vp]
        L.syn_encode_bf16.argtypes = [vp, u64, vp]
        L.syn_encode_e4m3.argtypes = [vp, u64, vp]
        L.syn_record_bytes.argtypes = [i32, i32, i32]
        L.syn_record_bytes.restype = u64
        L.syn_fill_records.argtypes = [u64, i32, i32, i32, i32, i32, i32, f32, vp, u64, i32]
        L.syn_router.argtypes = [u64, i32, i32, i32, i32, f32, f64, vp, vp]
        L.syn_tokens.argtypes = [u64, u64, i32, i32, i32, f64, i32, vp]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data if isinstance(a, np.ndarray) else int(a))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().syn_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal_f32(seed, stream, first, n, sigma=1.0):
    out = np.empty(n, dtype=np.float32)
    lib().syn_normal_f32(seed, stream, first, n, sigma, _ptr(out))
    return out


def encode_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().syn_encode_bf16(_ptr(x), x.size, _ptr(out))
    return out


def encode_e4m3(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().syn_encode_e4m3(_ptr(x), x.size, _ptr(out))
    return out


def record_bytes(wdt, H, F):
    return int(lib().syn_record_bytes(wdt, H, F))


def fill_records(seed, layer, e0, count, H, F, wdt, dst_ptr, stride, sigma=0.02, shared=False):
    """Write `count` expert records (experts e0..) of `layer` at dst_ptr (host memory)."""
    lib().syn_fill_records(seed, layer, e0, count, H, F, wdt, sigma, _ptr(dst_ptr), stride, 1 if shared else 0)


def records(seed, layer, E, H, F, wdt, stride=None, sigma=0.02, shared=False):
    """Expert records of a layer as a numpy uint8 array [E, stride]."""
    rb = record_bytes(wdt, H, F)
    stride = rb if stride is None else stride
    out = np.zeros((E, stride), dtype=np.uint8)
    fill_records(seed, layer, 0, E, H, F, wdt, out, stride, sigma, shared)
    return out


def router(seed, layer, E, H, wdt, zipf_s=1.2, sigma=0.02):
    """Router weights [E, H] (float32 or bf16 bits as uint16) and bias [E] float32."""
    w = np.empty((E, H), dtype=np.float32 if wdt == F32 else np.uint16)
    b = np.empty(E, dtype=np.float32)
    lib().syn_router(seed, layer, E, H, wdt, sigma, float(zipf_s), _ptr(w), _ptr(b))
    return w, b


def tokens(seed, tag, T, H, steps, rho, adt):
    """Hidden states [steps, T, H]: AR(1) per sequence when rho > 0, else i.i.d. N(0,1)."""
    out = np.empty((steps, T, H), dtype=np.float32 if adt == F32 else np.uint16)
    lib().syn_tokens(seed, tag, T, H, steps, float(rho), adt, _ptr(out))
    return out
