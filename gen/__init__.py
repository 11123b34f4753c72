"""Seeded synthetic inputs shared by the oracle side and the GPU side.

ctypes binding of ``libk3gen.so`` (plain C, see ``k3gen.h``). The module only
draws random numbers and lays them out as the canonical tensors of the
workloads; it holds none of the method's arithmetic.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libk3gen.so")
_lib = None

KIND_MATRIX, KIND_EXPERT, KIND_ROUTER, KIND_TOKENS, KIND_LOGITS, KIND_BIAS = 1, 2, 3, 4, 5, 6
KIND_SHARED = 7  # shared experts' bf16 weights


def build():
    """Compile libk3gen.so in place (gcc, C99, OpenMP)."""
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fopenmp", "-fPIC",
         "-shared", "k3gen.c", "-o", "libk3gen.so", "-lm"], cwd=_HERE)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, u32, i32, dbl, vp, sz = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t)
        L.k3g_mix64.restype = u64
        L.k3g_mix64.argtypes = [u64]
        L.k3g_splitmix64_next.restype = u64
        L.k3g_splitmix64_next.argtypes = [ctypes.POINTER(u64)]
        L.k3g_draw.restype = u64
        L.k3g_draw.argtypes = [u64, u64]
        L.k3g_key.restype = u64
        L.k3g_key.argtypes = [u64, u32, u32, u32, u32]
        L.k3g_bytes.argtypes = [u64, vp, sz]
        L.k3g_uniform_u8.argtypes = [u64, i32, i32, vp, sz]
        L.k3g_normal_f32.argtypes = [u64, dbl, dbl, vp, sz]
        L.k3g_normal_bf16.argtypes = [u64, dbl, dbl, vp, sz]
        L.k3g_uniform_f32.argtypes = [u64, vp, sz]
        L.k3g_f32_to_bf16.restype = ctypes.c_uint16
        L.k3g_f32_to_bf16.argtypes = [ctypes.c_float]
        L.k3g_mxfp4_matrix.argtypes = [u64, u32, u32, u32, u32, i32, i32, i32, i32, vp, vp]
        L.k3g_expert.argtypes = [u64, u32, u32, i32, i32, i32, i32] + [vp] * 6
        L.k3g_zipf_logits.argtypes = [u64, u32, u32, i32, i32, dbl, vp]
        L.k3g_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def set_threads(n):
    lib().k3g_set_threads(int(n))


def key(seed, cfg, kind, a=0, b=0):
    return lib().k3g_key(seed, cfg, kind, a, b)


def draws(k, n):
    """First n values of the counter-based SplitMix64 stream `k` (uint64)."""
    return np.array([lib().k3g_draw(k, i) for i in range(n)], dtype=np.uint64)


def mxfp4_matrix(seed, cfg, rows, cols, elo=120, ehi=134, kind=KIND_MATRIX, a=0, b=0):
    """Canonical MXFP4 matrix: (nib uint8[rows][cols/2], sc uint8[rows][cols/32])."""
    nib = np.empty((rows, cols // 2), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    lib().k3g_mxfp4_matrix(seed, cfg, kind, a, b, rows, cols, elo, ehi, _p(nib), _p(sc))
    return nib, sc


def expert(seed, cfg, e, hidden, inter, elo=120, ehi=134):
    """One routed expert as canonical MXFP4: dict gate/up/down -> (nib, sc)."""
    g = (np.empty((inter, hidden // 2), np.uint8), np.empty((inter, hidden // 32), np.uint8))
    u = (np.empty((inter, hidden // 2), np.uint8), np.empty((inter, hidden // 32), np.uint8))
    d = (np.empty((hidden, inter // 2), np.uint8), np.empty((hidden, inter // 32), np.uint8))
    lib().k3g_expert(seed, cfg, e, hidden, inter, elo, ehi,
                     _p(g[0]), _p(g[1]), _p(u[0]), _p(u[1]), _p(d[0]), _p(d[1]))
    return {"gate": g, "up": u, "down": d}


def normal_bf16(k, n, mu=0.0, sigma=1.0):
    out = np.empty(n, np.uint16)
    lib().k3g_normal_bf16(k, mu, sigma, _p(out), n)
    return out


def normal_f32(k, n, mu=0.0, sigma=1.0):
    out = np.empty(n, np.float32)
    lib().k3g_normal_f32(k, mu, sigma, _p(out), n)
    return out


def uniform_f32(k, n):
    out = np.empty(n, np.float32)
    lib().k3g_uniform_f32(k, _p(out), n)
    return out


def uniform_u8(k, n, lo, hi):
    out = np.empty(n, np.uint8)
    lib().k3g_uniform_u8(k, lo, hi, _p(out), n)
    return out


def random_bytes(k, n):
    out = np.empty(n, np.uint8)
    lib().k3g_bytes(k, _p(out), n)
    return out


def zipf_logits(seed, cfg, T, n, s=1.1, batch=0):
    out = np.empty((T, n), np.float32)
    lib().k3g_zipf_logits(seed, cfg, batch, T, n, s, _p(out))
    return out


def f32_to_bf16(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return np.array([lib().k3g_f32_to_bf16(float(v)) for v in a.ravel()],
                    dtype=np.uint16).reshape(a.shape)
