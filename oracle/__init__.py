"""Oracle: plain fp64 CPU reference of the MXFP4 routed-expert path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. The product
library (``mxfp4_packed_weight_amd``) never imports, links or calls it, and
shares no code with it.

ctypes binding of ``libk3oracle.so`` (plain C99, see ``k3oracle.h``): the
binding only marshals numpy arrays; every step is computed in C.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libk3oracle.so")
_lib = None


def build():
    """Compile libk3oracle.so in place (gcc, C99, fp64, OpenMP rows)."""
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Wshadow", "-fopenmp",
         "-fPIC", "-shared", "k3oracle.c", "-o", "libk3oracle.so", "-lm"], cwd=_HERE)


class Expert(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate_nib", "gate_sc", "up_nib", "up_sc", "down_nib", "down_sc")]


class Shared(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate", "up", "down")]


def _shared_table(shared):
    """shared: list of dicts gate/up/down -> bf16 arrays (uint16)."""
    table = (Shared * max(1, len(shared)))()
    keep = []
    for i, S in enumerate(shared):
        arrs = [_c(S[m], np.uint16) for m in ("gate", "up", "down")]
        table[i] = Shared(*[a.ctypes.data for a in arrs])
        keep.append(arrs)
    return table, keep


def _declare(L):
    i, d, vp = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    L.k3o_e2m1.restype = d
    L.k3o_e2m1.argtypes = [i]
    L.k3o_e8m0.restype = d
    L.k3o_e8m0.argtypes = [i]
    L.k3o_bf16_to_f64.restype = d
    L.k3o_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.k3o_f32_to_bf16.restype = ctypes.c_uint16
    L.k3o_f32_to_bf16.argtypes = [ctypes.c_float]
    L.k3o_mxfp4_gemv.argtypes = [vp, vp, i, i, i, vp, vp]
    L.k3o_mxfp4_dequant.argtypes = [vp, vp, i, i, i, vp]
    L.k3o_silu.restype = d
    L.k3o_silu.argtypes = [d]
    L.k3o_expert_swiglu.argtypes = [ctypes.POINTER(Expert), i, i, vp, vp, vp]
    L.k3o_router_logits.argtypes = [vp, vp, i, i, vp]
    L.k3o_topk.argtypes = [vp, vp, i, i, vp, vp]
    L.k3o_combine.argtypes = [vp, vp, i, i, vp]
    L.k3o_moe_layer.argtypes = [vp, vp, vp, i, i, i, i, vp, vp, vp]
    L.k3o_moe_from_logits.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp]
    L.k3o_permute.argtypes = [vp, i, i, i, vp, vp, vp, vp]
    L.k3o_mxfp4_quant.argtypes = [vp, i, i, vp, vp]
    L.k3o_mxfp4_matmul.argtypes = [vp, vp, i, vp, vp, i, i, vp]
    L.k3o_set_threads.argtypes = [i]
    L.k3o_shared_expert.argtypes = [ctypes.POINTER(Shared), i, i, vp, vp, vp]
    L.k3o_moe_layer_shared.argtypes = [vp, vp, vp, i, i, i, i, vp, i, i, vp, vp, vp]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = _declare(ctypes.CDLL(_SO))
    return _lib


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle returned {rc}")


def _expert_struct(E):
    arrs = [_c(a, np.uint8) for a in (E["gate"][0], E["gate"][1], E["up"][0],
                                      E["up"][1], E["down"][0], E["down"][1])]
    return Expert(*[a.ctypes.data for a in arrs]), arrs


def _expert_table(experts, n_experts):
    table = (Expert * n_experts)()
    keep = []
    for e, E in experts.items():
        s, arrs = _expert_struct(E)
        table[e] = s
        keep.append(arrs)
    return table, keep


class Oracle:
    """Bound oracle library. ``Oracle()`` uses libk3oracle.so; tests may pass
    the path of another build of k3oracle.c (e.g. one with a planted
    mistake) to check that the pins catch it."""

    def __init__(self, path=None):
        self.L = lib() if path is None else _declare(ctypes.CDLL(path))

    def set_threads(self, n):
        self.L.k3o_set_threads(int(n))

    def e2m1(self, code):
        return self.L.k3o_e2m1(int(code))

    def e8m0(self, e):
        return self.L.k3o_e8m0(int(e))

    def bf16_to_f64(self, a):
        a = _c(a, np.uint16)
        f = self.L.k3o_bf16_to_f64
        return np.array([f(int(v)) for v in a.ravel()], np.float64).reshape(a.shape)

    def f32_to_bf16(self, a):
        a = _c(a, np.float32)
        f = self.L.k3o_f32_to_bf16
        return np.array([f(float(v)) for v in a.ravel()], np.uint16).reshape(a.shape)

    def gemv(self, nib, sc, x, group=32):
        nib, sc = _c(nib, np.uint8), _c(sc, np.uint8)
        rows, cols = nib.shape[0], nib.shape[1] * 2
        x = _c(x, np.float64)
        y = np.zeros(rows, np.float64)
        _check(self.L.k3o_mxfp4_gemv(_p(nib), _p(sc), rows, cols, group, _p(x), _p(y)), "gemv")
        return y

    def dequant(self, nib, sc, group=32):
        nib, sc = _c(nib, np.uint8), _c(sc, np.uint8)
        rows, cols = nib.shape[0], nib.shape[1] * 2
        W = np.zeros((rows, cols), np.float64)
        _check(self.L.k3o_mxfp4_dequant(_p(nib), _p(sc), rows, cols, group, _p(W)), "dequant")
        return W

    def silu(self, v):
        return self.L.k3o_silu(float(v))

    def expert_swiglu(self, E, x):
        """Returns (y [hidden], h [inter]) in fp64."""
        inter, hidden = E["gate"][0].shape[0], E["gate"][0].shape[1] * 2
        s, keep = _expert_struct(E)
        x = _c(x, np.float64)
        y = np.zeros(hidden, np.float64)
        h = np.zeros(inter, np.float64)
        _check(self.L.k3o_expert_swiglu(ctypes.byref(s), hidden, inter, _p(x), _p(h), _p(y)),
               "expert")
        del keep
        return y, h

    def router_logits(self, x_bf16, R_bf16):
        x, R = _c(x_bf16, np.uint16), _c(R_bf16, np.uint16)
        n, hidden = R.shape
        out = np.zeros(n, np.float64)
        _check(self.L.k3o_router_logits(_p(x), _p(R), n, hidden, _p(out)), "router")
        return out

    def topk(self, logits, k, bias=None):
        logits = _c(logits, np.float64)
        b = None if bias is None else _c(bias, np.float64)
        idx = np.zeros(k, np.int32)
        w = np.zeros(k, np.float64)
        _check(self.L.k3o_topk(_p(logits), _p(b), logits.size, k, _p(idx), _p(w)), "topk")
        return idx, w

    def combine(self, w, ye):
        w, ye = _c(w, np.float64), _c(ye, np.float64)
        k, hidden = ye.shape
        y = np.zeros(hidden, np.float64)
        _check(self.L.k3o_combine(_p(w), _p(ye), k, hidden, _p(y)), "combine")
        return y

    def moe_layer(self, x_bf16, R_bf16, experts, k, hidden, inter):
        """experts: dict expert_id -> expert dict (only selected ones needed)."""
        x, R = _c(x_bf16, np.uint16), _c(R_bf16, np.uint16)
        n = R.shape[0]
        table, keep = _expert_table(experts, n)
        y = np.zeros(hidden, np.float64)
        idx = np.zeros(k, np.int32)
        w = np.zeros(k, np.float64)
        _check(self.L.k3o_moe_layer(_p(x), _p(R), ctypes.cast(table, ctypes.c_void_p), n,
                                    hidden, inter, k, _p(y), _p(idx), _p(w)), "moe_layer")
        del keep
        return y, idx, w

    def shared_expert(self, S, x):
        """S: dict gate/up [inter][hidden], down [hidden][inter] bf16 (uint16).
        Returns (y [hidden], h [inter]) in fp64."""
        inter, hidden = S["gate"].shape
        table, keep = _shared_table([S])
        x = _c(x, np.float64)
        y = np.zeros(hidden, np.float64)
        h = np.zeros(inter, np.float64)
        _check(self.L.k3o_shared_expert(table, hidden, inter, _p(x), _p(h), _p(y)), "shared")
        del keep
        return y, h

    def moe_layer_shared(self, x_bf16, R_bf16, experts, k, hidden, inter, shared):
        x, R = _c(x_bf16, np.uint16), _c(R_bf16, np.uint16)
        n = R.shape[0]
        table, keep = _expert_table(experts, n)
        stab, skeep = _shared_table(shared)
        inter_s = shared[0]["gate"].shape[0] if shared else 0
        y = np.zeros(hidden, np.float64)
        idx = np.zeros(k, np.int32)
        w = np.zeros(k, np.float64)
        _check(self.L.k3o_moe_layer_shared(_p(x), _p(R), ctypes.cast(table, ctypes.c_void_p),
                                           n, hidden, inter, k,
                                           ctypes.cast(stab, ctypes.c_void_p), len(shared),
                                           inter_s, _p(y), _p(idx), _p(w)), "moe_layer_shared")
        del keep, skeep
        return y, idx, w

    def moe_from_logits(self, X_bf16, logits, experts, k, hidden, inter, bias=None):
        X = _c(X_bf16, np.uint16)
        L = _c(logits, np.float64)
        T, n = L.shape
        b = None if bias is None else _c(bias, np.float64)
        table, keep = _expert_table(experts, n)
        Y = np.zeros((T, hidden), np.float64)
        idx = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float64)
        _check(self.L.k3o_moe_from_logits(_p(X), _p(L), _p(b),
                                          ctypes.cast(table, ctypes.c_void_p), T, n, hidden,
                                          inter, k, _p(Y), _p(idx), _p(w)), "moe_from_logits")
        del keep
        return Y, idx, w

    def permute(self, idx, n_experts):
        idx = _c(idx, np.int32)
        T, k = idx.shape
        counts = np.zeros(n_experts, np.int32)
        offsets = np.zeros(n_experts, np.int32)
        pt = np.zeros(T * k, np.int32)
        ps = np.zeros(T * k, np.int32)
        _check(self.L.k3o_permute(_p(idx), T, k, n_experts, _p(counts), _p(offsets), _p(pt),
                                  _p(ps)), "permute")
        return counts, offsets, pt, ps

    def mxfp4_quant(self, v):
        v = _c(v, np.float64)
        if v.ndim == 1:
            v = v.reshape(1, -1)
        rows, cols = v.shape
        nib = np.zeros((rows, cols // 2), np.uint8)
        sc = np.zeros((rows, cols // 32), np.uint8)
        _check(self.L.k3o_mxfp4_quant(_p(v), rows, cols, _p(nib), _p(sc)), "quant")
        return nib, sc

    def mxfp4_matmul(self, a_nib, a_sc, w_nib, w_sc):
        a_nib, a_sc = _c(a_nib, np.uint8), _c(a_sc, np.uint8)
        w_nib, w_sc = _c(w_nib, np.uint8), _c(w_sc, np.uint8)
        M, K = a_nib.shape[0], a_nib.shape[1] * 2
        N = w_nib.shape[0]
        C = np.zeros((M, N), np.float64)
        _check(self.L.k3o_mxfp4_matmul(_p(a_nib), _p(a_sc), M, _p(w_nib), _p(w_sc), N, K,
                                       _p(C)), "matmul")
        return C


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # Module-level convenience: oracle.gemv(...) == Oracle().gemv(...).
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
