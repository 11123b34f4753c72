"""Python binding of libk3moe.so, the MI355X (gfx950) MXFP4 routed-expert path.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in ``include/k3moe.h``. Functions carry the C names. Device
buffers are torch tensors on a ROCm device (torch provides memory and
streams, nothing else); host buffers of the ``*_host`` calls are numpy arrays.

The library must be built first (``python -m mxfp4_packed_weight_amd._build``
or ``__graft_entry__.build()``); importing works without it, but every call
raises ``K3LibraryMissing`` rather than falling back to anything else.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3moe.so")
_lib = None

K3_OK, K3_ERR_ARG, K3_ERR_CONFIG, K3_ERR_MEMORY, K3_ERR_DEVICE = 0, 1, 2, 3, 4
K3_MAX_EXPERTS, K3_MAX_TOPK, K3_MAX_SHARED = 4096, 64, 8
K3_WAIT_LIMIT_DEFAULT = 1 << 20

# (name, restype, argtypes) of every exported symbol in include/k3moe.h
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


class k3_cache_stats(ctypes.Structure):
    _fields_ = [(f, ctypes.c_uint64) for f in
                ("requests", "hits", "misses", "inflight_reuses", "evictions", "bytes_copied")]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


_stats_p = ctypes.POINTER(k3_cache_stats)
SIGNATURES = [
    ("k3_strerror", ctypes.c_char_p, [_i]),
    ("k3_last_error", ctypes.c_char_p, []),
    ("k3_abi_version", _i, []),
    ("k3_mxfp4_packed_bytes", _sz, [_i, _i]),
    ("k3_mxfp4_pack_host", _i, [_vp, _vp, _i, _i, _vp]),
    ("k3_mxfp4_unpack_host", _i, [_vp, _i, _i, _vp, _vp]),
    ("k3_mxfp4_pack", _i, [_vp, _vp, _i, _i, _vp, _vp]),
    ("k3_mxfp4_unpack", _i, [_vp, _i, _i, _vp, _vp, _vp]),
    ("k3_expert_packed_bytes", _sz, [_i, _i]),
    ("k3_expert_pack_host", _i, [_vp] * 6 + [_i, _i, _vp]),
    ("k3_expert_pack", _i, [_vp] * 6 + [_i, _i, _vp, _vp]),
    ("k3_mxfp4_gemv", _i, [_vp, _vp, _i, _i, _vp, _vp]),
    ("k3_expert_swiglu", _i, [_vp, _vp, _i, _i, _vp, _vp, _vp]),
    ("k3_expert_swiglu_workspace_bytes", _sz, [_i, _i]),
    ("k3_expert_swiglu_ws", _i, [_vp, _vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    ("k3_expert_gate_up", _i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    ("k3_expert_gate_up_routed", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    ("k3_expert_down", _i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    ("k3_moe_combine", _i, [_vp, _vp, _i, _i, _vp, _vp, _vp]),
    ("k3_router", _i, [_vp, _vp, _i, _i, _i, _vp, _vp]),
    ("k3_router_topk", _i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    ("k3_router_topk_f32", _i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    ("k3_router_topk_scaled", _i, [_vp, _vp, _i, _i, _i, ctypes.c_double, _vp, _vp, _vp]),
    ("k3_moe_workspace_bytes", _sz, [_i, _i, _i, _i, _i]),
    ("k3_moe_layer", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    ("k3_moe_layer_ex", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                             _vp, _sz, _vp]),
    ("k3_moe_layer_noalloc", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                  _vp]),
    ("k3_moe_permute_workspace_bytes", _sz, [_i, _i]),
    ("k3_moe_permute", _i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    ("k3_moe_batched_workspace_bytes", _sz, [_i, _i, _i, _i, _i]),
    ("k3_moe_layer_from_logits", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp,
                                      _vp, _vp, _sz, _vp]),
    ("k3_moe_layer_batched", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                  _sz, _vp]),
    ("k3_mxfp4_quantize_f32", _i, [_vp, _i, _i, _vp, _vp, _vp]),
    ("k3_mxfp4_quantize_bf16", _i, [_vp, _i, _i, _vp, _vp, _vp]),
    ("k3_moe_prefill_workspace_bytes", _sz, [_i, _i, _i, _i, _i]),
    ("k3_moe_prefill", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                            _vp, _vp, _vp, _sz, _vp]),
    ("k3_hbm_read_probe", _i, [_vp, _sz, _vp, _vp]),
    ("k3_set_wait_limit", _i, [_i]),
    ("k3_shared_expert_bytes", _sz, [_i, _i]),
    ("k3_shared_experts", _i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    ("k3_moe_layer_shared_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i]),
    ("k3_moe_layer_shared", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _sz, _vp]),
    ("k3_expert_dense_bytes", _sz, [_i, _i]),
    ("k3_expert_dequantize", _i, [_vp, _i, _i, _vp, _vp]),
    ("k3_experts_dense", _i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    ("k3_cache_create", _i, [_i, _sz, _i, ctypes.POINTER(_vp)]),
    ("k3_cache_destroy", None, [_vp]),
    ("k3_cache_set_source", _i, [_vp, _i, _vp]),
    ("k3_cache_pin", _i, [_vp, _i, _i]),
    ("k3_cache_fetch", _i, [_vp, _vp, _i, _vp]),
    ("k3_cache_table", _vp, [_vp]),
    ("k3_cache_get_stats", _i, [_vp, _stats_p]),
    ("k3_cache_histogram", _i, [_vp, _vp]),
    ("k3_cache_trace", _i, [_vp, _vp, _sz, ctypes.POINTER(_sz)]),
    ("k3_cache_replay", _i, [_vp, _sz, _i, _i, _vp, _i, _i, _stats_p]),
    ("k3_cache_replay_opt", _i, [_vp, _sz, _i, _i, _vp, _i, _i, _stats_p]),
    ("k3_moe_layer_from_logits_cached", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp,
                                             _vp, _vp, _vp, _sz, _vp]),
    ("k3_moe_layer_cached", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _sz, _vp]),
]


class K3LibraryMissing(RuntimeError):
    pass


class K3Error(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn}: status {status} ({strerror(status)}): {detail}")


def lib():
    """Load libk3moe.so (once). Raises K3LibraryMissing if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise K3LibraryMissing(
                f"{LIB_PATH} is not built; run __graft_entry__.build() "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(status):
    return lib().k3_strerror(int(status)).decode()


def last_error():
    return lib().k3_last_error().decode()


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != K3_OK:
        raise K3Error(name, rc, last_error())
    return rc


def _dp(t):
    """Device pointer of a torch tensor or a raw address (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _hp(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---- layout ---------------------------------------------------------------

def k3_mxfp4_packed_bytes(rows, cols):
    return lib().k3_mxfp4_packed_bytes(rows, cols)


def k3_expert_packed_bytes(hidden, inter):
    return lib().k3_expert_packed_bytes(hidden, inter)


def k3_mxfp4_pack_host(nib, sc):
    nib, sc = np.ascontiguousarray(nib, np.uint8), np.ascontiguousarray(sc, np.uint8)
    rows, cols = nib.shape[0], nib.shape[1] * 2
    out = np.empty(k3_mxfp4_packed_bytes(rows, cols), np.uint8)
    _call("k3_mxfp4_pack_host", _hp(nib), _hp(sc), rows, cols, _hp(out))
    return out


def k3_mxfp4_unpack_host(tiles, rows, cols):
    tiles = np.ascontiguousarray(tiles, np.uint8)
    nib = np.empty((rows, cols // 2), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    _call("k3_mxfp4_unpack_host", _hp(tiles), rows, cols, _hp(nib), _hp(sc))
    return nib, sc


def k3_expert_pack_host(E, hidden, inter):
    arrs = [np.ascontiguousarray(a, np.uint8) for a in
            (E["gate"][0], E["gate"][1], E["up"][0], E["up"][1], E["down"][0], E["down"][1])]
    out = np.empty(k3_expert_packed_bytes(hidden, inter), np.uint8)
    _call("k3_expert_pack_host", *[_hp(a) for a in arrs], hidden, inter, _hp(out))
    return out


def k3_mxfp4_pack(nib_d, sc_d, rows, cols, tiles_d, stream=None):
    _call("k3_mxfp4_pack", _dp(nib_d), _dp(sc_d), rows, cols, _dp(tiles_d), _stream(stream))


def k3_mxfp4_unpack(tiles_d, rows, cols, nib_d, sc_d, stream=None):
    _call("k3_mxfp4_unpack", _dp(tiles_d), rows, cols, _dp(nib_d), _dp(sc_d), _stream(stream))


def k3_expert_pack(gate_nib, gate_sc, up_nib, up_sc, down_nib, down_sc, hidden, inter,
                   expert_d, stream=None):
    _call("k3_expert_pack", _dp(gate_nib), _dp(gate_sc), _dp(up_nib), _dp(up_sc),
          _dp(down_nib), _dp(down_sc), hidden, inter, _dp(expert_d), _stream(stream))


# ---- compute --------------------------------------------------------------

def _nbytes(t):
    return t.numel() * t.element_size()


def k3_mxfp4_gemv(x, tiles, rows, cols, y, stream=None):
    _call("k3_mxfp4_gemv", _dp(x), _dp(tiles), rows, cols, _dp(y), _stream(stream))


def k3_expert_swiglu(x, expert, hidden, inter, y, h, stream=None):
    _call("k3_expert_swiglu", _dp(x), _dp(expert), hidden, inter, _dp(y), _dp(h),
          _stream(stream))


def k3_expert_swiglu_workspace_bytes(hidden, inter):
    return lib().k3_expert_swiglu_workspace_bytes(hidden, inter)


def k3_expert_swiglu_ws(x, expert, hidden, inter, y, ws, h=None, stream=None):
    _call("k3_expert_swiglu_ws", _dp(x), _dp(expert), hidden, inter, _dp(y), _dp(h), _dp(ws),
          _nbytes(ws), _stream(stream))


def k3_expert_gate_up(x, experts, idx, k, hidden, inter, h, stream=None):
    _call("k3_expert_gate_up", _dp(x), _dp(experts), _dp(idx), k, hidden, inter, _dp(h),
          _stream(stream))


def k3_expert_gate_up_routed(x, logits, experts, n_experts, k, hidden, inter, h, idx, w,
                             stream=None):
    _call("k3_expert_gate_up_routed", _dp(x), _dp(logits), _dp(experts), n_experts, k, hidden,
          inter, _dp(h), _dp(idx), _dp(w), _stream(stream))


def k3_expert_down(h, experts, idx, k, hidden, inter, yp, stream=None):
    _call("k3_expert_down", _dp(h), _dp(experts), _dp(idx), k, hidden, inter, _dp(yp),
          _stream(stream))


def k3_moe_combine(yp, w, k, hidden, y=None, y_f32=None, stream=None):
    _call("k3_moe_combine", _dp(yp), _dp(w), k, hidden, _dp(y), _dp(y_f32), _stream(stream))


def k3_router(x, router_w, T, hidden, n_experts, logits, stream=None):
    _call("k3_router", _dp(x), _dp(router_w), T, hidden, n_experts, _dp(logits),
          _stream(stream))


def k3_router_topk(logits, bias, T, n_experts, k, idx, w, stream=None):
    _call("k3_router_topk", _dp(logits), _dp(bias), T, n_experts, k, _dp(idx), _dp(w),
          _stream(stream))


def k3_router_topk_f32(logits, bias, T, n_experts, k, idx, w, stream=None):
    _call("k3_router_topk_f32", _dp(logits), _dp(bias), T, n_experts, k, _dp(idx), _dp(w),
          _stream(stream))


def k3_router_topk_scaled(logits, bias, T, n_experts, k, routed_scale, idx, w, stream=None):
    _call("k3_router_topk_scaled", _dp(logits), _dp(bias), T, n_experts, k, float(routed_scale),
          _dp(idx), _dp(w), _stream(stream))


def k3_moe_workspace_bytes(T, n_experts, hidden, inter, k):
    return lib().k3_moe_workspace_bytes(T, n_experts, hidden, inter, k)


def k3_moe_layer(x, router_w, experts, n_experts, hidden, inter, k, y, ws, stream=None):
    _call("k3_moe_layer", _dp(x), _dp(router_w), _dp(experts), n_experts, hidden, inter, k,
          _dp(y), _dp(ws), _nbytes(ws), _stream(stream))


def k3_moe_layer_ex(x, router_w, experts, n_experts, hidden, inter, k, y, ws, y_f32=None,
                    idx=None, w=None, logits=None, stream=None):
    _call("k3_moe_layer_ex", _dp(x), _dp(router_w), _dp(experts), n_experts, hidden, inter,
          k, _dp(y), _dp(y_f32), _dp(idx), _dp(w), _dp(logits), _dp(ws), _nbytes(ws),
          _stream(stream))


def k3_moe_layer_noalloc(x, router_w, experts, n_experts, hidden, inter, k, y, y_f32=None,
                         idx=None, w=None, logits=None, stream=None):
    _call("k3_moe_layer_noalloc", _dp(x), _dp(router_w), _dp(experts), n_experts, hidden,
          inter, k, _dp(y), _dp(y_f32), _dp(idx), _dp(w), _dp(logits), _stream(stream))


K3_NOALLOC_SCRATCH_BYTES = 2 << 20


# ---- batched decode -------------------------------------------------------

def k3_moe_permute_workspace_bytes(T, k):
    return lib().k3_moe_permute_workspace_bytes(T, k)


def k3_moe_permute(idx, T, k, n_experts, counts, offsets, pair_token, pair_slot, ws,
                   stream=None):
    _call("k3_moe_permute", _dp(idx), T, k, n_experts, _dp(counts), _dp(offsets),
          _dp(pair_token), _dp(pair_slot), _dp(ws), _nbytes(ws), _stream(stream))


def k3_moe_batched_workspace_bytes(T, n_experts, hidden, inter, k):
    return lib().k3_moe_batched_workspace_bytes(T, n_experts, hidden, inter, k)


def k3_moe_layer_from_logits(X, logits, bias, experts, n_experts, hidden, inter, k, T, Y, ws,
                             Y_f32=None, idx=None, w=None, stream=None):
    _call("k3_moe_layer_from_logits", _dp(X), _dp(logits), _dp(bias), _dp(experts), n_experts,
          hidden, inter, k, T, _dp(Y), _dp(Y_f32), _dp(idx), _dp(w), _dp(ws), _nbytes(ws),
          _stream(stream))


def k3_moe_layer_batched(X, router_w, experts, n_experts, hidden, inter, k, T, Y, ws,
                         Y_f32=None, idx=None, w=None, stream=None):
    _call("k3_moe_layer_batched", _dp(X), _dp(router_w), _dp(experts), n_experts, hidden,
          inter, k, T, _dp(Y), _dp(Y_f32), _dp(idx), _dp(w), _dp(ws), _nbytes(ws),
          _stream(stream))


# ---- prefill --------------------------------------------------------------

def k3_mxfp4_quantize_f32(v, rows, cols, nib, sc, stream=None):
    _call("k3_mxfp4_quantize_f32", _dp(v), rows, cols, _dp(nib), _dp(sc), _stream(stream))


def k3_mxfp4_quantize_bf16(v, rows, cols, nib, sc, stream=None):
    _call("k3_mxfp4_quantize_bf16", _dp(v), rows, cols, _dp(nib), _dp(sc), _stream(stream))


def k3_moe_prefill_workspace_bytes(T, n_experts, hidden, inter, k):
    return lib().k3_moe_prefill_workspace_bytes(T, n_experts, hidden, inter, k)


def k3_moe_prefill(X, logits, bias, experts, n_experts, hidden, inter, k, T, Y, ws, Y_f32=None,
                   idx=None, w=None, h_f32=None, h_nib=None, h_sc=None, stream=None):
    _call("k3_moe_prefill", _dp(X), _dp(logits), _dp(bias), _dp(experts), n_experts, hidden,
          inter, k, T, _dp(Y), _dp(Y_f32), _dp(idx), _dp(w), _dp(h_f32), _dp(h_nib), _dp(h_sc),
          _dp(ws), _nbytes(ws), _stream(stream))


# ---- measurement ------------------------------------------------------------

def k3_hbm_read_probe(buf, nbytes, sink, stream=None):
    _call("k3_hbm_read_probe", _dp(buf), nbytes, _dp(sink), _stream(stream))


def k3_set_wait_limit(polls):
    _call("k3_set_wait_limit", polls)


# ---- shared experts ---------------------------------------------------------

def k3_shared_expert_bytes(hidden, inter):
    return lib().k3_shared_expert_bytes(hidden, inter)


def k3_shared_experts(x, shared, n_shared, hidden, inter, h, ys, stream=None):
    _call("k3_shared_experts", _dp(x), _dp(shared), n_shared, hidden, inter, _dp(h), _dp(ys),
          _stream(stream))


def k3_moe_layer_shared_workspace_bytes(n_experts, hidden, inter, k, n_shared, inter_shared):
    return lib().k3_moe_layer_shared_workspace_bytes(n_experts, hidden, inter, k, n_shared,
                                                     inter_shared)


def k3_moe_layer_shared(x, router_w, experts, n_experts, hidden, inter, k, shared, n_shared,
                        inter_shared, y, ws, y_f32=None, idx=None, w=None, logits=None,
                        stream=None):
    _call("k3_moe_layer_shared", _dp(x), _dp(router_w), _dp(experts), n_experts, hidden, inter,
          k, _dp(shared), n_shared, inter_shared, _dp(y), _dp(y_f32), _dp(idx), _dp(w),
          _dp(logits), _dp(ws), _nbytes(ws), _stream(stream))


# ---- dequantise-then-multiply control -------------------------------------

def k3_expert_dense_bytes(hidden, inter):
    return lib().k3_expert_dense_bytes(hidden, inter)


def k3_expert_dequantize(expert, hidden, inter, dense, stream=None):
    _call("k3_expert_dequantize", _dp(expert), hidden, inter, _dp(dense), _stream(stream))


def k3_experts_dense(x, dense_experts, idx, k, hidden, inter, h, yp, stream=None):
    _call("k3_experts_dense", _dp(x), _dp(dense_experts), _dp(idx), k, hidden, inter, _dp(h),
          _dp(yp), _stream(stream))


# ---- expert cache ---------------------------------------------------------
# A cache is the opaque handle (an int) k3_cache_create returns; host blobs
# are pinned CPU torch tensors or numpy arrays that the caller keeps alive.

def _ids(ids):
    a = np.ascontiguousarray(ids, np.int32)
    return a, ctypes.c_void_p(a.ctypes.data)


def k3_cache_create(n_experts, expert_bytes, n_slots):
    h = _vp()
    _call("k3_cache_create", n_experts, expert_bytes, n_slots, ctypes.byref(h))
    return h.value


def k3_cache_destroy(cache):
    lib().k3_cache_destroy(_vp(cache))


def k3_cache_set_source(cache, expert, host_blob):
    ptr = host_blob.data_ptr() if hasattr(host_blob, "data_ptr") else host_blob.ctypes.data
    _call("k3_cache_set_source", _vp(cache), expert, _vp(ptr))


def k3_cache_pin(cache, expert, pinned=True):
    _call("k3_cache_pin", _vp(cache), expert, int(bool(pinned)))


def k3_cache_fetch(cache, ids, stream=None):
    a, p = _ids(ids)
    _call("k3_cache_fetch", _vp(cache), p, a.size, _stream(stream))


def k3_cache_table(cache):
    """Device address of the cache's expert pointer table (an int)."""
    return lib().k3_cache_table(_vp(cache))


def k3_cache_get_stats(cache):
    st = k3_cache_stats()
    _call("k3_cache_get_stats", _vp(cache), ctypes.byref(st))
    return st.as_dict()


def k3_cache_histogram(cache, n_experts):
    out = np.zeros(n_experts, np.uint64)
    _call("k3_cache_histogram", _vp(cache), _hp(out))
    return out


def k3_cache_trace(cache):
    n = _sz()
    _call("k3_cache_trace", _vp(cache), None, 0, ctypes.byref(n))
    out = np.zeros(max(1, n.value), np.int32)
    _call("k3_cache_trace", _vp(cache), _hp(out), out.size, ctypes.byref(n))
    return out[:n.value]


def k3_cache_replay(trace, n_experts, n_slots, pinned=(), request_size=1):
    t, tp = _ids(trace)
    pn, pp = _ids(pinned)
    st = k3_cache_stats()
    _call("k3_cache_replay", tp, t.size, n_experts, n_slots, pp if pn.size else None,
          pn.size, request_size, ctypes.byref(st))
    return st.as_dict()


def k3_cache_replay_opt(trace, n_experts, n_slots, pinned=(), request_size=1):
    t, tp = _ids(trace)
    pn, pp = _ids(pinned)
    st = k3_cache_stats()
    _call("k3_cache_replay_opt", tp, t.size, n_experts, n_slots, pp if pn.size else None,
          pn.size, request_size, ctypes.byref(st))
    return st.as_dict()


def k3_moe_layer_cached(x, router_w, cache, n_experts, hidden, inter, k, y, ws, y_f32=None,
                        idx=None, w=None, logits=None, stream=None):
    _call("k3_moe_layer_cached", _dp(x), _dp(router_w), _vp(cache), n_experts, hidden, inter,
          k, _dp(y), _dp(y_f32), _dp(idx), _dp(w), _dp(logits), _dp(ws), _nbytes(ws),
          _stream(stream))


def k3_moe_layer_from_logits_cached(X, logits, bias, cache, n_experts, hidden, inter, k, T, Y,
                                    ws, Y_f32=None, idx=None, w=None, stream=None):
    _call("k3_moe_layer_from_logits_cached", _dp(X), _dp(logits), _dp(bias), _vp(cache),
          n_experts, hidden, inter, k, T, _dp(Y), _dp(Y_f32), _dp(idx), _dp(w), _dp(ws),
          _nbytes(ws), _stream(stream))
