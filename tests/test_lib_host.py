"""Host-side checks of the GPU library (no GPU needed): the shared object
loads and exports every entry point its header declares, the tile layout is
the documented bijection on every configuration's shapes and on ragged ones,
and the argument checks refuse bad calls before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
from gen import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(K.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return K.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "k3moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(k3_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/k3moe.h but not exported"
    bound = {s[0] for s in K.SIGNATURES}
    assert set(names) == bound, "binding and header disagree"


def test_packed_bytes_formula(L):
    for rows, cols in [(256, 1024), (1536, 7168), (7168, 1536), (1, 32), (65, 96), (100, 160)]:
        G = cols // 32
        G4 = (G + 3) // 4
        assert K.k3_mxfp4_packed_bytes(rows, cols) == ((rows + 63) // 64) * 4352 * G4
    # no padding for the routed expert's shapes: the census size exactly
    assert K.k3_expert_packed_bytes(7168, 1536) == 17547264
    assert K.k3_mxfp4_packed_bytes(0, 32) == 0 and K.k3_mxfp4_packed_bytes(4, 33) == 0


@pytest.mark.parametrize("rows,cols", [(256, 1024), (1536, 7168), (7168, 1536), (1, 32),
                                       (63, 96), (65, 160), (100, 224), (3, 4000 - 4000 % 32)])
def test_pack_roundtrip_and_layout(L, rows, cols):
    nib, sc = gen.mxfp4_matrix(1, 50, rows, cols)
    tiles = K.k3_mxfp4_pack_host(nib, sc)
    n2, s2 = K.k3_mxfp4_unpack_host(tiles, rows, cols)
    assert np.array_equal(n2, nib) and np.array_equal(s2, sc)
    # layout spot checks from the header's byte formula
    G, G4 = cols // 32, (cols // 32 + 3) // 4
    tb = 4352 * G4

    def code_off(t, g, r):  # r: row inside the tile = the lane that owns it
        return t * tb + 4352 * (g // 4) + 1024 * (g % 4) + 16 * r

    def scale_off(t, g, r):
        return t * tb + 4352 * (g // 4) + 4096 + 4 * r + g % 4

    rng = np.random.default_rng(0)
    for _ in range(50):
        r, g = int(rng.integers(rows)), int(rng.integers(G))
        t, l = r // 64, r % 64
        off = code_off(t, g, l)
        assert np.array_equal(tiles[off:off + 16], nib[r, 16 * g:16 * g + 16])
        assert tiles[scale_off(t, g, l)] == sc[r, g]
    # padding: groups past G are zero codes with exponent 0, rows past `rows` too
    t_last = (rows - 1) // 64
    for l in range(64):
        r = t_last * 64 + l
        for g in range(4 * G4):
            if r >= rows or g >= G:
                off = code_off(t_last, g, l)
                assert tiles[scale_off(t_last, g, l)] == 0
                assert not np.any(tiles[off:off + 16])


def test_expert_pack_interleaves_gate_and_up(L):
    hidden, inter = 128, 96
    E = gen.expert(2, 51, 0, hidden, inter)
    blob = K.k3_expert_pack_host(E, hidden, inter)
    G4 = (hidden // 32 + 3) // 4
    ntiles = (inter + 31) // 32
    gu_bytes = ntiles * 4352 * G4
    gu = blob[:gu_bytes]
    vrows = ntiles * 64
    vn, vs = K.k3_mxfp4_unpack_host(gu, vrows, hidden)
    for v in range(vrows):
        t, l = v // 64, v % 64
        row = 32 * t + (l % 32)
        m = "up" if l >= 32 else "gate"
        if row < inter:
            assert np.array_equal(vn[v], E[m][0][row]) and np.array_equal(vs[v], E[m][1][row])
    dn, ds = K.k3_mxfp4_unpack_host(blob[gu_bytes:], hidden, inter)
    assert np.array_equal(dn, E["down"][0]) and np.array_equal(ds, E["down"][1])


def _fake(n):
    """Aligned non-NULL addresses; only passed to calls that must refuse before
    touching them."""
    return ctypes.c_void_p(0x10000 * n)


def test_refusals_before_launch(L):
    s = None
    rc = L.k3_mxfp4_gemv(None, _fake(1), 64, 64, _fake(2), s)
    assert rc == K.K3_ERR_ARG and "x is NULL" in K.last_error()
    rc = L.k3_mxfp4_gemv(ctypes.c_void_p(0x10004), _fake(1), 64, 64, _fake(2), s)
    assert rc == K.K3_ERR_ARG and "aligned" in K.last_error()
    rc = L.k3_mxfp4_gemv(_fake(3), _fake(1), 64, 48, _fake(2), s)
    assert rc == K.K3_ERR_CONFIG and "cols=48" in K.last_error()
    rc = L.k3_mxfp4_gemv(_fake(3), _fake(1), 0, 64, _fake(2), s)
    assert rc == K.K3_ERR_CONFIG
    rc = L.k3_router_topk(_fake(1), None, 1, 896, 17 + 64, _fake(2), _fake(3), s)
    assert rc == K.K3_ERR_CONFIG and "k=81" in K.last_error()
    rc = L.k3_router_topk(_fake(1), None, 1, 8, 9, _fake(2), _fake(3), s)
    assert rc == K.K3_ERR_CONFIG
    rc = L.k3_expert_swiglu(_fake(1), _fake(2), 7168, 1500, _fake(3), _fake(4), s)
    assert rc == K.K3_ERR_CONFIG and "inter=1500" in K.last_error()
    rc = L.k3_expert_swiglu(_fake(1), _fake(2), 7168, 8192, _fake(3), _fake(4), s)
    assert rc == K.K3_ERR_CONFIG  # inter above K3_MAX_INTER
    need = K.k3_moe_workspace_bytes(1, 896, 7168, 1536, 16)
    assert need > 0
    rc = L.k3_moe_layer(_fake(1), _fake(2), _fake(3), 896, 7168, 1536, 16, _fake(4), _fake(5),
                        need - 1, s)
    assert rc == K.K3_ERR_MEMORY and "is below the" in K.last_error()
    rc = L.k3_moe_layer(_fake(1), _fake(2), _fake(3), 896, 7168, 1536, 0, _fake(4), _fake(5),
                        need, s)
    assert rc == K.K3_ERR_CONFIG
    rc = L.k3_set_wait_limit(-1)
    assert rc == K.K3_ERR_CONFIG and "polls=-1" in K.last_error()
    text = open(os.path.join(ROOT, "include", "k3moe.h")).read()
    assert re.search(r"#define K3_WAIT_LIMIT_DEFAULT \(1 << 20\)", text)
    assert K.K3_WAIT_LIMIT_DEFAULT == 1 << 20


def test_refusals_at_the_size_limits(L):
    """Empty batches, and every size past its documented maximum, are
    refused before any launch (no GPU needed)."""
    s = None
    nb = K.k3_moe_batched_workspace_bytes(1, 16, 128, 64, 2)
    for T in (0, -1):
        rc = L.k3_moe_layer_from_logits(_fake(1), _fake(2), None, _fake(3), 16, 128, 64, 2, T,
                                        _fake(4), None, None, None, _fake(5), nb, s)
        assert rc == K.K3_ERR_CONFIG, T
    rc = L.k3_router_topk(_fake(1), None, 1, K.K3_MAX_EXPERTS + 1, 4, _fake(2), _fake(3), s)
    assert rc == K.K3_ERR_CONFIG
    rc = L.k3_expert_swiglu(_fake(1), _fake(2), 16384 + 32, 64, _fake(3), _fake(4), s)
    assert rc == K.K3_ERR_CONFIG  # hidden above K3_MAX_HIDDEN
    assert K.k3_expert_packed_bytes(16384, 4096) > 0
    assert K.k3_expert_packed_bytes(16384 + 32, 4096) == 0
    assert K.k3_moe_layer_shared_workspace_bytes(8, 128, 64, 2, K.K3_MAX_SHARED + 1, 64) == 0
    h = ctypes.c_void_p()
    for args in ((0, 256, 1), (8, 256, 0), (8, 256, 9), (8, 100, 4),
                 (K.K3_MAX_EXPERTS + 1, 256, 4)):
        rc = L.k3_cache_create(*args, ctypes.byref(h))
        assert rc == K.K3_ERR_CONFIG and h.value is None, args


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(K, "_lib", None)
    with pytest.raises(K.K3LibraryMissing):
        K.k3_mxfp4_packed_bytes(64, 64)


def test_routed_scale_refusals(L):
    """k3_router_topk_scaled refuses a scale that is not a positive finite
    factor before any launch."""
    s = ctypes.c_void_p(0)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        rc = L.k3_router_topk_scaled(_fake(1), None, 2, 896, 16, bad, _fake(2), _fake(3), s)
        assert rc == K.K3_ERR_CONFIG, (bad, rc)
        assert "routed_scale" in K.last_error()
