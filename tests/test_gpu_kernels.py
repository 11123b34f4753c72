"""GPU parity of the packing, GEMV, expert and routing kernels against the
oracle, through the C ABI, on the seeded workloads (single GEMV 256x1024, one
routed expert 7168/1536) and edge cases. Floating point: max normwise
relative error <= 1e-5 against the fp64 oracle; integer and byte work
(packing, top-k indices): bit-exact; every kernel rerun: bit-identical."""
import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
import oracle
from gen import workloads as W
from tests import _independent as I
from tests._gpu import TOL, empty, normwise, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available()
    K.lib()


def gpu_gemv(nib, sc, x):
    import torch
    rows, cols = nib.shape[0], nib.shape[1] * 2
    tiles = up(K.k3_mxfp4_pack_host(nib, sc))
    xd = up(np.asarray(x, np.float32))
    y = empty(rows, torch.float32)
    K.k3_mxfp4_gemv(xd, tiles, rows, cols, y)
    y1 = y.cpu().numpy().copy()
    K.k3_mxfp4_gemv(xd, tiles, rows, cols, y)
    y2 = y.cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "rerun not bit-identical"
    return y1


@pytest.mark.parametrize("rows,cols", [(256, 1024), (100, 224), (63, 96), (1, 32), (130, 7168)])
def test_device_pack_matches_host(rows, cols):
    import torch
    say(f"device pack rows={rows} cols={cols}")
    nib, sc = gen.mxfp4_matrix(3, 60, rows, cols)
    ref = K.k3_mxfp4_pack_host(nib, sc)
    tiles = empty(ref.size, torch.uint8)
    K.k3_mxfp4_pack(up(nib), up(sc), rows, cols, tiles)
    assert np.array_equal(tiles.cpu().numpy(), ref)
    n2, s2 = empty((rows, cols // 2), torch.uint8), empty((rows, cols // 32), torch.uint8)
    K.k3_mxfp4_unpack(tiles, rows, cols, n2, s2)
    assert np.array_equal(n2.cpu().numpy(), nib) and np.array_equal(s2.cpu().numpy(), sc)


def test_device_expert_pack_matches_host():
    import torch
    hidden, inter = 256, 96
    say(f"device expert pack hidden={hidden} inter={inter}")
    E = gen.expert(4, 61, 0, hidden, inter)
    ref = K.k3_expert_pack_host(E, hidden, inter)
    out = empty(ref.size, torch.uint8)
    parts = [up(E[m][i]) for m in ("gate", "up", "down") for i in (0, 1)]
    K.k3_expert_pack(*parts, hidden, inter, out)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_gemv_golden_fixture_exact():
    """The hand-decoded bytes of tests/golden: one-hot x recovers each value."""
    say("gemv golden fixture")
    data, rows = I.read_golden_rows("e2m1_nibble_order.txt")
    nib = np.array([data] * len(rows), np.uint8)
    sc = np.array([[r[0]] for r in rows], np.uint8)
    expected = np.array([r[1] for r in rows])
    for j in range(32):
        x = np.zeros(32, np.float32)
        x[j] = 1.0
        y = gpu_gemv(nib, sc, x)
        assert np.array_equal(y.astype(np.float64), expected[:, j] + 0.0), (j, y)


def test_gemv_c1_parity():
    say("gemv C1 256x1024 seed 0")
    nib, sc, x = W.c1_inputs(seed=0)
    y = gpu_gemv(nib, sc, x)
    ref = oracle.gemv(nib, sc, x.astype(np.float64))
    err = normwise(y, ref)
    say(f"gemv C1 normwise err {err:.3e}")
    assert err <= TOL


# K of 8192 and more: 64 or more quads per workgroup, the matrix-unit products;
# the shorter ones: the vector ALU
@pytest.mark.parametrize("rows,cols,elo,ehi", [(100, 224, 120, 134), (63, 96, 10, 20),
                                               (65, 160, 230, 240), (1, 32, 127, 127),
                                               (300, 7168, 120, 134), (129, 1536, 114, 120),
                                               (130, 8192, 120, 134), (64, 16384, 114, 120),
                                               (65, 8224, 10, 20)])
def test_gemv_shapes_and_exponent_range(rows, cols, elo, ehi):
    say(f"gemv rows={rows} cols={cols} e=[{elo},{ehi}]")
    nib, sc = gen.mxfp4_matrix(5, 62, rows, cols, elo, ehi)
    x = gen.normal_f32(gen.key(5, 62, gen.KIND_TOKENS), cols)
    y = gpu_gemv(nib, sc, x)
    ref = oracle.gemv(nib, sc, x.astype(np.float64))
    assert normwise(y, ref) <= TOL


@pytest.mark.parametrize("cols", [384, 8192])
def test_gemv_nan_scale_finite_x(cols):
    """Exponent 255 with finite activations (K = 8192: the matrix-unit
    products, whose 255 groups are zeroed in the registers)."""
    say(f"gemv exponent 255, finite activations, cols={cols}")
    rows = 130
    nib, sc = gen.mxfp4_matrix(8, 66, rows, cols)
    sc = sc.copy()
    sc[:, 3] = 255
    sc[7, :] = 255
    sc[64:70, 9] = 255
    x = gen.normal_f32(gen.key(8, 66, gen.KIND_TOKENS), cols)
    y = gpu_gemv(nib, sc, x)
    assert y[7] == 0.0
    ref = oracle.gemv(nib, sc, x.astype(np.float64))
    assert normwise(y, ref) <= TOL


def test_gemv_nan_scale_contains_nonfinite_x():
    say("gemv exponent 255 with NaN/Inf activations")
    rows, cols = 70, 256
    nib, sc = gen.mxfp4_matrix(6, 63, rows, cols)
    sc = sc.copy()
    sc[:, 2] = 255
    sc[5, :] = 255
    x = gen.normal_f32(gen.key(6, 63, gen.KIND_TOKENS), cols)
    x[64:96] = np.nan
    x[70] = np.inf
    y = gpu_gemv(nib, sc, x)
    assert np.all(np.isfinite(y)) and y[5] == 0.0
    ref = oracle.gemv(nib, sc, x.astype(np.float64))
    assert normwise(y, ref) <= TOL


def test_gemv_activation_groups_outside_digit_range():
    """Activation groups whose largest value is below 2^-87 or at least 2^122
    (beyond the exponents of the matrix unit's activation digits) send the
    workgroups to the vector-ALU products; results still match the oracle.
    That route sums a group's unscaled products in fp32, so the large group
    has one non-zero code per row (a finite group sum); weights scaled by
    2^-27 keep every product finite."""
    say("gemv activation groups of 2^-100 and 2^123")
    rows, cols = 200, 8192  # 64 quads per workgroup: the matrix route is tried first
    nib, sc = gen.mxfp4_matrix(12, 71, rows, cols, 98, 102)
    nib = nib.copy()
    nib[:, 64:80] = 0  # group 4 (elements 128..159): only element 128's code stays
    nib[:, 64] = gen.mxfp4_matrix(12, 73, rows, 32)[0][:, 0] & 0x0F
    x = gen.normal_f32(gen.key(12, 71, gen.KIND_TOKENS), cols).astype(np.float64)
    x[32:64] *= 2.0 ** -100  # group 1: largest value far below 2^-87
    x[128] = 1.5 * 2.0 ** 123  # group 4: largest value above 2^122
    x = x.astype(np.float32)
    y = gpu_gemv(nib, sc, x)
    ref = oracle.gemv(nib, sc, x.astype(np.float64))
    assert np.all(np.isfinite(y))
    assert normwise(y, ref) <= TOL


def test_gemv_extreme_exponent_bytes_on_the_matrix_unit():
    """Exponent bytes 0, 1, 2, 126..128, 252, 253, 254 mixed in every row, with
    activations around 2^-58 (inside the digits' range, so the matrix unit
    multiplies): each group scaled by the instruction's E8M0 scale, results
    within fp32 range of the oracle."""
    say("gemv exponent bytes 0..2, 126..128, 252..254 on the matrix unit")
    rows, cols = 192, 8192
    nib, _ = gen.mxfp4_matrix(13, 72, rows, cols)
    rng = np.random.default_rng(1372)
    sc = rng.choice(np.array([0, 1, 2, 126, 127, 128, 252, 253, 254], np.uint8),
                    size=(rows, cols // 32))
    x = (gen.normal_f32(gen.key(13, 72, gen.KIND_TOKENS), cols).astype(np.float64) *
         2.0 ** -58).astype(np.float32)
    y = gpu_gemv(nib, sc, x)
    ref = oracle.gemv(nib, sc, x.astype(np.float64))
    assert np.all(np.isfinite(y))
    assert normwise(y, ref) <= TOL


def _expert_on_gpu(E, x_bf16, hidden, inter):
    import torch
    blob = up(K.k3_expert_pack_host(E, hidden, inter))
    xd = up(x_bf16)
    y = empty(hidden, torch.float32)
    h = empty(inter, torch.float32)
    K.k3_expert_swiglu(xd, blob, hidden, inter, y, h)
    y1, h1 = y.cpu().numpy().copy(), h.cpu().numpy().copy()
    K.k3_expert_swiglu(xd, blob, hidden, inter, y, h)
    assert np.array_equal(y1.view(np.uint32), y.cpu().numpy().view(np.uint32))
    return y1, h1


@pytest.mark.parametrize("elo,ehi", [(120, 134), (114, 120)])
def test_expert_c2_parity(elo, ehi):
    hidden, inter = W.HIDDEN, W.INTER
    say(f"expert C2 hidden={hidden} inter={inter} e=[{elo},{ehi}]")
    E = W.expert_weights(0, W.C2, 0, hidden, inter, elo, ehi)
    x = W.tokens_bf16(0, W.C2, 1, hidden)[0]
    y, h = _expert_on_gpu(E, x, hidden, inter)
    oracle.set_threads(16)
    y_ref, h_ref = oracle.expert_swiglu(E, I.bf16_to_float_bits(x))
    eh, ey = normwise(h, h_ref), normwise(y, y_ref)
    say(f"expert C2 normwise err h {eh:.3e} y {ey:.3e}")
    assert eh <= TOL and ey <= TOL


def test_expert_nonfinite_x_takes_exact_path():
    """An Inf in x must give the oracle's result: rows reach Inf/NaN exactly
    where a finite-exponent group meets it."""
    hidden, inter = 128, 64
    say("expert with an Inf activation")
    E = gen.expert(9, 67, 0, hidden, inter, 114, 120)
    x = gen.normal_bf16(gen.key(9, 67, gen.KIND_TOKENS), hidden)
    E["gate"][1][:, 1] = 255  # gate group 1 (elements 32..63) skipped
    E["up"][1][:, 1] = 255
    x = x.copy()
    x[40] = 0x7F80  # +Inf in group 1
    y, h = _expert_on_gpu(E, x, hidden, inter)
    y_ref, h_ref = oracle.expert_swiglu(E, I.bf16_to_float_bits(x))
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(h_ref))
    assert normwise(h, h_ref) <= TOL and normwise(y, y_ref) <= TOL


def test_expert_small_ragged():
    hidden, inter = 96, 160  # ragged gate/up tile (inter % 64 != 0), G % 4 != 0
    say(f"expert hidden={hidden} inter={inter}")
    E = gen.expert(7, 64, 0, hidden, inter, 114, 120)
    x = gen.normal_bf16(gen.key(7, 64, gen.KIND_TOKENS), hidden)
    y, h = _expert_on_gpu(E, x, hidden, inter)
    y_ref, h_ref = oracle.expert_swiglu(E, I.bf16_to_float_bits(x))
    assert normwise(h, h_ref) <= TOL and normwise(y, y_ref) <= TOL


def _expert_one_launch(E, x_bf16, hidden, inter):
    """k3_expert_swiglu_ws (one launch, gate/up split along K): y and h,
    checked bit-identical over a rerun on the same workspace."""
    import torch
    blob = up(K.k3_expert_pack_host(E, hidden, inter))
    xd = up(x_bf16)
    ws = empty(K.k3_expert_swiglu_workspace_bytes(hidden, inter), torch.uint8)
    y = empty(hidden, torch.float32)
    h = empty(inter, torch.float32)
    K.k3_expert_swiglu_ws(xd, blob, hidden, inter, y, ws, h=h)
    y1, h1 = y.cpu().numpy().copy(), h.cpu().numpy().copy()
    y2 = empty(hidden, torch.float32)
    K.k3_expert_swiglu_ws(xd, blob, hidden, inter, y2, ws)  # h optional
    assert np.array_equal(y1.view(np.uint32), y2.cpu().numpy().view(np.uint32)), "rerun differs"
    return y1, h1


# C2 in both exponent ranges; a ragged gate/up tile with G % 4 != 0; the
# largest hidden with one gate/up tile (chunks of one quad); the largest
# inter with a one-quad K (one chunk per tile, 128 tiles)
@pytest.mark.parametrize("hidden,inter,elo,ehi", [(7168, 1536, 120, 134), (7168, 1536, 114, 120),
                                                  (96, 160, 114, 120), (16384, 32, 114, 120),
                                                  (128, 4096, 114, 120), (800, 224, 114, 120)])
def test_expert_one_launch_parity(hidden, inter, elo, ehi):
    say(f"expert in one launch hidden={hidden} inter={inter} e=[{elo},{ehi}]")
    E = gen.expert(10, 68, 0, hidden, inter, elo, ehi)
    x = gen.normal_bf16(gen.key(10, 68, gen.KIND_TOKENS), hidden)
    y, h = _expert_one_launch(E, x, hidden, inter)
    oracle.set_threads(16)
    y_ref, h_ref = oracle.expert_swiglu(E, I.bf16_to_float_bits(x))
    eh, ey = normwise(h, h_ref), normwise(y, y_ref)
    say(f"expert in one launch: normwise h {eh:.3e} y {ey:.3e}")
    assert eh <= TOL and ey <= TOL


def test_expert_one_launch_nonfinite_x_in_skipped_group():
    hidden, inter = 1024, 256
    say("expert in one launch with NaN/Inf activations inside 255 groups")
    E = gen.expert(9, 69, 0, hidden, inter, 114, 120)
    x = gen.normal_bf16(gen.key(9, 69, gen.KIND_TOKENS), hidden).copy()
    E["gate"][1][:, 3] = 255
    E["up"][1][:, 3] = 255
    x[100] = 0x7F80
    x[101] = 0x7FC0
    y, h = _expert_one_launch(E, x, hidden, inter)
    y_ref, h_ref = oracle.expert_swiglu(E, I.bf16_to_float_bits(x))
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(y))
    assert normwise(h, h_ref) <= TOL and normwise(y, y_ref) <= TOL


def test_expert_one_launch_captured_graph_takes_the_two_launches():
    """Under stream capture the call records k3_expert_swiglu's two launches:
    every replay gives their bits."""
    import torch
    hidden, inter = 512, 256
    E = gen.expert(11, 70, 0, hidden, inter, 114, 120)
    x = gen.normal_bf16(gen.key(11, 70, gen.KIND_TOKENS), hidden)
    blob = up(K.k3_expert_pack_host(E, hidden, inter))
    xd = up(x)
    ws = empty(K.k3_expert_swiglu_workspace_bytes(hidden, inter), torch.uint8)
    y = empty(hidden, torch.float32)
    yw, hw = empty(hidden, torch.float32), empty(inter, torch.float32)
    K.k3_expert_swiglu(xd, blob, hidden, inter, yw, hw)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        K.k3_expert_swiglu_ws(xd, blob, hidden, inter, y, ws, stream=s)
    for _ in range(3):
        y.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), yw.cpu().numpy().view(np.uint32))


def test_router_logits_and_topk():
    import torch
    n, hidden, T, k = W.N_EXPERTS, W.HIDDEN, 3, W.TOPK
    say(f"router n={n} hidden={hidden} T={T} k={k}")
    R = W.router_bf16(0, W.C3)
    X = W.tokens_bf16(0, W.C3, T)
    lg = empty((T, n), torch.float64)
    K.k3_router(up(X), up(R), T, hidden, n, lg)
    idx = empty((T, k), torch.int32)
    w = empty((T, k), torch.float32)
    K.k3_router_topk(lg, None, T, n, k, idx, w)
    lg_h, idx_h, w_h = lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    for t in range(T):
        ref = oracle.router_logits(X[t], R)
        assert np.max(np.abs(lg_h[t] - ref)) <= 1e-12 * np.max(np.abs(ref))
        ii, ww = oracle.topk(ref, k)
        keys = np.sort(ref)[::-1]
        say(f"router token {t}: gap k/k+1 = {keys[k - 1] - keys[k]:.3e}")
        assert np.array_equal(idx_h[t], ii)
        assert np.max(np.abs(w_h[t] - ww)) <= 1e-6


@pytest.mark.parametrize("case", ["ties", "bias", "k1", "kn", "zipf", "uniform", "all_equal",
                                  "k64", "coarse"])
def test_topk_cases(case):
    import torch
    say(f"topk case {case}")
    bias = None
    if case == "ties":
        L = np.array([[0.5, 1.0, 0.25, 1.0, 1.0, -2.0, 1.0, 0.0]], np.float32)
        k = 5
    elif case == "bias":
        L = gen.normal_f32(gen.key(1, 65, gen.KIND_LOGITS), 4 * 896).reshape(4, 896)
        bias = W.routing_bias(1, 896, 0.5)
        k = 16
    elif case == "k1":
        L = gen.normal_f32(gen.key(2, 65, gen.KIND_LOGITS), 2 * 896).reshape(2, 896)
        k = 1
    elif case == "kn":
        L = gen.normal_f32(gen.key(3, 65, gen.KIND_LOGITS), 2 * 40).reshape(2, 40)
        k = 40
    elif case == "zipf":
        L = W.zipf_router_logits(0, 64)
        k = 16
    elif case == "uniform":
        L = W.uniform_router_logits(0, 256)
        k = 16
    elif case == "all_equal":  # every key ties: more than 64 candidates
        L = np.full((2, 896), 0.5, np.float32)
        k = 16
    elif case == "k64":
        L = gen.normal_f32(gen.key(4, 65, gen.KIND_LOGITS), 3 * 896).reshape(3, 896)
        k = 64
    else:  # few distinct values: many ties inside the candidate set
        L = np.round(gen.normal_f32(gen.key(5, 65, gen.KIND_LOGITS), 4 * 896) * 2).reshape(
            4, 896).astype(np.float32) / 2
        k = 16
    T, n = L.shape
    idx = empty((T, k), torch.int32)
    w = empty((T, k), torch.float32)
    K.k3_router_topk_f32(up(L), None if bias is None else up(bias), T, n, k, idx, w)
    idx_h, w_h = idx.cpu().numpy(), w.cpu().numpy()
    for t in range(T):
        ii, ww = oracle.topk(L[t].astype(np.float64), k,
                             None if bias is None else bias.astype(np.float64))
        assert np.array_equal(idx_h[t], ii), (case, t, idx_h[t], ii)
        assert np.max(np.abs(w_h[t] - ww)) <= 1e-6


@pytest.mark.parametrize("scale", [1.0, 2.5, 0.125])
def test_topk_routed_scale(scale):
    """k3_router_topk_scaled: the same selection as k3_router_topk (bias
    included), weights = the oracle's renormalised weights times the scale;
    scale 1 gives k3_router_topk's bits."""
    import torch
    T, n, k = 5, 896, 16
    L = gen.normal_f32(gen.key(3, 71, gen.KIND_LOGITS), T * n).reshape(T, n).astype(np.float64)
    bias = W.routing_bias(3, n, 0.5).astype(np.float32)
    idx = empty((T, k), torch.int32)
    w = empty((T, k), torch.float32)
    K.k3_router_topk_scaled(up(L), up(bias), T, n, k, scale, idx, w)
    idx0 = empty((T, k), torch.int32)
    w0 = empty((T, k), torch.float32)
    K.k3_router_topk(up(L), up(bias), T, n, k, idx0, w0)
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(gi, idx0.cpu().numpy())
    if scale == 1.0:
        assert np.array_equal(gw.view(np.uint32), w0.cpu().numpy().view(np.uint32))
    for t in range(T):
        ri, rw = oracle.topk(L[t], k, bias.astype(np.float64))
        assert np.array_equal(gi[t], ri)
        assert np.max(np.abs(gw[t] - scale * rw)) <= 1e-6 * scale


def test_hbm_read_probe_runs_and_refuses():
    """The calibration read streams a buffer and leaves the sink alone
    (ordinary data does not fold to its magic value); bad sizes are refused."""
    import torch
    buf = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    K.k3_hbm_read_probe(buf, buf.numel(), sink)
    torch.cuda.synchronize()
    assert int(sink.sum()) == 0
    for n in (0, 15, 17):
        with pytest.raises(K.K3Error) as e:
            K.k3_hbm_read_probe(buf, n, sink)
        assert e.value.status == K.K3_ERR_CONFIG
