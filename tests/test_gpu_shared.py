"""GPU parity of the shared experts (bf16 SwiGLU on every token) and of the
decode layer with them, through the C ABI, against the oracle.

- k3_shared_experts: h within 1e-5 normwise of the oracle per shared expert,
  ys within 1e-5 of the oracle's summed outputs, for 1..3 shared experts on
  small and ragged shapes and for two 7168/1536 experts; reruns bit-identical.
- k3_moe_layer_shared: indices bit-exact; y_f32 within 1e-5 of the oracle's
  layer with shared experts; y_f32 equal bit for bit to the plain layer's
  y_f32 plus ys in fp32 (the shared output joins after the rank-order sum);
  y equal to RNE of y_f32; n_shared = 0 gives the plain layer's bits.
- The shared layer captured in a HIP graph (separate launches) matches the
  eager layer bit for bit over several replays.
"""
import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
import oracle
from gen import device as D
from gen import workloads as W
from tests._gpu import TOL, empty, normwise, say, up

pytestmark = pytest.mark.gpu


def shared_on_device(shared):
    """Device blobs (gate, up, down back to back) and their pointer table."""
    blobs = [up(np.concatenate([S["gate"].ravel(), S["up"].ravel(), S["down"].ravel()]))
             for S in shared]
    table = up(np.array([b.data_ptr() for b in blobs], np.uint64))
    return blobs, table


def oracle_shared_sum(shared, x_bf16):
    xf = oracle.bf16_to_f64(x_bf16)
    ys, hs = np.zeros(len(x_bf16)), []
    for S in shared:
        y, h = oracle.shared_expert(S, xf)
        ys += y
        hs.append(h)
    return ys, hs


@pytest.mark.parametrize("hidden,inter,ns", [(256, 96, 1), (384, 224, 2), (96, 32, 3),
                                             (7168, 1536, 2)])
def test_shared_experts_against_oracle(hidden, inter, ns):
    import torch
    say(f"shared experts hidden={hidden} inter={inter} n_shared={ns}")
    shared = W.shared_experts_bf16(4, 90, ns, hidden, inter)
    blobs, table = shared_on_device(shared)
    x = W.tokens_bf16(4, 90, 1, hidden)[0]
    xd = up(x)
    h = empty((ns, inter), torch.float32)
    ys = empty(hidden, torch.float32)
    K.k3_shared_experts(xd, table, ns, hidden, inter, h, ys)
    oracle.set_threads(16)
    ys_ref, hs_ref = oracle_shared_sum(shared, x)
    h_np, ys_np = h.cpu().numpy(), ys.cpu().numpy()
    for s in range(ns):
        assert normwise(h_np[s], hs_ref[s]) <= TOL
    assert normwise(ys_np, ys_ref) <= TOL
    ys2 = empty(hidden, torch.float32)
    K.k3_shared_experts(xd, table, ns, hidden, inter, h, ys2)
    assert np.array_equal(ys2.cpu().numpy().view(np.uint32), ys_np.view(np.uint32))


def small_layer(seed, cfg, n, hidden, inter):
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    return pool, R


def run_shared_layer(pool, R_d, xd, n, hidden, inter, k, table, ns, inter_s, ws):
    import torch
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    idx = empty(k, torch.int32)
    w = empty(k, torch.float32)
    K.k3_moe_layer_shared(xd, R_d, pool.table, n, hidden, inter, k, table, ns, inter_s, y, ws,
                          y_f32=y32, idx=idx, w=w)
    return dict(y=y.cpu().numpy().view(np.uint16), y32=y32.cpu().numpy(),
                idx=idx.cpu().numpy(), w=w.cpu().numpy())


@pytest.mark.parametrize("n,hidden,inter,k,inter_s", [(40, 256, 96, 8, 160), (24, 384, 224, 4, 96)])
def test_layer_with_shared_experts(n, hidden, inter, k, inter_s):
    import torch
    cfg, seed = 91, 5
    say(f"layer with shared experts n={n} hidden={hidden} inter={inter} inter_s={inter_s}")
    pool, R = small_layer(seed, cfg, n, hidden, inter)
    R_d = up(R)
    shared = W.shared_experts_bf16(seed, cfg, 2, hidden, inter_s, 0.5)
    blobs, table = shared_on_device(shared)
    ws = empty(K.k3_moe_layer_shared_workspace_bytes(n, hidden, inter, k, 2, inter_s),
               torch.uint8)
    ws_plain = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    experts = {e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120) for e in range(n)}
    oracle.set_threads(16)
    for t in range(3):
        x = W.tokens_bf16(seed, cfg, 1, hidden, batch=t)[0]
        xd = up(x)
        out = run_shared_layer(pool, R_d, xd, n, hidden, inter, k, table, 2, inter_s, ws)
        y_ref, idx_ref, w_ref = oracle.moe_layer_shared(x, R, experts, k, hidden, inter, shared)
        assert np.array_equal(out["idx"], idx_ref)
        assert np.max(np.abs(out["w"] - w_ref)) <= 1e-6
        assert normwise(out["y32"], y_ref) <= TOL
        assert np.array_equal(out["y"], oracle.f32_to_bf16(out["y32"]))
        # composition: the plain layer's fp32 output plus ys, in fp32
        y32p = empty(hidden, torch.float32)
        yb = empty(hidden, torch.int16)
        K.k3_moe_layer_ex(xd, R_d, pool.table, n, hidden, inter, k, yb, ws_plain, y_f32=y32p)
        h = empty((2, inter_s), torch.float32)
        ys = empty(hidden, torch.float32)
        K.k3_shared_experts(xd, table, 2, hidden, inter_s, h, ys)
        want = (y32p.cpu().numpy() + ys.cpu().numpy()).astype(np.float32)
        assert np.array_equal(out["y32"].view(np.uint32), want.view(np.uint32)), t
        # no shared experts: the plain layer's bits
        out0 = run_shared_layer(pool, R_d, xd, n, hidden, inter, k, table, 0, inter_s, ws)
        assert np.array_equal(out0["y32"].view(np.uint32), y32p.cpu().numpy().view(np.uint32))


def test_shared_layer_in_a_captured_graph():
    import torch
    cfg, seed, n, hidden, inter, k, inter_s = 92, 6, 32, 256, 160, 6, 96
    say("shared layer in a captured graph: 3 replays")
    pool, R = small_layer(seed, cfg, n, hidden, inter)
    R_d = up(R)
    shared = W.shared_experts_bf16(seed, cfg, 2, hidden, inter_s, 0.5)
    blobs, table = shared_on_device(shared)
    nb = K.k3_moe_layer_shared_workspace_bytes(n, hidden, inter, k, 2, inter_s)
    ws, ws_e = empty(nb, torch.uint8), empty(nb, torch.uint8)
    X = W.tokens_bf16(seed, cfg, 3, hidden)
    xin = empty(hidden, torch.int16)
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    s = torch.cuda.Stream()
    xin.copy_(up(X[0]))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        K.k3_moe_layer_shared(xin, R_d, pool.table, n, hidden, inter, k, table, 2, inter_s, y,
                              ws, y_f32=y32, stream=s)
    for t in range(3):
        xin.copy_(up(X[t]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y32.cpu().numpy().copy()
        eager = run_shared_layer(pool, R_d, up(X[t]), n, hidden, inter, k, table, 2, inter_s,
                                 ws_e)
        assert np.array_equal(got.view(np.uint32), eager["y32"].view(np.uint32)), t


def test_shared_refusals():
    import torch
    d = empty(64, torch.float32)
    assert K.k3_shared_expert_bytes(7168, 1536) == 6 * 7168 * 1536
    assert K.k3_moe_layer_shared_workspace_bytes(8, 128, 64, 2, K.K3_MAX_SHARED + 1, 64) == 0
    with pytest.raises(K.K3Error) as e:
        K.k3_shared_experts(d, d, 0, 128, 64, d, d)
    assert e.value.status == K.K3_ERR_CONFIG
    with pytest.raises(K.K3Error) as e:
        K.k3_shared_experts(d, d, 1, 128, 48, d, d)
    assert e.value.status == K.K3_ERR_CONFIG
