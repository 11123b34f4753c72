"""GPU checks of the dequantise-then-multiply control through the C ABI.

- k3_expert_dequantize: every weight of gate, up and down equals the
  oracle's dequantisation (fp64, cast to fp32: exact for exponent bytes
  0..252) bit for bit, on ragged shapes, on groups whose exponent bytes are
  the edge values 0, 1, 2, 252 and 255 (255: zeros), and on one full-size
  expert (7168/1536).
- k3_experts_dense: h and the slot outputs within 1e-5 normwise of the
  oracle's expert (fp64), for k slots read through a pointer table in a
  permuted order; the packed path's slot outputs agree with it to the same
  bound; reruns are bit-identical.
"""
import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
import oracle
from gen import workloads as W
from mxfp4_packed_weight_amd.pool import ExpertPool
from tests._gpu import TOL, empty, normwise, say, up

pytestmark = pytest.mark.gpu


def dense_of(pool, e):
    import torch
    n = K.k3_expert_dense_bytes(pool.hidden, pool.inter) // 4
    d = empty(n, torch.float32)
    K.k3_expert_dequantize(pool.expert_view(e), pool.hidden, pool.inter, d)
    return d


def check_dequant(E, hidden, inter):
    import torch
    pool = ExpertPool(1, hidden, inter, "cuda")
    pool.load(0, E)
    d = dense_of(pool, 0).cpu().numpy()
    parts = [("gate", inter * hidden, (inter, hidden)), ("up", inter * hidden, (inter, hidden)),
             ("down", hidden * inter, (hidden, inter))]
    off = 0
    for name, n, shape in parts:
        got = d[off:off + n].reshape(shape)
        ref = oracle.dequant(*E[name]).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
        off += n


@pytest.mark.parametrize("hidden,inter", [(96, 64), (128, 160), (256, 96), (32, 32)])
def test_dequantize_ragged(hidden, inter):
    say(f"dequantize hidden={hidden} inter={inter}")
    E = W.expert_weights(5, 80, 0, hidden, inter, 114, 140)
    check_dequant(E, hidden, inter)


def test_dequantize_edge_exponents():
    """Exponent bytes 0 (subnormal results), 1, 2, 252 and 255 (zeros)."""
    hidden, inter = 128, 64
    say("dequantize edge exponents")
    rng = np.random.default_rng(4)
    E = {}
    for name, rows, cols in (("gate", inter, hidden), ("up", inter, hidden),
                             ("down", hidden, inter)):
        nib = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
        sc = rng.choice(np.array([0, 1, 2, 127, 252, 255], np.uint8), (rows, cols // 32))
        E[name] = (nib, sc)
    check_dequant(E, hidden, inter)


def test_dequantize_full_size_expert():
    say("dequantize one 7168/1536 expert (132 MB of fp32)")
    E = W.expert_weights(0, W.C3, 3)
    check_dequant(E, W.HIDDEN, W.INTER)


@pytest.mark.parametrize("hidden,inter,k", [(256, 96, 5), (7168, 1536, 4)])
def test_experts_dense_against_oracle(hidden, inter, k):
    import torch
    say(f"experts_dense hidden={hidden} inter={inter} k={k}")
    cfg, seed, n = 81, 6, k + 2
    Es = [W.expert_weights(seed, cfg, e, hidden, inter, 120, 134) for e in range(n)]
    pool = ExpertPool(n, hidden, inter, "cuda")
    for e, E in enumerate(Es):
        pool.load(e, E)
    dense = [dense_of(pool, e) for e in range(n)]
    table = up(np.array([d.data_ptr() for d in dense], np.uint64))
    order = np.random.default_rng(7).permutation(n)[:k].astype(np.int32)
    idx = up(order)
    x = W.tokens_bf16(seed, cfg, 1, hidden)[0]
    xd = up(x)
    h = empty((k, inter), torch.float32)
    yp = empty((k, hidden), torch.float32)
    K.k3_experts_dense(xd, table, idx, k, hidden, inter, h, yp)
    h_np, yp_np = h.cpu().numpy(), yp.cpu().numpy()
    # packed path on the same slots
    hp = empty((k, inter), torch.float32)
    ypp = empty((k, hidden), torch.float32)
    K.k3_expert_gate_up(xd, pool.table, idx, k, hidden, inter, hp)
    K.k3_expert_down(hp, pool.table, idx, k, hidden, inter, ypp)
    xf = oracle.bf16_to_f64(x)
    oracle.set_threads(16)
    for j, e in enumerate(order):
        y_ref, h_ref = oracle.expert_swiglu(Es[e], xf)
        assert normwise(h_np[j], h_ref) <= TOL
        assert normwise(yp_np[j], y_ref) <= TOL
        assert normwise(ypp.cpu().numpy()[j], yp_np[j]) <= 2 * TOL
    # rerun: bit-identical
    yp2 = empty((k, hidden), torch.float32)
    K.k3_experts_dense(xd, table, idx, k, hidden, inter, h, yp2)
    assert np.array_equal(yp2.cpu().numpy().view(np.uint32), yp_np.view(np.uint32))


def test_dense_refusals():
    import torch
    assert K.k3_expert_dense_bytes(7168, 1536) == 12 * 7168 * 1536
    assert K.k3_expert_dense_bytes(7168, 1537) == 0
    d = empty(16, torch.float32)
    with pytest.raises(K.K3Error) as e:
        K.k3_expert_dequantize(d, 7168, 33, d)
    assert e.value.status == K.K3_ERR_CONFIG
    with pytest.raises(K.K3Error) as e:
        K.k3_experts_dense(d, d, d, 0, 128, 64, d, d)
    assert e.value.status == K.K3_ERR_CONFIG
