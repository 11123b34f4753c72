"""The decode layer without a caller workspace (k3_moe_layer_noalloc, its
scratch a static device array in the library) against the workspace entry
point k3_moe_layer_ex: two calls in a row, the second at a smaller shape,
each bit-identical to k3_moe_layer_ex on the same inputs (and so within the
oracle bar the layer's own tests hold it to), plus a refusal above the
static scratch's size. Scratch left by the first, larger call must not leak
into the second."""
import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
import oracle
from gen import device as D
from tests._gpu import TOL, empty, normwise, say, up

pytestmark = pytest.mark.gpu


def _case(seed, cfg, n, hidden, inter):
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.05).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    return pool, R, x


def _outs(hidden, n, k):
    import torch
    return dict(y=empty(hidden, torch.int16), y32=empty(hidden, torch.float32),
                idx=empty(k, torch.int32), w=empty(k, torch.float32),
                logits=empty(n, torch.float64))


def _host(o):
    return {key: v.cpu().numpy() for key, v in o.items()}


def test_noalloc_layer_matches_workspace_layer():
    import torch
    cases = [(5, 81, 64, 1024, 512, 8), (6, 82, 20, 256, 128, 3)]  # the second is smaller
    for seed, cfg, n, hidden, inter, k in cases:
        say(f"noalloc layer n={n} hidden={hidden} inter={inter} k={k}")
        pool, R, x = _case(seed, cfg, n, hidden, inter)
        xd, Rd = up(x), up(R)
        a = _outs(hidden, n, k)
        K.k3_moe_layer_noalloc(xd, Rd, pool.table, n, hidden, inter, k, a["y"], y_f32=a["y32"],
                               idx=a["idx"], w=a["w"], logits=a["logits"])
        b = _outs(hidden, n, k)
        ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
        K.k3_moe_layer_ex(xd, Rd, pool.table, n, hidden, inter, k, b["y"], ws, y_f32=b["y32"],
                          idx=b["idx"], w=b["w"], logits=b["logits"])
        torch.cuda.synchronize()
        ha, hb = _host(a), _host(b)
        for key in ha:
            assert np.array_equal(ha[key].view(np.uint8), hb[key].view(np.uint8)), key
        experts = {int(e): gen.expert(seed, cfg, int(e), hidden, inter, 114, 120)
                   for e in hb["idx"]}
        y_ref, idx_ref, _ = oracle.moe_layer(x, R, experts, k, hidden, inter)
        assert np.array_equal(ha["idx"], idx_ref)
        err = normwise(ha["y32"], y_ref)
        assert err <= TOL, err
        say(f"noalloc layer: bit-identical to the workspace call, normwise {err:.3e}")


def test_noalloc_layer_refuses_shapes_beyond_its_scratch():
    import torch
    n, hidden, inter, k = 64, 16384, 4096, 64  # about 4.3 MB of scratch
    assert K.k3_moe_workspace_bytes(1, n, hidden, inter, k) > K.K3_NOALLOC_SCRATCH_BYTES
    x = empty(hidden, torch.int16)
    R = empty((n, hidden), torch.int16)
    table = empty(n, torch.int64)
    y = empty(hidden, torch.int16)
    with pytest.raises(K.K3Error) as e:
        K.k3_moe_layer_noalloc(x, R, table, n, hidden, inter, k, y)
    assert e.value.status == K.K3_ERR_MEMORY and "static scratch" in K.last_error()
