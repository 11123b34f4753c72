"""The bounded hand-off waits, run out on purpose from the host.

The launches whose workgroups wait for each other's data (the decode
layer's expert launch and the one-expert launch) poll each hand-off a
bounded number of times. If the polls run out, the launch still ends and
reports it in its output (NaN in fp32, 0x7FC0 in bf16) instead of hanging.
k3_set_wait_limit(0) makes every such wait fail at once, so that report is
checked here without holding the device; every kernel still exits
normally. The limit is restored afterwards, and the next calls must give
their usual bits: each call marks its arrival slots with a value of its own,
so a failed call leaves nothing that a later one could mistake for an
arrival."""
import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
from gen import device as D
from tests._gpu import assert_same, empty, layer_outputs, say, up

pytestmark = pytest.mark.gpu


def test_layer_waits_that_run_out_report_nan():
    import torch
    cfg, seed, n, hidden, inter, k = 77, 13, 20, 256, 128, 4
    say(f"decode layer with its waits run out, n={n} hidden={hidden} inter={inter} k={k}")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = up(gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02))
    xd = up(gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden))
    ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    ref = layer_outputs(pool, R, xd, n, hidden, inter, k, ws)
    assert np.all(np.isfinite(ref["y32"]))
    try:
        K.k3_set_wait_limit(0)
        out = layer_outputs(pool, R, xd, n, hidden, inter, k, ws)
        torch.cuda.synchronize()
    finally:
        K.k3_set_wait_limit(K.K3_WAIT_LIMIT_DEFAULT)
    assert np.all(np.isnan(out["y32"])), "a wait that ran out must show in y_f32"
    assert np.all(out["y"] == 0x7FC0), "a wait that ran out must show in y"
    assert np.array_equal(out["idx"], ref["idx"])  # selected before any hand-off
    assert_same(layer_outputs(pool, R, xd, n, hidden, inter, k, ws), ref)


def test_one_expert_launch_waits_that_run_out_report_nan():
    import torch
    hidden, inter = 512, 256
    say(f"expert in one launch with its wait run out, hidden={hidden} inter={inter}")
    E = gen.expert(14, 78, 0, hidden, inter, 114, 120)
    blob = up(K.k3_expert_pack_host(E, hidden, inter))
    xd = up(gen.normal_bf16(gen.key(14, 78, gen.KIND_TOKENS), hidden))
    ws = empty(K.k3_expert_swiglu_workspace_bytes(hidden, inter), torch.uint8)

    def run():
        y = empty(hidden, torch.float32)
        K.k3_expert_swiglu_ws(xd, blob, hidden, inter, y, ws)
        return y.cpu().numpy()

    ref = run()
    assert np.all(np.isfinite(ref))
    try:
        K.k3_set_wait_limit(0)
        bad = run()
    finally:
        K.k3_set_wait_limit(K.K3_WAIT_LIMIT_DEFAULT)
    assert np.all(np.isnan(bad)), "a wait that ran out must show in y"
    assert np.array_equal(run().view(np.uint32), ref.view(np.uint32))
