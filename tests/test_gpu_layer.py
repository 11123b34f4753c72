"""GPU parity of the whole decode MoE layer (router -> top-k -> experts ->
combine -> bf16) against the oracle: the 896-expert, top-16 layer at full
size (15.7 GB of packed experts resident), plus small layers covering k = 1,
k = n and ragged expert shapes. y (fp32 before the cast): normwise <= 1e-5;
top-k indices bit-exact; weights within 1e-6; the bf16 cast bit-exact
against round-to-nearest-even of the GPU's own fp32 y; reruns
bit-identical; the stage-by-stage calls give the same bits as the layer.

The layer's last launch folds the combine into the down projection (its
workgroups hand partials over through arrival slots marked with a per-call
value); the stage-by-stage calls run down and combine as two launches. Both
must give identical bits, also on workspaces that start as random bytes and
over runs of calls with changing tokens on one workspace."""
import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
import oracle
from gen import device as D
from gen import workloads as W
from tests._gpu import (TOL, assert_same, empty, layer_outputs, make_cache, normwise,
                        pinned_copy, say, up)

pytestmark = pytest.mark.gpu


def run_layer(pool, R_d, x, n, hidden, inter, k):
    import torch
    ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    idx = empty(k, torch.int32)
    w = empty(k, torch.float32)
    lg = empty(n, torch.float64)
    xd = up(x)
    K.k3_moe_layer_ex(xd, R_d, pool.table, n, hidden, inter, k, y, ws, y_f32=y32, idx=idx, w=w,
                      logits=lg)
    out = dict(y=y.cpu().numpy().view(np.uint16), y32=y32.cpu().numpy(), idx=idx.cpu().numpy(),
               w=w.cpu().numpy(), logits=lg.cpu().numpy())
    # rerun: bit-identical, and the plain entry point gives the same bf16 bits
    y2 = empty(hidden, torch.int16)
    K.k3_moe_layer(xd, R_d, pool.table, n, hidden, inter, k, y2, ws)
    assert np.array_equal(y2.cpu().numpy().view(np.uint16), out["y"]), "rerun differs"
    # stage by stage through the public calls
    h = empty((k, inter), torch.float32)
    yp = empty((k, hidden), torch.float32)
    y3 = empty(hidden, torch.float32)
    K.k3_expert_gate_up(xd, pool.table, idx, k, hidden, inter, h)
    if n <= 1024:  # the layer's own first stage: top-k inside gate/up
        h2 = empty((k, inter), torch.float32)
        idx2 = empty(k, torch.int32)
        w2 = empty(k, torch.float32)
        K.k3_expert_gate_up_routed(xd, lg, pool.table, n, k, hidden, inter, h2, idx2, w2)
        assert np.array_equal(idx2.cpu().numpy(), out["idx"])
        assert np.array_equal(w2.cpu().numpy().view(np.uint32), out["w"].view(np.uint32))
        assert np.array_equal(h2.cpu().numpy().view(np.uint32), h.cpu().numpy().view(np.uint32))
    K.k3_expert_down(h, pool.table, idx, k, hidden, inter, yp)
    K.k3_moe_combine(yp, w, k, hidden, None, y3)
    assert np.array_equal(y3.cpu().numpy().view(np.uint32), out["y32"].view(np.uint32))
    return out


def stage_outputs(pool, R_d, xd, n, hidden, inter, k):
    """The layer as separate public calls: router, routed gate/up, down,
    combine (two launches where the layer folds them into one)."""
    import torch
    lg = empty(n, torch.float64)
    h = empty((k, inter), torch.float32)
    idx = empty(k, torch.int32)
    w = empty(k, torch.float32)
    yp = empty((k, hidden), torch.float32)
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    K.k3_router(xd, R_d, 1, hidden, n, lg)
    K.k3_expert_gate_up_routed(xd, lg, pool.table, n, k, hidden, inter, h, idx, w)
    K.k3_expert_down(h, pool.table, idx, k, hidden, inter, yp)
    K.k3_moe_combine(yp, w, k, hidden, y, y32)
    return dict(y=y.cpu().numpy().view(np.uint16), y32=y32.cpu().numpy(),
                idx=idx.cpu().numpy(), w=w.cpu().numpy(), logits=lg.cpu().numpy())


def check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, elo, ehi, weights=None):
    """weights(e), when given, returns expert e's canonical weights (else
    they are generated from seed, cfg, elo and ehi)."""
    lg_ref = oracle.router_logits(x, R)
    assert np.max(np.abs(out["logits"] - lg_ref)) <= 1e-12 * np.max(np.abs(lg_ref))
    idx_ref, _ = oracle.topk(lg_ref, k)
    assert np.array_equal(out["idx"], idx_ref), (out["idx"], idx_ref)
    if weights is None:
        weights = lambda e: W.expert_weights(seed, cfg, e, hidden, inter, elo, ehi)  # noqa: E731
    experts = {int(e): weights(int(e)) for e in idx_ref}
    oracle.set_threads(16)
    y_ref, idx2, w_ref = oracle.moe_layer(x, R, experts, k, hidden, inter)
    assert np.array_equal(idx2, idx_ref)
    assert np.max(np.abs(out["w"] - w_ref)) <= 1e-6
    err = normwise(out["y32"], y_ref)
    assert err <= TOL, err
    assert np.array_equal(out["y"], oracle.f32_to_bf16(out["y32"]))
    keys = np.sort(lg_ref)[::-1]
    return err, (keys[k - 1] - keys[k]) if k < n else float("inf")


@pytest.fixture(scope="module")
def c3_pool():
    import torch
    say("building the 896-expert pool (7168/1536, 15.7 GB packed)")
    pool = D.build_expert_pool(0, W.C3, W.N_EXPERTS, log=say)
    R = W.router_bf16(0, W.C3)
    return pool, R, up(R)


@pytest.mark.parametrize("token", [0, 1, 2])
def test_decode_layer_c3_full_size(c3_pool, token):
    pool, R, R_d = c3_pool
    n, hidden, inter, k = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    x = W.tokens_bf16(0, W.C3, 1, hidden, batch=token)[0]
    say(f"decode layer C3 token {token}")
    out = run_layer(pool, R_d, x, n, hidden, inter, k)
    err, gap = check_against_oracle(out, x, R, 0, W.C3, n, hidden, inter, k, W.ELO, W.EHI)
    say(f"decode layer C3 token {token}: idx {out['idx'].tolist()} normwise {err:.3e} "
        f"gap {gap:.3e}")


@pytest.mark.parametrize("n,hidden,inter,k", [(20, 128, 64, 1), (12, 96, 160, 12),
                                              (40, 256, 96, 16), (70, 512, 1536, 64)])
def test_decode_layer_small(n, hidden, inter, k):
    cfg, seed = 70, 3
    say(f"decode layer n={n} hidden={hidden} inter={inter} k={k}")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    out = run_layer(pool, up(R), x, n, hidden, inter, k)
    check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, 114, 120)


def test_decode_layer_c3_shapes_with_exponent_255():
    """Experts of the C3 shape (7168/1536, top-16, so both stages of the
    expert launch run on the matrix unit) whose gate, up and down hold
    exponent byte 255 in about 8% of their groups: such a group contributes
    nothing ([A176] "What byte-identical actually costs"; [SAT] "Reduction
    one"), which the matrix route does by zeroing the group's codes before
    the product. Against the oracle, which skips the group; the layer's bits
    equal the stage-by-stage calls' (run_layer)."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    cfg, seed, n, hidden, inter, k = 74, 9, 24, W.HIDDEN, W.INTER, W.TOPK
    say(f"decode layer with exponent 255, n={n} hidden={hidden} inter={inter} k={k}")
    pool = ExpertPool(n, hidden, inter)
    ex = {}
    rng = np.random.default_rng(2550)
    for e in range(n):
        E = W.expert_weights(seed, cfg, e, hidden, inter, 114, 120)
        for part in ("gate", "up", "down"):
            nib, sc = E[part]
            sc = sc.copy()
            sc[rng.random(sc.shape) < 0.08] = 255
            E[part] = (nib, sc)
        ex[e] = E
        pool.load(e, E)
    torch.cuda.synchronize()
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    out = run_layer(pool, up(R), x, n, hidden, inter, k)
    assert all(int((ex[int(e)][p][1] == 255).sum()) > 0 for e in out["idx"]
               for p in ("gate", "up", "down"))
    err, _ = check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, 114, 120,
                                  weights=lambda e: ex[e])
    say(f"decode layer exponent 255: y {err:.3e}")


def test_decode_layer_c3_shapes_activation_group_off_the_digit_range():
    """x with one group of 32 values near 2^-100, below the range of the
    matrix unit's activation digits (2^-87): the expert launch's gate/up
    stage flags it while building x's digits and streams its tiles on the
    vector ALU instead; down (h in range) stays on the matrix unit. C3
    expert shape, top-16 of 24. Against the oracle; the layer's bits equal
    the stage-by-stage calls', which make the same choice."""
    cfg, seed, n, hidden, inter, k = 75, 10, 24, W.HIDDEN, W.INTER, W.TOPK
    say(f"decode layer with an x group near 2^-100, n={n} hidden={hidden} inter={inter} k={k}")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=4)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    f[32:64] *= np.float32(2.0 ** -100)  # exact: a power of two, far from underflow
    x = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.max(np.abs(f[32:64])) < 2.0 ** -87 and np.max(np.abs(f[32:64])) > 0
    out = run_layer(pool, up(R), x, n, hidden, inter, k)
    err, _ = check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, 114, 120)
    # The same token with that group zeroed (a zero group is in range) takes the
    # matrix route: the selection is the same and y agrees to rounding, but
    # not in every bit, since the two routes sum in different orders.
    import torch
    x0 = x.copy()
    x0[32:64] = 0
    ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    o0 = layer_outputs(pool, up(R), up(x0), n, hidden, inter, k, ws)
    assert np.array_equal(o0["idx"], out["idx"])
    assert normwise(o0["y32"], out["y32"]) <= TOL
    assert not np.array_equal(o0["y32"].view(np.uint32), out["y32"].view(np.uint32))
    say(f"decode layer, x group off the digit range: y {err:.3e}")


def test_decode_layer_c3_shapes_h_group_off_the_digit_range():
    """Every expert's gate and up rows 0..31 carry exponent byte 67
    (weights near 2^-60), so h's first group of 32 is near 2^-108: below
    the activation digits' range (2^-87), though an ordinary fp32 value.
    The expert launch's down stage flags it while building h's digits and
    streams on the vector ALU (its wait for the producers is then passed
    again, at once); gate/up stays on the matrix unit. C3 expert shape,
    top-16 of 24. Against the oracle; the layer's bits equal the
    stage-by-stage calls'."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    cfg, seed, n, hidden, inter, k = 76, 11, 24, W.HIDDEN, W.INTER, W.TOPK
    say(f"decode layer with an h group near 2^-108, n={n} hidden={hidden} inter={inter} k={k}")
    pool = ExpertPool(n, hidden, inter)
    ex = {}
    for e in range(n):
        E = W.expert_weights(seed, cfg, e, hidden, inter, 114, 120)
        for part in ("gate", "up"):
            nib, sc = E[part]
            sc = sc.copy()
            sc[:32, :] = 67
            E[part] = (nib, sc)
        ex[e] = E
        pool.load(e, E)
    torch.cuda.synchronize()
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    out = run_layer(pool, up(R), x, n, hidden, inter, k)
    err, _ = check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, 114, 120,
                                  weights=lambda e: ex[e])
    # h's first group is in the flagged range for every selected expert
    xf = oracle.bf16_to_f64(x)
    for e in out["idx"][:4]:
        g = oracle.gemv(*ex[int(e)]["gate"], xf)[:32]
        u = oracle.gemv(*ex[int(e)]["up"], xf)[:32]
        h = g / (1.0 + np.exp(-g)) * u
        assert 0 < np.max(np.abs(h)) < 2.0 ** -87, np.max(np.abs(h))
    say(f"decode layer, h group off the digit range: y {err:.3e}")


def test_decode_layer_4096_experts_top64():
    """The largest selection the ABI takes: 4096 experts (beyond 1024 the
    layer ranks with the separate top-k launch), k = 64, small experts."""
    n, hidden, inter, k, cfg, seed = K.K3_MAX_EXPERTS, 64, 32, K.K3_MAX_TOPK, 71, 4
    say("decode layer n=4096 k=64 (separate launches)")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=4)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.05).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    out = run_layer(pool, up(R), x, n, hidden, inter, k)
    check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, 114, 120)


def test_decode_layer_largest_expert_shape():
    """hidden = K3_MAX_HIDDEN (16384) and inter = K3_MAX_INTER (4096): 107 MB
    per expert, through the single expert launch."""
    n, hidden, inter, k, cfg, seed = 8, 16384, 4096, 2, 72, 5
    say("decode layer hidden=16384 inter=4096 k=2")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=4)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    x = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_TOKENS), hidden)
    out = run_layer(pool, up(R), x, n, hidden, inter, k)
    check_against_oracle(out, x, R, seed, cfg, n, hidden, inter, k, 114, 120)


def test_layer_over_many_tokens_on_one_workspace():
    """Twenty calls in a row on one workspace that starts as random bytes,
    a new token each time (every call must wait on its own arrival values,
    not on a previous call's); each compared bit for bit with the
    stage-by-stage calls, and the first and last with the oracle."""
    import torch
    cfg, seed, n, hidden, inter, k = 74, 8, 48, 384, 224, 8
    say("layer: 20 tokens on one random-filled workspace")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    R_d = up(R)
    nb = K.k3_moe_workspace_bytes(1, n, hidden, inter, k)
    ws = up(np.random.default_rng(1).integers(0, 256, nb, dtype=np.uint8))
    X = W.tokens_bf16(seed, cfg, 20, hidden)
    for t in range(20):
        xd = up(X[t])
        out = layer_outputs(pool, R_d, xd, n, hidden, inter, k, ws)
        assert_same(out, stage_outputs(pool, R_d, xd, n, hidden, inter, k))
        if t in (0, 19):
            check_against_oracle(out, X[t], R, seed, cfg, n, hidden, inter, k, 114, 120)


def test_layer_calls_on_two_streams(c3_pool):
    """Layer calls issued on two streams with two workspaces, alternating
    from one host thread and then from two host threads at once, with no
    synchronisation between the streams: every output equals, bit for bit,
    the same token's output from one stream alone, and is within 1e-5 of
    the oracle (the library orders its whole-grid expert launches across
    streams, so they never hold the device together)."""
    import threading
    import torch
    pool, R, R_d = c3_pool
    n, hidden, inter, k = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    X = W.tokens_bf16(0, W.C3, 2, hidden, batch=11)
    xs = [up(X[0]), up(X[1])]
    ws = [empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8) for _ in range(2)]
    ref = [layer_outputs(pool, R_d, xs[i], n, hidden, inter, k, ws[0]) for i in range(2)]
    for i in range(2):
        err, _ = check_against_oracle(ref[i], X[i], R, 0, W.C3, n, hidden, inter, k, W.ELO, W.EHI)
        say(f"two streams: token {i} normwise {err:.3e} against the oracle")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    reps = 6
    outs = [[empty(hidden, torch.float32) for _ in range(2 * reps)] for _ in range(2)]
    ybf = [[empty(hidden, torch.int16) for _ in range(2 * reps)] for _ in range(2)]
    torch.cuda.synchronize()

    def issue(i, r):
        K.k3_moe_layer_ex(xs[i], R_d, pool.table, n, hidden, inter, k, ybf[i][r], ws[i],
                          y_f32=outs[i][r], stream=streams[i])

    say("two streams: alternating calls from one thread")
    for r in range(reps):
        issue(0, r)
        issue(1, r)
    torch.cuda.synchronize()
    say("two streams: two host threads at once")
    errs = []

    def worker(i):
        try:
            for r in range(reps, 2 * reps):
                issue(i, r)
        except Exception as e:  # reported by the main thread
            errs.append(e)
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i in range(2):
        want = ref[i]["y32"].view(np.uint32)
        for r in range(2 * reps):
            got = outs[i][r].cpu().numpy().view(np.uint32)
            assert np.array_equal(got, want), (i, r)
            assert np.array_equal(ybf[i][r].cpu().numpy().view(np.uint16), ref[i]["y"]), (i, r)
    say(f"two streams: {2 * 2 * reps} calls bit-identical to the one-stream outputs")


def test_layer_c3_tokens_in_a_row(c3_pool):
    """Eight C3 tokens back to back on one workspace, each bit-identical to the
    stage-by-stage calls (the full-size grid: 768 gate/up and 1792 down
    tiles)."""
    import torch
    pool, R, R_d = c3_pool
    n, hidden, inter, k = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    X = W.tokens_bf16(0, W.C3, 8, hidden, batch=5)
    say("layer: 8 C3 tokens in a row")
    for t in range(8):
        xd = up(X[t])
        out = layer_outputs(pool, R_d, xd, n, hidden, inter, k, ws)
        assert_same(out, stage_outputs(pool, R_d, xd, n, hidden, inter, k))


def test_cached_layer_c3_full_size(c3_pool):
    """The C3 layer with the 896 experts in pinned host memory behind a
    40-slot HBM cache: six tokens, each bit-identical (y, fp32 y, indices,
    weights) to the layer on the resident pool, the first and the last
    within 1e-5 of the oracle, the cache's counters equal to the host replay
    of its trace."""
    import torch
    pool, R, R_d = c3_pool
    n, hidden, inter, k = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    say("cached layer C3: pinned host copy of the 896 experts, 40 slots")
    host = pinned_copy(pool)
    ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    X = W.tokens_bf16(0, W.C3, 6, hidden, batch=7)
    c = make_cache(pool, host, 40)
    try:
        trace = []
        for t in range(6):
            xd = up(X[t])
            want = layer_outputs(pool, R_d, xd, n, hidden, inter, k, ws)
            y = empty(hidden, torch.int16)
            y32 = empty(hidden, torch.float32)
            idx = empty(k, torch.int32)
            w = empty(k, torch.float32)
            K.k3_moe_layer_cached(xd, R_d, c, n, hidden, inter, k, y, ws, y_f32=y32, idx=idx,
                                  w=w)
            assert np.array_equal(idx.cpu().numpy(), want["idx"])
            assert np.array_equal(w.cpu().numpy().view(np.uint32), want["w"].view(np.uint32))
            assert np.array_equal(y32.cpu().numpy().view(np.uint32), want["y32"].view(np.uint32))
            assert np.array_equal(y.cpu().numpy().view(np.uint16), want["y"])
            trace.extend(want["idx"].tolist())
            if t in (0, 5):  # the cached layer against the oracle itself
                lg = empty(n, torch.float64)
                K.k3_router(xd, R_d, 1, hidden, n, lg)
                got = dict(y=y.cpu().numpy().view(np.uint16), y32=y32.cpu().numpy(),
                           idx=idx.cpu().numpy(), w=w.cpu().numpy(), logits=lg.cpu().numpy())
                err, _ = check_against_oracle(got, X[t], R, 0, W.C3, n, hidden, inter, k,
                                              W.ELO, W.EHI)
                say(f"cached layer C3 token {t}: normwise {err:.3e} against the oracle")
        st = K.k3_cache_get_stats(c)
        ref = K.k3_cache_replay(np.array(trace, np.int32), n, 40, (), k)
        ref["bytes_copied"] = st["misses"] * pool.expert_bytes
        assert st == ref, (st, ref)
        say(f"cached layer C3: {st}")
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)
        del host


def test_layer_with_shared_experts_c3_full_size(c3_pool):
    """The C3 layer with two 7168/1536 bf16 shared experts (132 MB): indices
    bit-exact, y within 1e-5 of the oracle's layer with shared experts."""
    import torch
    pool, R, R_d = c3_pool
    n, hidden, inter, k = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    say("layer with 2 shared experts, C3")
    shared = W.shared_experts_bf16(0, W.C3)
    blobs = [up(np.concatenate([S["gate"].ravel(), S["up"].ravel(), S["down"].ravel()]))
             for S in shared]
    table = up(np.array([b.data_ptr() for b in blobs], np.uint64))
    ws = empty(K.k3_moe_layer_shared_workspace_bytes(n, hidden, inter, k, 2, inter),
               torch.uint8)
    x = W.tokens_bf16(0, W.C3, 1, hidden, batch=11)[0]
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    idx = empty(k, torch.int32)
    K.k3_moe_layer_shared(up(x), R_d, pool.table, n, hidden, inter, k, table, 2, inter, y, ws,
                          y_f32=y32, idx=idx)
    lg = oracle.router_logits(x, R)
    idx_ref, _ = oracle.topk(lg, k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    experts = {int(e): W.expert_weights(0, W.C3, int(e)) for e in idx_ref}
    oracle.set_threads(16)
    y_ref, _, _ = oracle.moe_layer_shared(x, R, experts, k, hidden, inter, shared)
    assert normwise(y32.cpu().numpy(), y_ref) <= TOL


def test_layer_in_a_captured_graph():
    """Captured into a HIP graph, the layer takes the separate launches (its
    single expert launch marks stages with a per-call value a replay would
    repeat). Replays with new tokens copied into the captured input must
    match eager calls bit for bit and the oracle within 1e-5; eager work
    and synchronisation run between the replays."""
    import torch
    cfg, seed, n, hidden, inter, k = 75, 9, 32, 256, 160, 6
    say("layer in a captured graph: 4 replays")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    R_d = up(R)
    X = W.tokens_bf16(seed, cfg, 4, hidden)
    ws = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    xin = empty(hidden, torch.int16)
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    s = torch.cuda.Stream()
    xin.copy_(up(X[0]))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        K.k3_moe_layer_ex(xin, R_d, pool.table, n, hidden, inter, k, y, ws, y_f32=y32,
                          stream=s)
    ws_e = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    for t in range(4):
        xin.copy_(up(X[t]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y32.cpu().numpy().copy()
        eager = layer_outputs(pool, R_d, up(X[t]), n, hidden, inter, k, ws_e)
        # the eager layer runs the single expert launch; the replay the
        # separate ones, whose bits the stage-by-stage calls give
        stages = stage_outputs(pool, R_d, up(X[t]), n, hidden, inter, k)
        assert np.array_equal(got.view(np.uint32), stages["y32"].view(np.uint32)), t
        assert np.array_equal(got.view(np.uint32), eager["y32"].view(np.uint32)), t
        experts = {e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120) for e in range(n)}
        y_ref, _, _ = oracle.moe_layer(X[t], R, experts, k, hidden, inter)
        assert normwise(got, y_ref) <= TOL
