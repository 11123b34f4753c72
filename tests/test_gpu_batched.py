"""GPU parity of batched decode through the C ABI against the oracle.

- The token->expert permutation (counts, offsets, pair token and slot) is
  compared bit-exactly with the oracle's stable sort by (expert, token),
  including duplicates inside a token, out-of-range entries, one token and
  batches of several thousand pairs.
- The batched layer from given logits and through the router: top-k indices
  bit-exact; each token's fp32 output within 1e-5 normwise of the oracle's
  per-token layer; bf16 output bit-exact against RNE of the GPU's own fp32;
  reruns bit-identical.
- The C4 workload at full size: 64 tokens with Zipf(1.1)-skewed logits over
  the 896-expert pool (15.7 GB resident). Every token's routing and output is
  compared with the oracle, and batch invariance is reported.
- Edge exponent bytes on both the short and the steady K paths, and NaN or
  infinite activations inside groups whose exponent byte is 255.
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


def gpu_permute(idx, n):
    import torch
    T, k = idx.shape
    counts = empty(n, torch.int32)
    offsets = empty(n, torch.int32)
    pt = empty(T * k, torch.int32)
    ps = empty(T * k, torch.int32)
    ws = empty(K.k3_moe_permute_workspace_bytes(T, k), torch.uint8)
    K.k3_moe_permute(up(idx.astype(np.int32)), T, k, n, counts, offsets, pt, ps, ws)
    return [a.cpu().numpy() for a in (counts, offsets, pt, ps)]


def check_permutation(idx, n):
    c, o, pt, ps = gpu_permute(idx, n)
    rc, ro, rpt, rps = oracle.permute(idx, n)
    P = int(rc.sum())
    assert np.array_equal(c, rc) and np.array_equal(o, ro)
    assert np.array_equal(pt[:P], rpt[:P]) and np.array_equal(ps[:P], rps[:P])
    return c


# (2048, 16, 896) and (100, 64, 4096): chunks of 64 tokens placed by workgroups
# of their own; (16448, 4, 64): 257 chunks, one workgroup places them all.
@pytest.mark.parametrize("T,k,n", [(64, 16, 896), (1, 1, 1), (1, 16, 896), (3, 5, 7),
                                   (2048, 16, 896), (100, 64, 4096), (37, 8, 13),
                                   (16448, 4, 64)])
def test_permute_matches_oracle(T, k, n):
    say(f"permute T={T} k={k} n={n}")
    rng = np.random.default_rng(T * 1000 + k)
    idx = np.stack([rng.choice(n, k, replace=False) if k <= n else rng.integers(0, n, k)
                    for _ in range(T)]).astype(np.int32)
    check_permutation(idx, n)


def test_permute_duplicates_within_a_token():
    say("permute with repeated experts inside a token")
    rng = np.random.default_rng(7)
    idx = rng.integers(0, 5, size=(40, 6)).astype(np.int32)
    check_permutation(idx, 5)


def test_permute_exact_and_fast_chunks_mixed():
    """Chunks of 64 tokens that take the exact path (a repeated expert inside
    a token, an out-of-range entry) between chunks that take the fast one,
    with every entry of a chunk held by one thread, and 33 chunks (each entry
    read from device memory)."""
    rng = np.random.default_rng(11)
    for T, k, n in ((300, 8, 896), (2112, 16, 896)):
        say(f"permute with mixed chunks T={T} k={k} n={n}")
        idx = np.stack([rng.choice(n, k, replace=False) for _ in range(T)]).astype(np.int32)
        idx[5, 1] = idx[5, 0]          # chunk 0: repeated expert
        idx[130, 3] = idx[130, 2]      # chunk 2
        idx[200, 0] = n + 3            # chunk 3: out of range
        keep = (idx >= 0) & (idx < n)
        c, o, pt, ps = gpu_permute(idx, n)
        ref = sorted(((t, j) for t in range(T) for j in range(k) if keep[t, j]),
                     key=lambda p: (idx[p], p[0], p[1]))
        assert c.sum() == keep.sum()
        assert np.array_equal(c, np.bincount(idx[keep], minlength=n))
        assert pt[:len(ref)].tolist() == [t for t, _ in ref]
        assert ps[:len(ref)].tolist() == [j for _, j in ref]


def test_permute_skips_out_of_range_entries():
    say("permute with entries outside [0, n)")
    idx = np.array([[0, 3, -1], [5, 2, 2], [1, 99, 0]], np.int32)
    c, o, pt, ps = gpu_permute(idx, 4)
    keep = [(t, j) for t in range(3) for j in range(3) if 0 <= idx[t, j] < 4]
    ref = sorted(keep, key=lambda p: (idx[p], p[0], p[1]))
    assert c.tolist() == [2, 1, 2, 1] and o.tolist() == [0, 2, 3, 5]
    assert pt[:6].tolist() == [t for t, _ in ref] and ps[:6].tolist() == [j for _, j in ref]


def run_batched(pool, X, n, hidden, inter, k, logits=None, R_d=None, bias=None):
    import torch
    T = X.shape[0]
    ws = empty(K.k3_moe_batched_workspace_bytes(T, n, hidden, inter, k), torch.uint8)
    Y = empty((T, hidden), torch.int16)
    Y32 = empty((T, hidden), torch.float32)
    idx = empty((T, k), torch.int32)
    w = empty((T, k), torch.float32)
    Xd = up(X)
    b = None if bias is None else up(np.asarray(bias, np.float32))

    def call(Yo, Y32o):
        if logits is not None:
            K.k3_moe_layer_from_logits(Xd, up(np.asarray(logits, np.float64)), b, pool.table,
                                       n, hidden, inter, k, T, Yo, ws, Y_f32=Y32o, idx=idx,
                                       w=w)
        else:
            K.k3_moe_layer_batched(Xd, R_d, pool.table, n, hidden, inter, k, T, Yo, ws,
                                   Y_f32=Y32o, idx=idx, w=w)

    call(Y, Y32)
    out = dict(Y=Y.cpu().numpy().view(np.uint16), Y32=Y32.cpu().numpy(),
               idx=idx.cpu().numpy(), w=w.cpu().numpy())
    Y2 = empty((T, hidden), torch.float32)
    call(None, Y2)
    assert np.array_equal(Y2.cpu().numpy().view(np.uint32), out["Y32"].view(np.uint32)), \
        "rerun differs"
    assert np.array_equal(out["Y"], oracle.f32_to_bf16(out["Y32"]))
    return out


def check_tokens(out, X, logits, experts_of, k, hidden, inter, tokens):
    """Oracle layer from the same logits for the given tokens."""
    oracle.set_threads(16)
    errs = []
    for t in tokens:
        idx_ref, w_ref = oracle.topk(logits[t], k)
        assert np.array_equal(out["idx"][t], idx_ref), (t, out["idx"][t], idx_ref)
        assert np.max(np.abs(out["w"][t] - w_ref)) <= 1e-6
        ex = {int(e): experts_of(int(e)) for e in idx_ref}
        Y_ref, _, _ = oracle.moe_from_logits(X[t:t + 1], logits[t:t + 1], ex, k, hidden, inter)
        err = normwise(out["Y32"][t], Y_ref[0])
        assert err <= TOL, (t, err)
        errs.append(err)
    return max(errs)


# hidden 800: 25 groups (a last quad of one group) and K long enough for the
# matrix-unit gate/up's steady loop; inter 96: 3 gate/up tiles (a padding wave)
@pytest.mark.parametrize("n,hidden,inter,k,T", [(24, 256, 128, 4, 10), (13, 96, 160, 13, 5),
                                                (40, 512, 96, 16, 33), (9, 128, 64, 1, 70),
                                                (12, 800, 96, 4, 40)])
def test_batched_from_logits_small(n, hidden, inter, k, T):
    cfg, seed = 71, 4
    say(f"batched from logits n={n} hidden={hidden} inter={inter} k={k} T={T}")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    X = W.tokens_bf16(seed, cfg, T, hidden)
    logits = W.zipf_router_logits(seed, T, n, 1.1, cfg).astype(np.float64)
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits)
    err = check_tokens(out, X, logits,
                       lambda e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120),
                       k, hidden, inter, range(T))
    say(f"batched small: max normwise {err:.3e}")


@pytest.mark.parametrize("case", ["all_equal", "coarse"])
def test_one_token_fused_topk_with_tied_logits(case):
    """T = 1 from logits takes the decode layer's fused launch. Its top-k
    either leaves the routing weights to the waves that combine (at most 64
    candidates: key ties among them, "coarse") or computes them on its
    single-wave path (more than 64: every logit equal). idx, w and y against
    the oracle, ties to the lower expert index."""
    cfg, seed = 73, 6
    n, hidden, inter, k = 96, 256, 128, 8
    say(f"fused top-k with tied logits ({case}) n={n} k={k}")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    X = W.tokens_bf16(seed, cfg, 1, hidden)
    if case == "all_equal":
        logits = np.full((1, n), 0.25)
    else:
        logits = np.round(W.zipf_router_logits(seed, 1, n, 1.1, cfg).astype(np.float64) * 4) / 4
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits)
    check_tokens(out, X, logits, lambda e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120),
                 k, hidden, inter, [0])


def _edge_exponent_expert(seed, cfg, e, hidden, inter, xmax_col):
    """An expert whose gate/up and down exponent bytes include 0, 1, 2 and
    255 at random places, and gate rows 0, 1 and 2 with exponent bytes 253, 254 and
    252 on a group holding a single code 0.5, at the column whose
    activations are smallest (xmax_col: max |x| per column), so that every
    product and sum stays finite in fp32. Those gate rows reach about 1e38;
    their up rows take exponent byte 60 (weights near 1e-20), so that h, and
    down's unscaled group sums of up to 32 * 6 * |h| (the group's exponent
    is applied after its sum), stay far inside the fp32 range."""
    E = W.expert_weights(seed, cfg, e, hidden, inter, 114, 120)
    rng = np.random.default_rng(1000 + e)
    c = int(np.argmin(xmax_col))
    g, j = c // 32, c % 32
    for part in ("gate", "up"):
        nib, sc = E[part]
        nib, sc = nib.copy(), sc.copy()
        rows, G = sc.shape
        hit = rng.random((rows, G)) < 0.08
        sc[hit] = rng.choice(np.array([0, 1, 2, 255], np.uint8), int(hit.sum()))
        if part == "gate":
            for r, ex in ((0, 253), (1, 254), (2, 252)):
                nib[r, 16 * g:16 * g + 16] = 0
                nib[r, 16 * g + j // 2] = 0x01 << (4 * (j % 2))  # element j: code 1 (0.5)
                sc[r, g] = ex
        else:
            sc[0:3, :] = 60
        E[part] = (nib, sc)
    nib, sc = E["down"]
    sc = sc.copy()
    hit = rng.random(sc.shape) < 0.08
    sc[hit] = rng.choice(np.array([0, 1, 2, 255], np.uint8), int(hit.sum()))
    E["down"] = (nib, sc)
    return E


def test_batched_edge_exponents():
    """Exponent bytes outside 2..252 (the matrix-unit stages' exact route)
    and 255 (skipped groups), at a K that runs the steady loop."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    from tests import _independent as I
    cfg, seed, n, hidden, inter, k, T = 74, 8, 6, 1024, 128, 3, 20
    say(f"batched edge exponents n={n} hidden={hidden} inter={inter} k={k} T={T}")
    X = W.tokens_bf16(seed, cfg, T, hidden)
    xmax_col = np.abs(I.bf16_to_float_bits(X.reshape(-1)).reshape(T, hidden)).max(axis=0)
    assert xmax_col.min() < 2.0  # 2^127 * 0.5 * max|x| stays below the fp32 maximum
    pool = ExpertPool(n, hidden, inter)
    ex = {e: _edge_exponent_expert(seed, cfg, e, hidden, inter, xmax_col) for e in range(n)}
    for e in range(n):
        pool.load(e, ex[e])
    torch.cuda.synchronize()
    logits = W.zipf_router_logits(seed, T, n, 1.1, cfg).astype(np.float64)
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits)
    assert np.all(np.isfinite(out["Y32"]))
    err = check_tokens(out, X, logits, lambda e: ex[e], k, hidden, inter, range(T))
    say(f"batched edge exponents: max normwise {err:.3e}")


def test_batched_edge_exponents_steady_down():
    """Edge exponent bytes (0, 1, 2, 253, 254, 255) with inter 768, so that
    down's K (24 groups, six quads) runs the steady loop of both down
    launches, and a batch whose experts get items of at most 5 pairs (the
    packed launch) and of more (one instruction per piece); every token
    against the oracle."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    from tests import _independent as I
    cfg, seed, n, hidden, inter, k, T = 77, 9, 6, 1024, 768, 3, 40
    say(f"batched edge exponents n={n} hidden={hidden} inter={inter} k={k} T={T}")
    X = W.tokens_bf16(seed, cfg, T, hidden)
    xmax_col = np.abs(I.bf16_to_float_bits(X.reshape(-1)).reshape(T, hidden)).max(axis=0)
    assert xmax_col.min() < 2.0
    pool = ExpertPool(n, hidden, inter)
    ex = {e: _edge_exponent_expert(seed, cfg, e, hidden, inter, xmax_col) for e in range(n)}
    for e in range(n):
        pool.load(e, ex[e])
    torch.cuda.synchronize()
    logits = W.zipf_router_logits(seed, T, n, 1.1, cfg).astype(np.float64)
    idx = np.stack([oracle.topk(logits[t], k)[0] for t in range(T)])
    counts = np.bincount(idx.ravel(), minlength=n)
    items = [min(16, c - i) for c in counts.tolist() if c for i in range(0, c, 16)]
    assert min(items) <= 5 < max(items), items
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits)
    assert np.all(np.isfinite(out["Y32"]))
    err = check_tokens(out, X, logits, lambda e: ex[e], k, hidden, inter, range(T))
    say(f"batched edge exponents (steady down): max normwise {err:.3e}")


def test_batched_nonfinite_x_in_skipped_group():
    """NaN and infinite activations inside a gate/up group whose exponent
    byte is 255 in every row: the group is skipped, not multiplied by zero,
    so the rows stay finite and match the oracle, which skips it ([A176]
    "What byte-identical actually costs")."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    cfg, seed, n, hidden, inter, k, T = 78, 11, 8, 1024, 256, 3, 6
    say(f"batched layer, NaN/Inf x inside 255 groups, T={T}")
    X = W.tokens_bf16(seed, cfg, T, hidden).copy()
    g0 = 9
    X[:, 32 * g0 + 5] = 0x7F80            # +Inf
    X[1::2, 32 * g0 + 17] = 0xFF80        # -Inf
    X[::3, 32 * g0 + 30] = 0x7FC0         # NaN
    pool = ExpertPool(n, hidden, inter)
    ex = {}
    for e in range(n):
        E = W.expert_weights(seed, cfg, e, hidden, inter, 114, 120)
        for part in ("gate", "up"):
            nib, sc = E[part]
            sc = sc.copy()
            sc[:, g0] = 255
            E[part] = (nib, sc)
        ex[e] = E
        pool.load(e, E)
    torch.cuda.synchronize()
    logits = W.zipf_router_logits(seed, T, n, 1.1, cfg).astype(np.float64)
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits)
    assert np.all(np.isfinite(out["Y32"]))
    err = check_tokens(out, X, logits, lambda e: ex[e], k, hidden, inter, range(T))
    say(f"batched NaN/Inf in skipped groups: max normwise {err:.3e}")


def test_batched_router_path_small():
    cfg, seed, n, hidden, inter, k, T = 72, 5, 30, 256, 128, 6, 12
    say("batched layer through the router")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(seed, cfg, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(
        n, hidden)
    X = W.tokens_bf16(seed, cfg, T, hidden)
    out = run_batched(pool, X, n, hidden, inter, k, R_d=up(R))
    oracle.set_threads(16)
    ex_all = {e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120) for e in range(n)}
    for t in range(T):
        y_ref, idx_ref, _ = oracle.moe_layer(X[t], R, ex_all, k, hidden, inter)
        assert np.array_equal(out["idx"][t], idx_ref)
        assert normwise(out["Y32"][t], y_ref) <= TOL


@pytest.fixture(scope="module")
def c4_pool():
    say("building the 896-expert pool (7168/1536, 15.7 GB packed)")
    return D.build_expert_pool(0, W.C3, W.N_EXPERTS, log=say)


def _cached(fn):
    memo = {}

    def get(e):
        if e not in memo:
            memo[e] = fn(e)
        return memo[e]
    return get


def test_batched_c4_full_size(c4_pool):
    """The C4 workload at full size, every one of its 64 tokens against the
    oracle. Also reports (a printed fact, not a gate) whether the batched
    path is batch-invariant: each token's fp32 output beside the same
    token's single-token decode launch, bit for bit."""
    import torch
    n, hidden, inter, k, T = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK, 64
    say("batched decode C4: 64 tokens, Zipf(1.1) logits, top-16 of 896")
    X = W.tokens_bf16(0, W.C4, T, hidden)
    logits = W.zipf_router_logits(0, T, n, 1.1, W.C4).astype(np.float64)
    out = run_batched(c4_pool, X, n, hidden, inter, k, logits=logits)
    for t in range(T):
        idx_ref, _ = oracle.topk(logits[t], k)
        assert np.array_equal(out["idx"][t], idx_ref), t
    counts = check_permutation(out["idx"], n)
    distinct = int((counts > 0).sum())
    say(f"C4 distinct experts {distinct}, hottest expert on {int(counts.max())} tokens")
    assert 250 <= distinct <= 420
    # both down launches run: items (runs cut at 16 tokens) of <= 5 and > 5 pairs
    items = [min(16, c - i) for c in counts.tolist() if c for i in range(0, c, 16)]
    assert min(items) <= 5 < max(items), items
    err = check_tokens(out, X, logits,
                       _cached(lambda e: W.expert_weights(0, W.C3, e, hidden, inter)),
                       k, hidden, inter, range(T))
    say(f"C4 all 64 tokens: max normwise {err:.3e}")
    # batch invariance (reported): the same token alone through the decode launch
    ws1 = empty(K.k3_moe_batched_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    same, worst = 0, 0.0
    for t in range(T):
        Y1 = empty((1, hidden), torch.float32)
        K.k3_moe_layer_from_logits(up(X[t:t + 1]), up(logits[t:t + 1]), None, c4_pool.table,
                                   n, hidden, inter, k, 1, None, ws1, Y_f32=Y1)
        y1 = Y1.cpu().numpy()[0]
        same += int(np.array_equal(y1.view(np.uint32), out["Y32"][t].view(np.uint32)))
        worst = max(worst, normwise(out["Y32"][t], y1))
    say(f"C4 batch invariance: {same} of {T} tokens bit-identical to their single-token "
        f"decode launch; max normwise difference {worst:.3e}")


def test_one_token_from_logits_takes_the_decode_launch(c4_pool):
    """T = 1 without a bias runs the single-token decode layer's expert
    launch (the launch the decode layer makes after its router, and the one
    the benchmark times): bit-identical to k3_moe_layer_ex on the same token
    and router, and within 1e-5 of the oracle, over several tokens on one
    workspace."""
    import torch
    n, hidden, inter, k = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    R = W.router_bf16(0, W.C3)
    R_d = up(R)
    X = W.tokens_bf16(0, W.C3, 4, hidden, batch=9)
    wsb = empty(K.k3_moe_batched_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    wsl = empty(K.k3_moe_workspace_bytes(1, n, hidden, inter, k), torch.uint8)
    say("one token from logits vs the decode layer")
    for t in range(4):
        xd = up(X[t:t + 1])
        lg = empty((1, n), torch.float64)
        K.k3_router(xd, R_d, 1, hidden, n, lg)
        Y = empty((1, hidden), torch.int16)
        Y32 = empty((1, hidden), torch.float32)
        idx = empty((1, k), torch.int32)
        w = empty((1, k), torch.float32)
        K.k3_moe_layer_from_logits(xd, lg, None, c4_pool.table, n, hidden, inter, k, 1, Y, wsb,
                                   Y_f32=Y32, idx=idx, w=w)
        y = empty(hidden, torch.int16)
        y32 = empty(hidden, torch.float32)
        K.k3_moe_layer_ex(xd, R_d, c4_pool.table, n, hidden, inter, k, y, wsl, y_f32=y32)
        assert np.array_equal(Y32.cpu().numpy()[0].view(np.uint32), y32.cpu().numpy().view(np.uint32))
        assert np.array_equal(Y.cpu().numpy()[0], y.cpu().numpy())
        if t == 0:
            out = dict(idx=idx.cpu().numpy(), w=w.cpu().numpy(), Y32=Y32.cpu().numpy())
            err = check_tokens(out, X[t:t + 1], lg.cpu().numpy(),
                               lambda e: W.expert_weights(0, W.C3, e, hidden, inter),
                               k, hidden, inter, [0])
            say(f"one token from logits: normwise {err:.3e}")


def test_batched_layer_with_routing_bias():
    """The routing bias steers selection only ([ZOR] "How is the C engine
    actually built?", invariant 3): batched layer from logits with a bias
    against the oracle's layer with the same bias (selection on sigmoid +
    bias, weights from the unbiased scores)."""
    cfg, seed, n, hidden, inter, k, T = 76, 10, 40, 256, 128, 6, 9
    say("batched layer with a routing bias")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    X = W.tokens_bf16(seed, cfg, T, hidden)
    logits = W.zipf_router_logits(seed, T, n, 1.1, cfg).astype(np.float64)
    bias = W.routing_bias(seed, n, 0.5).astype(np.float32)
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits, bias=bias)
    ex = {e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120) for e in range(n)}
    oracle.set_threads(16)
    Y_ref, idx_ref, w_ref = oracle.moe_from_logits(X, logits, ex, k, hidden, inter,
                                                   bias=bias.astype(np.float64))
    plain = np.stack([oracle.topk(logits[t], k)[0] for t in range(T)])
    assert not np.array_equal(np.sort(plain, 1), np.sort(idx_ref, 1)), "bias changed nothing"
    assert np.array_equal(out["idx"], idx_ref)
    assert np.max(np.abs(out["w"] - w_ref)) <= 1e-6
    for t in range(T):
        assert normwise(out["Y32"][t], Y_ref[t]) <= TOL, t


def test_batched_beyond_grid_y():
    """More tokens than the grid's y extent (65535): the combine strides over
    tokens."""
    cfg, seed, n, hidden, inter, k, T = 74, 7, 4, 64, 32, 1, 70000
    say(f"batched from logits, T={T} tokens")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    X = W.tokens_bf16(seed, cfg, T, hidden)
    logits = W.uniform_router_logits(seed, T, n, cfg).astype(np.float64)
    out = run_batched(pool, X, n, hidden, inter, k, logits=logits)
    err = check_tokens(out, X, logits,
                       lambda e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120),
                       k, hidden, inter, [0, 1, 65534, 65535, 65536, T - 1])
    say(f"T={T}: max normwise {err:.3e} on sampled tokens")
