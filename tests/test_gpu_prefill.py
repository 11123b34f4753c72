"""GPU parity of the prefill path (MXFP4 activations, FP4 x FP4 grouped
GEMMs on the block-scaled matrix instruction) through the C ABI, staged as
the quantiser's rounding makes necessary (GPU h in fp32 and oracle h in fp64
can sit on opposite sides of an E2M1 rounding boundary):

1. the quantiser: bit-exact against the oracle's on the same values
   (exact ties, saturation, zero blocks, signed zeros, subnormals, bf16 x);
2. gate/up: the GPU's fp32 h against the oracle's SiLU(gate) * up computed
   from the oracle's MXFP4 x MXFP4 products on the same quantised x,
   <= 1e-5 normwise per pair;
3. the fused quantisation of h: bit-exact against the oracle's quantiser
   applied to the GPU's own fp32 h;
4. down and combine: Y against the oracle's products on the GPU's quantised
   h, summed in rank order, <= 1e-5 normwise per token; top-k bit-exact;
   reruns bit-identical.
"""
import numpy as np
import pytest

import mxfp4_packed_weight_amd as K
import oracle
from gen import device as D
from gen import workloads as W
from tests._gpu import TOL, empty, normwise, say, up

pytestmark = pytest.mark.gpu


def gpu_quant(v, bf16=False):
    import torch
    rows, cols = v.shape
    nib = empty((rows, cols // 2), torch.uint8)
    sc = empty((rows, cols // 32), torch.uint8)
    if bf16:
        K.k3_mxfp4_quantize_bf16(up(v), rows, cols, nib, sc)
    else:
        K.k3_mxfp4_quantize_f32(up(np.asarray(v, np.float32)), rows, cols, nib, sc)
    return nib.cpu().numpy(), sc.cpu().numpy()


def bf16_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_quantizer_edge_cases():
    say("quantiser edge cases")
    rng = np.random.default_rng(3)
    blocks = []
    for E in [-130, -127, -20, -3, 0, 5, 100, 125]:
        s = np.float32(2.0) ** np.float32(max(E, -149))
        # exact ties and the saturation region, with amax = 4 * 2^E
        ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0, 5.5, 6.0, 7.9,
                         0.2, 0.3, 0.7, 0.8, 1.2, 1.3, 1.7, 1.8, 2.4, 2.6, 3.4, 3.6, 4.9,
                         5.1, 0.0, -0.0, -0.25, -0.75, -5.0, -2.5, -1.25], np.float32)
        blocks.append(ties * s)
    blocks.append(np.zeros(32, np.float32))
    blocks.append(np.full(32, -0.0, np.float32))
    blocks.append(np.array([1e-45] * 16 + [3e-45] * 16, np.float32))  # subnormals
    blocks.append(np.array([3.0e38, -1.0e-30] * 16, np.float32))
    for _ in range(64):
        blocks.append((rng.standard_normal(32) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32))
    v = np.stack(blocks).reshape(-1, 64)
    n, s = gpu_quant(v)
    rn, rs = oracle.mxfp4_quant(v.astype(np.float64))
    assert np.array_equal(s, rs), np.argwhere(s != rs)[:5]
    assert np.array_equal(n, rn), np.argwhere(n != rn)[:5]


def test_quantizer_bf16_tokens():
    say("quantiser on bf16 tokens")
    X = W.tokens_bf16(0, W.C5, 16, 7168)
    n, s = gpu_quant(X, bf16=True)
    rn, rs = oracle.mxfp4_quant(bf16_to_f64(X))
    assert np.array_equal(s, rs) and np.array_equal(n, rn)


def run_prefill(pool, X, logits, n, hidden, inter, k):
    import torch
    T = X.shape[0]
    P = T * k
    ws = empty(K.k3_moe_prefill_workspace_bytes(T, n, hidden, inter, k), torch.uint8)
    Y = empty((T, hidden), torch.int16)
    Y32 = empty((T, hidden), torch.float32)
    idx = empty((T, k), torch.int32)
    w = empty((T, k), torch.float32)
    h32 = empty((P, inter), torch.float32)
    hn = empty((P, inter // 2), torch.uint8)
    hs = empty((P, inter // 32), torch.uint8)
    Xd, Ld = up(X), up(np.asarray(logits, np.float64))
    K.k3_moe_prefill(Xd, Ld, None, pool.table, n, hidden, inter, k, T, Y, ws, Y_f32=Y32, idx=idx,
                     w=w, h_f32=h32, h_nib=hn, h_sc=hs)
    out = dict(Y=Y.cpu().numpy().view(np.uint16), Y32=Y32.cpu().numpy(), idx=idx.cpu().numpy(),
               w=w.cpu().numpy(), h32=h32.cpu().numpy(), hn=hn.cpu().numpy(),
               hs=hs.cpu().numpy())
    Y2 = empty((T, hidden), torch.float32)
    K.k3_moe_prefill(Xd, Ld, None, pool.table, n, hidden, inter, k, T, None, ws, Y_f32=Y2)
    assert np.array_equal(Y2.cpu().numpy().view(np.uint32), out["Y32"].view(np.uint32)), \
        "rerun differs"
    assert np.array_equal(out["Y"], oracle.f32_to_bf16(out["Y32"]))
    return out


def check_prefill(out, X, logits, experts_of, k, hidden, inter, tokens):
    """Stages 2-4 for the given tokens (stage 1 on all of X)."""
    T = X.shape[0]
    xn, xs = oracle.mxfp4_quant(bf16_to_f64(X))
    gn, gs = gpu_quant(X, bf16=True)
    assert np.array_equal(xn, gn) and np.array_equal(xs, gs)
    for t in range(T):
        idx_ref, _ = oracle.topk(logits[t], k)
        assert np.array_equal(out["idx"][t], idx_ref), t
    counts, offsets, pt, ps = oracle.permute(out["idx"], logits.shape[1])
    q_of = {(int(t), int(j)): q for q, (t, j) in enumerate(zip(pt, ps))}
    silu = np.vectorize(oracle.silu)
    errs_h, errs_y = [], []
    cache = {}
    for t in tokens:
        y = np.zeros(hidden, np.float64)
        idx_ref, w_ref = oracle.topk(logits[t], k)
        assert np.max(np.abs(out["w"][t] - w_ref)) <= 1e-6
        for j in range(k):
            e = int(out["idx"][t, j])
            if e not in cache:
                cache[e] = experts_of(e)
            E = cache[e]
            q = q_of[(t, j)]
            g = oracle.mxfp4_matmul(xn[t:t + 1], xs[t:t + 1], *E["gate"])[0]
            u = oracle.mxfp4_matmul(xn[t:t + 1], xs[t:t + 1], *E["up"])[0]
            with np.errstate(over="ignore"):
                h_ref = silu(g) * u
            errs_h.append(normwise(out["h32"][q], h_ref))
            assert errs_h[-1] <= TOL, (t, j, errs_h[-1])
            qn, qs = oracle.mxfp4_quant(out["h32"][q].astype(np.float64))
            assert np.array_equal(out["hn"][q], qn[0]) and np.array_equal(out["hs"][q], qs[0]), \
                (t, j)
            y += float(out["w"][t, j]) * oracle.mxfp4_matmul(qn, qs, *E["down"])[0]
        errs_y.append(normwise(out["Y32"][t], y))
        assert errs_y[-1] <= TOL, (t, errs_y[-1])
    return max(errs_h), max(errs_y)


# The GEMM kernels take a steady path when K has at least 4 quads of 128
# (K >= 512, with the weight ring two quads deep) and a short path below; tile groups of four are ragged when a
# matrix's tile count is not a multiple of 4, and the last quad is partial
# when K % 128 != 0. The last three cases put the steady path on gate/up,
# then on down (with experts of more than 64 tokens, two items each), with
# ragged tile groups and partial last quads.
@pytest.mark.parametrize("n,hidden,inter,k,T", [(12, 256, 128, 4, 40), (5, 96, 160, 5, 70),
                                                (30, 512, 96, 8, 200), (3, 128, 64, 1, 9),
                                                (10, 800, 224, 3, 50), (6, 288, 800, 2, 90),
                                                (4, 256, 800, 2, 200)])
def test_prefill_small(n, hidden, inter, k, T):
    cfg, seed = 73, 6
    say(f"prefill n={n} hidden={hidden} inter={inter} k={k} T={T}")
    pool = D.build_expert_pool(seed, cfg, n, hidden, inter, 114, 120, workers=2)
    X = W.tokens_bf16(seed, cfg, T, hidden)
    logits = W.uniform_router_logits(seed, T, n, cfg).astype(np.float64)
    out = run_prefill(pool, X, logits, n, hidden, inter, k)
    eh, ey = check_prefill(out, X, logits,
                           lambda e: W.expert_weights(seed, cfg, e, hidden, inter, 114, 120),
                           k, hidden, inter, range(T))
    say(f"prefill small: h {eh:.3e} y {ey:.3e}")


@pytest.fixture(scope="module")
def c5_pool():
    say("building the 896-expert pool (7168/1536, 15.7 GB packed)")
    return D.build_expert_pool(0, W.C3, W.N_EXPERTS, log=say)


def test_prefill_weight_exponent_255():
    """Weight groups with exponent byte 255 scattered through gate, up and
    down contribute nothing ([A176] "What byte-identical actually costs";
    [SAT] "Reduction one"), at K long enough for the steady path of both
    GEMMs (hidden 1024, inter 768); every token staged against the oracle,
    which skips those groups."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    cfg, seed, n, hidden, inter, k, T = 79, 12, 6, 1024, 768, 2, 60
    say(f"prefill with weight exponent 255, n={n} hidden={hidden} inter={inter} T={T}")
    pool = ExpertPool(n, hidden, inter)
    ex = {}
    rng = np.random.default_rng(255)
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
    assert all(int((ex[e][p][1] == 255).sum()) > 0 for e in range(n) for p in ("gate", "up", "down"))
    X = W.tokens_bf16(seed, cfg, T, hidden)
    logits = W.uniform_router_logits(seed, T, n, cfg).astype(np.float64)
    out = run_prefill(pool, X, logits, n, hidden, inter, k)
    eh, ey = check_prefill(out, X, logits, lambda e: ex[e], k, hidden, inter, range(T))
    say(f"prefill exponent 255: h {eh:.3e} y {ey:.3e}")


def test_prefill_c5_full_size(c5_pool):
    """The C5 workload at full size. Every pair of the most-loaded expert is
    checked through stages 2 and 3 (one oracle product over all its tokens),
    and whole tokens through stage 4: tokens 0, 1023, 2047 and the first,
    middle and last token of the most-loaded expert (its first and last
    tokens fall in different work items when it holds more than 64)."""
    n, hidden, inter, k, T = W.N_EXPERTS, W.HIDDEN, W.INTER, W.TOPK, 2048
    say("prefill C5: 2048 tokens, uniform logits, top-16 of 896")
    X = W.tokens_bf16(0, W.C5, T, hidden)
    logits = W.uniform_router_logits(0, T, n, W.C5).astype(np.float64)
    out = run_prefill(c5_pool, X, logits, n, hidden, inter, k)
    counts, offsets, pt, ps = oracle.permute(out["idx"], n)
    hot = int(np.argmax(counts))
    say(f"C5 experts used {int((counts > 0).sum())}, tokens per expert "
        f"{counts.mean():.1f} (max {int(counts.max())}, expert {hot})")
    # stages 2 and 3 on every pair of the most-loaded expert
    oracle.set_threads(16)
    E = W.expert_weights(0, W.C3, hot, hidden, inter)
    qs = np.arange(offsets[hot], offsets[hot] + counts[hot])
    toks = pt[qs]
    xn, xs = oracle.mxfp4_quant(bf16_to_f64(X[toks]))
    g = oracle.mxfp4_matmul(xn, xs, *E["gate"])
    u = oracle.mxfp4_matmul(xn, xs, *E["up"])
    silu = np.vectorize(oracle.silu)
    with np.errstate(over="ignore"):
        h_ref = silu(g) * u
    worst = 0.0
    for i, q in enumerate(qs):
        worst = max(worst, normwise(out["h32"][q], h_ref[i]))
        qn, qsc = oracle.mxfp4_quant(out["h32"][q].astype(np.float64))
        assert np.array_equal(out["hn"][q], qn[0]) and np.array_equal(out["hs"][q], qsc[0]), q
    assert worst <= TOL, worst
    say(f"C5 most-loaded expert {hot}: {len(qs)} pairs, h within {worst:.3e}")
    sample = sorted({0, 1023, 2047, int(toks[0]), int(toks[len(toks) // 2]), int(toks[-1])})
    eh, ey = check_prefill(out, X, logits,
                           lambda e: W.expert_weights(0, W.C3, e, hidden, inter),
                           k, hidden, inter, sample)
    say(f"C5 sampled tokens {sample}: h {eh:.3e} y {ey:.3e}")
