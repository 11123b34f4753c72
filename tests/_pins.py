"""Pin checks for the oracle. Each takes an ``oracle.Oracle`` instance and
raises AssertionError when the oracle disagrees with a fact fixed
independently of it. ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on builds with planted mistakes and
expects at least one to fail."""
import math
from fractions import Fraction

import numpy as np

import gen
from gen import workloads as W
from tests import _independent as I


def check_e2m1_table(O):
    for c in range(16):
        v = O.e2m1(c)
        assert Fraction(v) == I.e2m1_from_bits(c), (c, v)
        assert math.copysign(1.0, v) == (-1.0 if I.e2m1_signbit(c) else 1.0), c


def check_e8m0(O):
    for e in range(255):
        assert Fraction(O.e8m0(e)) == Fraction(2) ** (e - 127), e
    assert math.isnan(O.e8m0(255))


def check_golden_nibble_order(O):
    data, rows = I.read_golden_rows("e2m1_nibble_order.txt")
    nib = np.array([data] * len(rows), np.uint8)
    sc = np.array([[r[0]] for r in rows], np.uint8)
    expected = np.array([r[1] for r in rows])
    W_ = O.dequant(nib, sc)
    assert np.array_equal(W_, expected), "dequant differs from the hand-decoded fixture"
    assert np.array_equal(np.signbit(W_[:2]), np.signbit(expected[:2]))
    for j in range(32):  # one-hot x recovers column j exactly
        x = np.zeros(32)
        x[j] = 1.0
        y = O.gemv(nib, sc, x)
        assert np.array_equal(y, expected[:, j] + 0.0), (j, y, expected[:, j])


def check_bruteforce_4x32(O):
    """Every code at every position of every row of a 4x32 matrix, one-hot x."""
    rng_scales = [120, 127, 131, 134]
    for r in range(4):
        for p in range(32):
            for c in range(16):
                codes = np.zeros((4, 32), np.uint8)
                codes[r, p] = c
                nib = I.pack_codes(codes)
                sc = np.array([[s] for s in rng_scales], np.uint8)
                x = np.zeros(32)
                x[p] = 1.0
                y = O.gemv(nib, sc, x)
                exp = np.zeros(4)
                exp[r] = float(I.e2m1_from_bits(c) * Fraction(2) ** (rng_scales[r] - 127))
                assert np.array_equal(y, exp), (r, p, c, y)


def check_all_scale_bytes(O):
    codes = np.array([[(i * 7 + 3) % 16 for i in range(32)]], np.uint8)
    nib = I.pack_codes(codes)
    x = np.array([float(k % 5 - 2) for k in range(32)])
    base = sum(I.e2m1_from_bits(int(c)) * Fraction(v) for c, v in zip(codes[0], x))
    for e in range(256):
        y = O.gemv(nib, np.array([[e]], np.uint8), x)
        exp = 0 if e == 255 else base * Fraction(2) ** (e - 127)
        assert Fraction(y[0]) == exp, (e, y[0])


def check_exact_rational(O, rows=6, cols=256, seed=7):
    nib, sc = gen.mxfp4_matrix(seed, 99, rows, cols)
    sc[0, 3] = 255
    x = gen.normal_f32(gen.key(seed, 99, gen.KIND_TOKENS), cols)
    y = O.gemv(nib, sc, x.astype(np.float64))
    ys, mags = I.exact_gemv(nib, sc, x)
    n_add = 32 + cols // 32  # additions on any path through the nested sums
    for r in range(rows):
        bound = Fraction(n_add) * Fraction(2) ** -53 * mags[r] * Fraction(101, 100)
        assert abs(Fraction(y[r]) - ys[r]) <= bound, (r, float(Fraction(y[r]) - ys[r]))


def check_exact_dyadic(O, rows=5, cols=128, seed=3):
    """With x dyadic and small, every partial sum is exact: equality."""
    nib, sc = gen.mxfp4_matrix(seed, 98, rows, cols)
    x = np.array([((k * 37) % 13 - 6) * 0.25 for k in range(cols)])
    y = O.gemv(nib, sc, x)
    ys, _ = I.exact_gemv(nib, sc, x)
    for r in range(rows):
        assert Fraction(y[r]) == ys[r], r


def check_scale_shift(O):
    nib, sc = gen.mxfp4_matrix(11, 97, 8, 192, 121, 133)
    x = gen.normal_f32(gen.key(11, 97, gen.KIND_TOKENS), 192).astype(np.float64)
    y1 = O.gemv(nib, sc, x)
    y2 = O.gemv(nib, (sc + 1).astype(np.uint8), x)
    assert np.array_equal(y2, 2.0 * y1)


def check_nan_containment(O):
    nib, sc = gen.mxfp4_matrix(5, 96, 4, 128)
    x = gen.normal_f32(gen.key(5, 96, gen.KIND_TOKENS), 128).astype(np.float64)
    sc2 = sc.copy()
    sc2[:, 1] = 255
    xn = x.copy()
    xn[32:64] = np.nan
    xn[40] = np.inf
    y_nan = O.gemv(nib, sc2, xn)
    xz = x.copy()
    xz[32:64] = 0.0
    y_ref = O.gemv(nib, sc2, xz)
    assert np.all(np.isfinite(y_nan))
    assert np.array_equal(y_nan, y_ref)


def check_dequant_crosscheck(O):
    nib, sc, x = W.c1_inputs(seed=0)
    sc = sc.copy()
    sc[3, 5] = 255
    y = O.gemv(nib, sc, x.astype(np.float64))
    Wn = I.dequant_numpy(nib, sc)
    yn = Wn @ x.astype(np.float64)
    assert np.max(np.abs(y - yn)) <= 1e-12 * np.max(np.abs(yn))



def check_expert_crosscheck(O, hidden=256, inter=96, seed=21, elo=114, ehi=120):
    E = gen.expert(seed, 95, 0, hidden, inter, elo, ehi)
    x = I.bf16_to_float_bits(gen.normal_bf16(gen.key(seed, 95, gen.KIND_TOKENS), hidden))
    y, h = O.expert_swiglu(E, x)
    g = I.dequant_numpy(*E["gate"]) @ x
    u = I.dequant_numpy(*E["up"]) @ x
    hh = np.array([I.silu_tanh_form(a) for a in g]) * u
    yy = I.dequant_numpy(*E["down"]) @ hh
    assert np.max(np.abs(h - hh)) <= 1e-12 * np.max(np.abs(hh))
    assert np.max(np.abs(y - yy)) <= 1e-12 * np.max(np.abs(yy))


def check_shared_expert_crosscheck(O, hidden=320, inter=96, seed=22):
    """The shared expert (bf16 weights) against numpy: matrices widened from
    their bf16 bits, matmul, SiLU in its tanh form."""
    from gen import workloads as W
    S = W.shared_experts_bf16(seed, 96, 1, hidden, inter, 0.05)[0]
    x = I.bf16_to_float_bits(gen.normal_bf16(gen.key(seed, 96, gen.KIND_TOKENS), hidden))
    y, h = O.shared_expert(S, x)
    g = I.bf16_to_float_bits(S["gate"]) @ x
    u = I.bf16_to_float_bits(S["up"]) @ x
    hh = np.array([I.silu_tanh_form(a) for a in g]) * u
    yy = I.bf16_to_float_bits(S["down"]) @ hh
    assert np.max(np.abs(h - hh)) <= 1e-12 * np.max(np.abs(hh))
    assert np.max(np.abs(y - yy)) <= 1e-12 * np.max(np.abs(yy))


def check_shared_expert_by_hand(O):
    """hidden 32, inter 32: gate row i = 2 e_i, up row i = e_{i+1}, down =
    identity rows 0..31, x_j = j/8: h_i = SiLU(2 x_i) x_{i+1}, y = h."""
    n = 32
    def bf(a):
        return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gate = np.zeros((n, n)); up = np.zeros((n, n)); down = np.eye(n)
    for i in range(n):
        gate[i, i] = 2.0
        up[i, (i + 1) % n] = 1.0
    x = np.arange(n) / 8.0
    S = {"gate": bf(gate), "up": bf(up), "down": bf(down)}
    y, h = O.shared_expert(S, x)
    want = np.array([2 * x[i] / (1 + np.exp(-2 * x[i])) * x[(i + 1) % n] for i in range(n)])
    assert np.max(np.abs(h - want)) <= 1e-14 * np.max(np.abs(want))
    assert np.max(np.abs(y - want)) <= 1e-14 * np.max(np.abs(want))


def check_layer_shared_adds(O, seed=33):
    """The layer with shared experts is the routed layer plus each shared
    output (numpy-computed), added in order."""
    from gen import workloads as W
    n, hidden, inter, k, inter_s = 12, 128, 64, 3, 96
    R = gen.normal_bf16(gen.key(seed, 97, gen.KIND_ROUTER), n * hidden, 0, 0.05).reshape(n, hidden)
    x = gen.normal_bf16(gen.key(seed, 97, gen.KIND_TOKENS), hidden)
    experts = {e: gen.expert(seed, 97, e, hidden, inter, 114, 120) for e in range(n)}
    shared = W.shared_experts_bf16(seed, 97, 2, hidden, inter_s, 0.05)
    y0, idx0, w0 = O.moe_layer(x, R, experts, k, hidden, inter)
    y1, idx1, w1 = O.moe_layer_shared(x, R, experts, k, hidden, inter, shared)
    assert np.array_equal(idx0, idx1) and np.array_equal(w0, w1)
    xf = I.bf16_to_float_bits(x)
    want = y0.copy()
    for S in shared:
        g = I.bf16_to_float_bits(S["gate"]) @ xf
        u = I.bf16_to_float_bits(S["up"]) @ xf
        want += I.bf16_to_float_bits(S["down"]) @ (np.array([I.silu_tanh_form(a) for a in g]) * u)
    assert np.max(np.abs(y1 - want)) <= 1e-12 * np.max(np.abs(want))
    # no shared experts: the plain layer, bit for bit
    y2, _, _ = O.moe_layer_shared(x, R, experts, k, hidden, inter, [])
    assert np.array_equal(y2, y0)


def check_silu(O):
    assert O.silu(0.0) == 0.0
    for v in [0.1, 0.5, 1.0, 2.0, 5.0, 10.0, 30.0, 100.0, 1000.0]:
        for s in (1.0, -1.0):
            a, b = O.silu(s * v), I.silu_tanh_form(s * v)
            assert abs(a - b) <= 1e-15 * abs(b), (s * v, a, b)
    assert O.silu(1000.0) == 1000.0
    assert O.silu(-1000.0) == 0.0


def check_router_logits(O, n=40, hidden=320, seed=4):
    x = gen.normal_bf16(gen.key(seed, 94, gen.KIND_TOKENS), hidden)
    R = gen.normal_bf16(gen.key(seed, 94, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(n, hidden)
    l = O.router_logits(x, R)
    xf, Rf = I.bf16_to_float_bits(x), I.bf16_to_float_bits(R)
    for e in range(n):
        terms = [Fraction(a) * Fraction(b) for a, b in zip(Rf[e], xf)]
        exact = sum(terms)
        bound = Fraction(hidden) * Fraction(2) ** -53 * sum(abs(t) for t in terms)
        assert abs(Fraction(l[e]) - exact) <= bound, e


def check_topk_bruteforce(O, seed=8):
    for T, n, k in [(3, 896, 16), (2, 64, 8), (1, 20, 20)]:
        L = gen.normal_f32(gen.key(seed, 93, gen.KIND_LOGITS, T), T * n).reshape(T, n)
        for t in range(T):
            idx, w = O.topk(L[t].astype(np.float64), k)
            order = sorted(range(n), key=lambda e: (-float(L[t, e]), e))[:k]
            assert list(idx) == order
            s = np.array([I.sigmoid(float(L[t, e])) for e in order])
            assert np.max(np.abs(w - s / s.sum())) <= 1e-15
            assert abs(w.sum() - 1.0) <= 1e-15
            # top-k of l and of sigmoid(l) agree (sigmoid is increasing)
            order_s = sorted(range(n), key=lambda e: (-I.sigmoid(float(L[t, e])), e))[:k]
            assert set(order_s) == set(order)


def check_topk_ties_lower_index(O):
    logits = np.array([0.5, 1.0, 0.25, 1.0, 1.0, -2.0])
    idx, w = O.topk(logits, 3)
    assert list(idx) == [1, 3, 4]
    idx, w = O.topk(logits, 6)
    assert list(idx) == [1, 3, 4, 0, 2, 5]


def check_topk_bias_selects_only(O):
    n, k = 12, 3
    logits = np.array([0.1 * i for i in range(n)])  # top-3 unbiased: 11, 10, 9
    bias = np.zeros(n)
    bias[0] = 5.0  # forces expert 0 in
    idx, w = O.topk(logits, k, bias)
    assert list(idx) == [0, 11, 10]
    s = np.array([I.sigmoid(logits[e]) for e in idx])  # weights from unbiased scores
    assert np.max(np.abs(w - s / s.sum())) <= 1e-15


def check_combine(O, seed=12):
    hidden, k = 256, 5
    ye = gen.normal_f32(gen.key(seed, 92, gen.KIND_TOKENS), k * hidden).reshape(k, hidden)
    ye = ye.astype(np.float64)
    w = np.array([0.3, 0.25, 0.2, 0.15, 0.1])
    y = O.combine(w, ye)
    assert np.max(np.abs(y - w @ ye)) <= 1e-15 * np.max(np.abs(y)) * k
    same = np.repeat(ye[:1], k, axis=0)
    assert np.max(np.abs(O.combine(w, same) - ye[0])) <= 4e-16 * np.max(np.abs(ye[0])) * k
    y1 = O.combine(np.array([1.0]), ye[:1])
    assert np.array_equal(y1, ye[0])
    # linearity in w
    w2 = np.array([0.1, 0.1, 0.5, 0.2, 0.1])
    lhs = O.combine(w + w2, ye)
    rhs = O.combine(w, ye) + O.combine(w2, ye)
    assert np.max(np.abs(lhs - rhs)) <= 1e-14 * np.max(np.abs(lhs))


def check_moe_layer_small(O, seed=31):
    n, hidden, inter, k = 10, 128, 64, 3
    R = gen.normal_bf16(gen.key(seed, 91, gen.KIND_ROUTER), n * hidden, 0, 0.02).reshape(n, hidden)
    x = gen.normal_bf16(gen.key(seed, 91, gen.KIND_TOKENS), hidden)
    experts = {e: gen.expert(seed, 91, e, hidden, inter, 114, 120) for e in range(n)}
    y, idx, w = O.moe_layer(x, R, experts, k, hidden, inter)
    xf, Rf = I.bf16_to_float_bits(x), I.bf16_to_float_bits(R)
    l = Rf @ xf
    order = sorted(range(n), key=lambda e: (-l[e], e))[:k]
    assert list(idx) == order
    s = np.array([I.sigmoid(l[e]) for e in order])
    wi = s / s.sum()
    assert np.max(np.abs(w - wi)) <= 1e-14
    yy = np.zeros(hidden)
    for j, e in enumerate(order):
        Ex = experts[e]
        g = I.dequant_numpy(*Ex["gate"]) @ xf
        u = I.dequant_numpy(*Ex["up"]) @ xf
        h = np.array([I.silu_tanh_form(a) for a in g]) * u
        yy += wi[j] * (I.dequant_numpy(*Ex["down"]) @ h)
    assert np.max(np.abs(y - yy)) <= 1e-12 * np.max(np.abs(yy))


def check_quant_ties_and_saturation(O):
    # Block with amax 4 -> E = 0 (2^2 <= 4 < 2^3, minus 2): values are codes.
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (0.3, 1), (0.7, 1), (2.9, 5), (4.9, 6), (5.1, 7), (-0.75, 10), (-5.0, 14),
             (-0.2, 0), (0.0, 0)]
    v = np.zeros(32)
    v[0] = 4.0
    for i, (val, _) in enumerate(cases):
        v[1 + i] = val
    nib, sc = O.mxfp4_quant(v)
    codes = I.unpack_codes(nib)[0]
    assert sc[0, 0] == 127 and codes[0] == 6
    for i, (val, c) in enumerate(cases):
        assert codes[1 + i] == c, (val, codes[1 + i], c)
    # saturation: amax 7.9 -> E = 0, 7.9 -> 6
    v2 = np.zeros(32)
    v2[3] = 7.9
    v2[4] = -7.0
    nib2, sc2 = O.mxfp4_quant(v2)
    c2 = I.unpack_codes(nib2)[0]
    assert sc2[0, 0] == 127 and c2[3] == 7 and c2[4] == 15


def check_quant_invariants(O, seed=14):
    v = gen.normal_f32(gen.key(seed, 90, gen.KIND_TOKENS), 64 * 96).reshape(64, 96).astype(np.float64)
    v *= np.exp(np.linspace(-20, 20, 64))[:, None]
    v[5, 32:64] = 0.0
    nib, sc = O.mxfp4_quant(v)
    codes = I.unpack_codes(nib)
    for r in range(64):
        for g in range(3):
            blk = codes[r, 32 * g:32 * g + 32]
            if not np.any(v[r, 32 * g:32 * g + 32]):
                assert sc[r, g] == 0 and not np.any(blk)
                continue
            mags = [abs(float(I.e2m1_from_bits(int(c)))) for c in blk]
            assert max(mags) in (4.0, 6.0), (r, g, max(mags))
            # every decoded value is the nearest representable one
            s = Fraction(2) ** (int(sc[r, g]) - 127)
            for i in range(32):
                t = Fraction(float(v[r, 32 * g + i])) / s
                got = I.e2m1_from_bits(int(blk[i]))
                best = min(abs(abs(t) - abs(I.e2m1_from_bits(m))) for m in range(8))
                assert abs(abs(t) - abs(got)) == best or abs(t) > 6


def check_quant_roundtrip(O, seed=15):
    codes = (gen.random_bytes(gen.key(seed, 89, gen.KIND_MATRIX), 8 * 64) & 15).reshape(8, 64)
    codes[:, 0] = 7  # magnitude 6 in the first group
    codes[:, 32] = 14  # magnitude 4 in the second group
    codes[codes == 8] = 0  # canonical zero
    nib = I.pack_codes(codes)
    sc = np.array([[110 + r, 140 - r] for r in range(8)], np.uint8)
    v = I.dequant_numpy(nib, sc)
    nib2, sc2 = O.mxfp4_quant(v)
    assert np.array_equal(sc2, sc) and np.array_equal(nib2, nib)


def check_matmul(O, seed=16):
    a = gen.mxfp4_matrix(seed, 88, 7, 96, 118, 130, a=0)
    w = gen.mxfp4_matrix(seed, 88, 9, 96, 118, 130, a=1)
    w[1][2, 1] = 255
    C = O.mxfp4_matmul(a[0], a[1], w[0], w[1])
    Cn = I.dequant_numpy(*a) @ I.dequant_numpy(*w).T
    assert np.max(np.abs(C - Cn)) <= 1e-12 * np.max(np.abs(Cn))


def check_permute(O, seed=17):
    L = W.zipf_router_logits(seed, 64, 896)
    idx = np.array([O.topk(L[t].astype(np.float64), 16)[0] for t in range(64)])
    counts, offsets, pt, ps = O.permute(idx, 896)
    assert counts.sum() == 64 * 16
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)[:-1]]))
    seen = set(zip(pt.tolist(), ps.tolist()))
    assert len(seen) == 64 * 16  # bijection onto the (t, j) pairs
    for e in np.nonzero(counts)[0]:
        toks = pt[offsets[e]:offsets[e] + counts[e]]
        assert np.all(np.diff(toks) > 0)
        for t, j in zip(toks, ps[offsets[e]:offsets[e] + counts[e]]):
            assert idx[t, j] == e


def _bits_to_f32(u):
    return np.array(u, np.uint32).view(np.float32)


def check_bf16_rne(O, seed=41):
    """The fp32 -> bf16 cast of the layer's output is round to nearest, ties
    to even. Pinned by exact rational comparison of the two bf16 neighbours
    (tests/_independent.py) on hand-picked ties and their neighbours, signed
    zeros, infinities, NaN and the overflow edge, and by torch's CPU bf16
    conversion on random bit patterns."""
    fixed = [0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0x3F818001, 0x3F817FFF,
             0xBF808000, 0xBF818000, 0x00000000, 0x80000000, 0x7F800000, 0xFF800000,
             0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000, 0x7F7E8000, 0x00008000,
             0x00018000, 0x00017FFF, 0x0000FFFF, 0x007F8000, 0x3F800000, 0x4B7FFF80]
    rnd = gen.random_bytes(gen.key(seed, 87, gen.KIND_MATRIX), 4 * 6000).view(np.uint32)
    ties = (rnd[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    near = np.concatenate([ties + np.uint32(1), ties - np.uint32(1)])
    pats = np.concatenate([np.array(fixed, np.uint32), ties, near, rnd[2000:]])
    f = _bits_to_f32(pats)
    finite = ~np.isnan(f)
    got = O.f32_to_bf16(f).astype(np.uint32)
    for u, g in zip(pats[:len(fixed) + 400], got[:len(fixed) + 400]):
        if np.isnan(_bits_to_f32(u)):
            continue
        assert g == I.bf16_nearest_even_bits(int(u)), (hex(int(u)), hex(int(g)))
    import torch
    want = torch.from_numpy(f[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got[finite].astype(np.uint16), want.view(np.uint16))
    # NaN stays NaN of the same sign
    nan_in = _bits_to_f32(np.array([0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FFFFFFF], np.uint32))
    nb = O.f32_to_bf16(nan_in).astype(np.uint32)
    for u, g in zip([0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FFFFFFF], nb):
        assert (g & 0x7F80) == 0x7F80 and (g & 0x7F) != 0, hex(int(g))
        assert (g >> 15) == (u >> 31)


def check_moe_from_logits(O, seed=34):
    """The batched oracle: T tokens routed from given logits rows (with a
    routing bias) equal T separate one-token calls bit for bit, and each
    token equals an independent numpy route (key sigma(l) + b sorted by
    Python, unbiased renormalised weights, experts expanded and multiplied
    by numpy)."""
    n, hidden, inter, k, T = 12, 128, 64, 3, 4
    X = gen.normal_bf16(gen.key(seed, 86, gen.KIND_TOKENS), T * hidden).reshape(T, hidden)
    L = gen.normal_f32(gen.key(seed, 86, gen.KIND_LOGITS), T * n).reshape(T, n).astype(np.float64)
    L[2] = -L[1]               # makes tokens 1 and 2 pick different sets
    bias = np.linspace(-0.2, 0.3, n)
    experts = {e: gen.expert(seed, 86, e, hidden, inter, 114, 120) for e in range(n)}
    Y, idx, w = O.moe_from_logits(X, L, experts, k, hidden, inter, bias=bias)
    assert len({tuple(sorted(r)) for r in idx.tolist()}) >= 3, idx
    for t in range(T):
        y1, i1, w1 = O.moe_from_logits(X[t:t + 1], L[t:t + 1], experts, k, hidden, inter,
                                       bias=bias)
        assert np.array_equal(Y[t], y1[0]) and np.array_equal(idx[t], i1[0])
        assert np.array_equal(w[t], w1[0])
        key = [I.sigmoid(L[t, e]) + bias[e] for e in range(n)]
        order = sorted(range(n), key=lambda e: (-key[e], e))[:k]
        assert list(idx[t]) == order, (t, idx[t], order)
        s = np.array([I.sigmoid(L[t, e]) for e in order])
        wi = s / s.sum()
        assert np.max(np.abs(w[t] - wi)) <= 1e-15
        xf = I.bf16_to_float_bits(X[t])
        yy = np.zeros(hidden)
        for j, e in enumerate(order):
            Ex = experts[e]
            g = I.dequant_numpy(*Ex["gate"]) @ xf
            u = I.dequant_numpy(*Ex["up"]) @ xf
            h = np.array([I.silu_tanh_form(a) for a in g]) * u
            yy += wi[j] * (I.dequant_numpy(*Ex["down"]) @ h)
        assert np.max(np.abs(Y[t] - yy)) <= 1e-12 * np.max(np.abs(yy)), t


ALL = [check_e2m1_table, check_e8m0, check_golden_nibble_order, check_bruteforce_4x32,
       check_all_scale_bytes, check_exact_rational, check_exact_dyadic, check_scale_shift,
       check_nan_containment, check_dequant_crosscheck, check_expert_crosscheck, check_silu,
       check_router_logits, check_topk_bruteforce, check_topk_ties_lower_index,
       check_topk_bias_selects_only, check_combine, check_moe_layer_small,
       check_quant_ties_and_saturation, check_quant_invariants, check_quant_roundtrip,
       check_matmul, check_permute, check_shared_expert_crosscheck, check_shared_expert_by_hand,
       check_layer_shared_adds, check_bf16_rne, check_moe_from_logits]
