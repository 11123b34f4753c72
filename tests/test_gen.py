"""The seeded input generator: SplitMix64 against its published first outputs
from state 0 (Steele, Lea, Flood 2014 reference implementation), the
counter-based access against the sequential one, determinism, independent
regeneration of one expert, and the value ranges of each workload."""
import ctypes

import numpy as np

import gen
from gen import workloads as W


def test_splitmix64_published_vector():
    st = ctypes.c_uint64(0)
    seq = [gen.lib().k3g_splitmix64_next(ctypes.byref(st)) for _ in range(3)]
    assert seq == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_matches_sequential():
    k = gen.key(5, 3, gen.KIND_EXPERT, 17, 2)
    st = ctypes.c_uint64(k)
    seq = [gen.lib().k3g_splitmix64_next(ctypes.byref(st)) for _ in range(100)]
    assert list(gen.draws(k, 100)) == seq


def test_expert_regenerates_alone_and_differs():
    a = gen.expert(0, W.C3, 123, 256, 64)
    b = gen.expert(0, W.C3, 123, 256, 64)
    c = gen.expert(0, W.C3, 124, 256, 64)
    for m in ("gate", "up", "down"):
        for i in range(2):
            assert np.array_equal(a[m][i], b[m][i])
        assert not np.array_equal(a[m][0], c[m][0])


def test_threads_do_not_change_bytes():
    k = gen.key(1, 1, 1)
    gen.set_threads(1)
    a = gen.random_bytes(k, 3 << 20)
    s1 = gen.uniform_u8(k, 3 << 18, 120, 134)
    gen.set_threads(8)
    b = gen.random_bytes(k, 3 << 20)
    s2 = gen.uniform_u8(k, 3 << 18, 120, 134)
    gen.set_threads(1)
    assert np.array_equal(a, b) and np.array_equal(s1, s2)


def test_workload_value_ranges():
    nib, sc, x = W.c1_inputs()
    assert nib.shape == (256, 512) and sc.shape == (256, 32)
    assert sc.min() == 120 and sc.max() == 134
    counts = np.bincount(np.concatenate([nib.ravel() & 15, nib.ravel() >> 4]), minlength=16)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()
    assert abs(float(x.mean())) < 0.1 and 0.9 < float(x.std()) < 1.1
    R = W.router_bf16(0, n_experts=32, hidden=7168)
    Rf = (R.astype(np.uint32) << 16).view(np.float32)
    assert 0.019 < float(Rf.std()) < 0.021
    L = W.uniform_router_logits(0, 4)
    assert L.min() >= 0.0 and L.max() < 1.0


def test_zipf_logits_skew():
    """Top-16 of the Zipf logits is a draw without replacement weighted by
    rank^-1.1: the hottest expert appears in nearly every token."""
    import oracle
    L = W.zipf_router_logits(0, 64)
    idx = np.array([oracle.topk(L[t].astype(np.float64), 16)[0] for t in range(64)])
    counts = np.bincount(idx.ravel(), minlength=896)
    assert counts.max() >= 56
    assert 250 <= np.count_nonzero(counts) <= 420
