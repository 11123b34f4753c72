"""GPU checks of the expert cache through the C ABI.

- The decode layer through a cache of fewer slots than experts gives the
  same bits (y, fp32 y, top-k indices, weights, logits) as the layer on the
  fully resident pool, token after token, while experts are evicted and
  copied back in from pinned host blobs.
- The live cache's counters equal those of the host-only replay of the
  trace it recorded (every copy there had finished: the layer waits for the
  selection before fetching), its histogram is the trace's, and every copy
  moved one expert blob.
- After each fetch the device table sends every requested expert to its own
  slot (one request is never handed one slot twice: [SAT] "The bug the code
  confesses to") and every other expert to a slot or to the all-zero blob.
- A repeated request issues no second copy: while the first copies are
  still queued it waits for them (in-flight reuse, the third slot state of
  [SAT] "The bug the code confesses to"), afterwards it hits. Pinned
  experts keep their slot through evictions ([SAT] "The cache the project
  exists for").
- Refusals: ids outside the pool, an expert with no source, a request larger
  than the evictable slots, a capture of the cached layer.
- Batched decode through a cache gives the resident batched layer's bits,
  batch after batch with evictions between them, and a batch that names
  more experts than the cache holds is refused with the cache unchanged.
"""
import ctypes

import numpy as np
import pytest

import gen
import mxfp4_packed_weight_amd as K
from gen import device as D
from gen import workloads as W
import oracle
from tests._gpu import TOL, empty, make_cache, normwise, pinned_copy, say, up

pytestmark = pytest.mark.gpu

CFG, SEED, N, HIDDEN, INTER, KTOP = 76, 11, 48, 384, 224, 8


def hip_runtime():
    """The HIP runtime this process already runs (torch's and the library's:
    one runtime per process), opened by the path it was mapped from."""
    paths = {line.split()[-1] for line in open("/proc/self/maps")
             if "libamdhip64" in line and line.split()[-1].startswith("/")}
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths.pop())


def read_table(cache, n):
    """The cache's device pointer table, copied to the host."""
    import torch
    torch.cuda.synchronize()
    hip = hip_runtime()
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    out = np.zeros(n, np.uint64)
    rc = hip.hipMemcpy(out.ctypes.data, K.k3_cache_table(cache), 8 * n, 2)  # device to host
    assert rc == 0
    return out


def layer(fn, table_or_cache, xd, R_d, n, hidden, inter, k, ws):
    import torch
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    idx = empty(k, torch.int32)
    w = empty(k, torch.float32)
    lg = empty(n, torch.float64)
    fn(xd, R_d, table_or_cache, n, hidden, inter, k, y, ws, y_f32=y32, idx=idx, w=w, logits=lg)
    return dict(y=y.cpu().numpy().view(np.uint16), y32=y32.cpu().numpy().view(np.uint32),
                idx=idx.cpu().numpy(), w=w.cpu().numpy().view(np.uint32),
                logits=lg.cpu().numpy().view(np.uint64))


def check_table(tab, idx, slot_lo, n_slots, expert_bytes):
    sel = tab[idx]
    assert len(set(sel.tolist())) == len(idx), "two requested experts share a slot"
    off = sel.astype(np.int64) - int(slot_lo)
    assert np.all((off >= 0) & (off < n_slots * expert_bytes) & (off % expert_bytes == 0))
    inside = (tab >= slot_lo) & (tab < slot_lo + n_slots * expert_bytes)
    outside = np.unique(tab[~inside])
    assert outside.size <= 1, "non-resident entries must all name the zero blob"
    resident = tab[inside]
    assert len(np.unique(resident)) == resident.size, "two experts share a slot"
    return outside


@pytest.fixture(scope="module")
def small_pool():
    pool = D.build_expert_pool(SEED, CFG, N, HIDDEN, INTER, 114, 120, workers=2)
    R = gen.normal_bf16(gen.key(SEED, CFG, gen.KIND_ROUTER), N * HIDDEN, 0, 0.02).reshape(
        N, HIDDEN)
    return pool, up(R), pinned_copy(pool)


def test_cached_layer_matches_resident_layer(small_pool):
    import torch
    pool, R_d, host = small_pool
    slots, tokens = 12, 24
    say(f"cached layer: {N} experts through {slots} slots, {tokens} tokens")
    ws = empty(K.k3_moe_workspace_bytes(1, N, HIDDEN, INTER, KTOP), torch.uint8)
    ws2 = empty(K.k3_moe_workspace_bytes(1, N, HIDDEN, INTER, KTOP), torch.uint8)
    X = W.tokens_bf16(SEED, CFG, tokens, HIDDEN)
    c = make_cache(pool, host, slots)
    try:
        slot_lo = None
        trace = []
        for t in range(tokens):
            xd = up(X[t])
            want = layer(K.k3_moe_layer_ex, pool.table, xd, R_d, N, HIDDEN, INTER, KTOP, ws)
            got = layer(K.k3_moe_layer_cached, c, xd, R_d, N, HIDDEN, INTER, KTOP, ws2)
            for key in want:
                assert np.array_equal(got[key], want[key]), (t, key)
            trace.extend(got["idx"].tolist())
            if t in (0, tokens - 1):  # the cached layer against the oracle itself
                R_h = R_d.cpu().numpy().view(np.uint16)
                ex = {e: W.expert_weights(SEED, CFG, e, HIDDEN, INTER, 114, 120)
                      for e in got["idx"].tolist()}
                y_ref, idx_ref, w_ref = oracle.moe_layer(X[t], R_h, ex, KTOP, HIDDEN, INTER)
                assert np.array_equal(got["idx"], idx_ref)
                assert np.max(np.abs(got["w"].view(np.float32) - w_ref)) <= 1e-6
                assert normwise(got["y32"].view(np.float32), y_ref) <= TOL, t
            tab = read_table(c, N)
            if slot_lo is None:
                slot_lo = int(tab[got["idx"]].min())  # first token fills slots 0..k-1
            check_table(tab, got["idx"], slot_lo, slots, pool.expert_bytes)
        st = K.k3_cache_get_stats(c)
        ref = K.k3_cache_replay(np.array(trace, np.int32), N, slots, (), KTOP)
        assert st["bytes_copied"] == st["misses"] * pool.expert_bytes
        ref["bytes_copied"] = st["bytes_copied"]
        assert st == ref
        assert st["evictions"] > 0, "the run must evict to exercise the cache"
        assert np.array_equal(K.k3_cache_trace(c), np.array(trace, np.int32))
        assert np.array_equal(K.k3_cache_histogram(c, N),
                              np.bincount(trace, minlength=N).astype(np.uint64))
        say(f"cached layer: {st}")
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)


def test_repeat_request_and_pins(small_pool):
    import torch
    pool, _, host = small_pool
    c = make_cache(pool, host, 10)
    try:
        K.k3_cache_pin(c, 0)
        K.k3_cache_pin(c, 1)
        first = list(range(8))
        K.k3_cache_fetch(c, first)
        K.k3_cache_fetch(c, first)  # no synchronisation: copies may be in flight
        st = K.k3_cache_get_stats(c)
        assert st["misses"] == 8 and st["hits"] + st["inflight_reuses"] == 8
        assert st["bytes_copied"] == 8 * pool.expert_bytes
        tab0 = read_table(c, N)
        K.k3_cache_fetch(c, list(range(8, 16)))  # evicts 2..7, never 0 and 1
        tab1 = read_table(c, N)
        assert tab1[0] == tab0[0] and tab1[1] == tab0[1]
        zero = np.unique(tab0[16:])
        assert zero.size == 1
        assert np.all(tab1[2:8] == zero[0])
        st = K.k3_cache_get_stats(c)
        assert st["evictions"] == 6 and st["misses"] == 16
        # unpinned, expert 0 is the least recently used and goes first
        K.k3_cache_pin(c, 0, False)
        K.k3_cache_fetch(c, [20])
        tab2 = read_table(c, N)
        assert tab2[0] == zero[0] and tab2[20] == tab0[0] and tab2[1] == tab0[1]
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)


def test_inflight_copy_is_waited_for_not_repeated(small_pool):
    """The stream is held by a bounded spin kernel, so the first fetch's
    copies are still queued when the same experts are requested again: all
    eight are in-flight reuses (no hit, no second copy). Once the stream
    drains they are hits, and gate/up through the cache's table gives the
    same bits as through the resident pool's."""
    import torch
    pool, _, host = small_pool
    ids = [3, 9, 14, 22, 27, 31, 40, 45]
    c = make_cache(pool, host, 10)
    try:
        torch.cuda.synchronize()
        torch.cuda._sleep(50_000_000)  # tens of milliseconds of spinning, then it ends
        K.k3_cache_fetch(c, ids)
        K.k3_cache_fetch(c, ids)
        st = K.k3_cache_get_stats(c)
        assert st["misses"] == 8 and st["inflight_reuses"] == 8 and st["hits"] == 0, st
        assert st["bytes_copied"] == 8 * pool.expert_bytes
        torch.cuda.synchronize()
        K.k3_cache_fetch(c, ids)
        st = K.k3_cache_get_stats(c)
        assert st["hits"] == 8 and st["misses"] == 8, st
        xd = up(W.tokens_bf16(SEED, CFG, 1, HIDDEN)[0])
        idx = up(np.array(ids, np.int32))
        h_pool = empty((8, INTER), torch.float32)
        h_cache = empty((8, INTER), torch.float32)
        K.k3_expert_gate_up(xd, pool.table, idx, 8, HIDDEN, INTER, h_pool)
        K.k3_expert_gate_up(xd, K.k3_cache_table(c), idx, 8, HIDDEN, INTER, h_cache)
        assert np.array_equal(h_pool.cpu().numpy().view(np.uint32),
                              h_cache.cpu().numpy().view(np.uint32))
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)


def test_cache_refusals(small_pool):
    import torch
    pool, R_d, host = small_pool
    c = K.k3_cache_create(N, pool.expert_bytes, 4)
    try:
        K.k3_cache_set_source(c, 3, host[3 * pool.expert_bytes:4 * pool.expert_bytes])
        for ids, status in [([N], K.K3_ERR_ARG), ([-1], K.K3_ERR_ARG),
                            ([5], K.K3_ERR_CONFIG)]:
            with pytest.raises(K.K3Error) as e:
                K.k3_cache_fetch(c, ids)
            assert e.value.status == status
        for e_ in range(N):
            K.k3_cache_set_source(c, e_, host[e_ * pool.expert_bytes:(e_ + 1) * pool.expert_bytes])
        with pytest.raises(K.K3Error) as e:
            K.k3_cache_fetch(c, [0, 1, 2, 3, 4])
        assert e.value.status == K.K3_ERR_MEMORY
        assert K.k3_cache_get_stats(c)["requests"] == 0  # a refused request changes nothing
        with pytest.raises(K.K3Error) as e:
            K.k3_cache_create(N, pool.expert_bytes, N + 1)
        assert e.value.status == K.K3_ERR_CONFIG
        # captured, the cached layer is refused before it queues anything
        ws = empty(K.k3_moe_workspace_bytes(1, N, HIDDEN, INTER, KTOP), torch.uint8)
        xd = up(W.tokens_bf16(SEED, CFG, 1, HIDDEN)[0])
        y = empty(HIDDEN, torch.int16)
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        refused = None
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            try:
                K.k3_moe_layer_cached(xd, R_d, c, N, HIDDEN, INTER, KTOP, y, ws, stream=s)
            except K.K3Error as err:
                refused = err
            y.zero_()
        assert refused is not None and refused.status == K.K3_ERR_CONFIG
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)


def batched_outputs(fn, arg, X, L, T, ws):
    import torch
    Y = empty((T, HIDDEN), torch.int16)
    Y32 = empty((T, HIDDEN), torch.float32)
    idx = empty((T, KTOP), torch.int32)
    w = empty((T, KTOP), torch.float32)
    fn(X, L, None, arg, N, HIDDEN, INTER, KTOP, T, Y, ws, Y_f32=Y32, idx=idx, w=w)
    return dict(Y=Y.cpu().numpy().view(np.uint16), Y32=Y32.cpu().numpy().view(np.uint32),
                idx=idx.cpu().numpy(), w=w.cpu().numpy().view(np.uint32))


def test_batched_cached_layer_matches_resident(small_pool):
    """Batches of 4 tokens (top-8 of 48) through 36 slots: each batch fits,
    their union does not, so experts are evicted between batches. Every batch
    gives the resident batched layer's bits, and the last one is within 1e-5
    of the oracle; the counters equal the replay with one request per
    batch."""
    import torch
    pool, _, host = small_pool
    T, slots, nb = 4, 36, 6
    say(f"batched cached layer: {nb} batches of {T} tokens through {slots} slots")
    ws = empty(K.k3_moe_batched_workspace_bytes(T, N, HIDDEN, INTER, KTOP), torch.uint8)
    ws2 = empty(K.k3_moe_batched_workspace_bytes(T, N, HIDDEN, INTER, KTOP), torch.uint8)
    c = make_cache(pool, host, slots)
    try:
        trace = []
        for b in range(nb):
            X = up(W.tokens_bf16(SEED, CFG, T, HIDDEN, batch=b))
            L = up(gen.uniform_f32(gen.key(SEED, CFG, gen.KIND_LOGITS, b, 0), T * N).astype(
                np.float64).reshape(T, N))
            want = batched_outputs(K.k3_moe_layer_from_logits, pool.table, X, L, T, ws)
            got = batched_outputs(K.k3_moe_layer_from_logits_cached, c, X, L, T, ws2)
            for key in want:
                assert np.array_equal(got[key], want[key]), (b, key)
            trace.extend(got["idx"].ravel().tolist())
            if b == nb - 1:  # the last batch (after evictions) against the oracle itself
                Xh, Lh = X.cpu().numpy().view(np.uint16), L.cpu().numpy()
                ex = {e: W.expert_weights(SEED, CFG, e, HIDDEN, INTER, 114, 120)
                      for e in np.unique(got["idx"]).tolist()}
                oracle.set_threads(16)
                Y_ref, idx_ref, w_ref = oracle.moe_from_logits(Xh, Lh, ex, KTOP, HIDDEN, INTER)
                assert np.array_equal(got["idx"], idx_ref)
                assert np.max(np.abs(got["w"].view(np.float32) - w_ref)) <= 1e-6
                for t in range(T):
                    err = normwise(got["Y32"][t].view(np.float32), Y_ref[t])
                    assert err <= TOL, (t, err)
                say(f"batched cached layer, batch {b}: within {TOL} of the oracle")
        st = K.k3_cache_get_stats(c)
        ref = K.k3_cache_replay(np.array(trace, np.int32), N, slots, (), T * KTOP)
        ref["bytes_copied"] = st["misses"] * pool.expert_bytes
        assert st == ref
        assert st["evictions"] > 0
        say(f"batched cached layer: {st}")
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)


def test_batched_cached_layer_refuses_a_batch_larger_than_the_cache(small_pool):
    """Five tokens whose top-8 sets are disjoint name 40 experts: more than
    36 slots hold, so the call is refused and the cache is unchanged."""
    import torch
    pool, _, host = small_pool
    T = 5
    L = np.zeros((T, N))
    for t in range(T):
        L[t, 8 * t:8 * t + 8] = 10.0 - np.arange(8) * 0.1
    ws = empty(K.k3_moe_batched_workspace_bytes(T, N, HIDDEN, INTER, KTOP), torch.uint8)
    c = make_cache(pool, host, 36)
    try:
        X = up(W.tokens_bf16(SEED, CFG, T, HIDDEN))
        with pytest.raises(K.K3Error) as e:
            batched_outputs(K.k3_moe_layer_from_logits_cached, c, X, up(L), T, ws)
        assert e.value.status == K.K3_ERR_MEMORY
        assert K.k3_cache_get_stats(c)["requests"] == 0
    finally:
        torch.cuda.synchronize()
        K.k3_cache_destroy(c)
