"""Host-only checks of the expert cache's policy through k3_cache_replay (no
GPU: the replay runs the same planner as k3_cache_fetch, with every copy
taken as finished).

Pins:
- a cyclic scan over N + 1 keys through N least-recently-used slots never
  hits, and a pinned prefix of P keys plus one rotating slot over a cycle
  of M keys hits exactly P of every M requests after the first cycle (the
  90-of-93 = 96.8% case); [A176] "The interesting design decisions", the
  trunk's pinned prefix against LRU;
- one request of k distinct misses into k empty slots takes k copies and
  evicts nothing (the same batch must never be handed one slot twice);
  [SAT] "The bug the code confesses to";
- an independent model of LRU with pinning, written here from the pages'
  description ([SAT] "The cache the project exists for": least recently
  used unpinned slot; [ZOR] "Reduction four": slots empty, in flight or
  holding an expert), agrees count for count on random skewed traces;
- the optimal offline replay (Belady's farthest-next-use rule, which the
  pages' cache study sets against LRU, [A176] "The interesting design
  decisions") reaches the fewest misses found by brute force over every
  eviction choice on tiny traces, agrees with an independent model on skewed
  traces, never misses more than LRU, and misses 3 per cycle on the 93-key
  scan through 90 slots where LRU misses every time.
"""
import numpy as np
import pytest

import mxfp4_packed_weight_amd as K


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(K.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    K.lib()


def lru_model(trace, n_slots, pinned=(), request_size=1):
    """LRU with pinning over requests of `request_size` ids. A slot named by
    the current request is not evicted for another id of the same request;
    a repeat of an id that this request itself brought in is an in-flight
    reuse (its copy was issued moments ago); a repeat of an older resident
    id is a hit."""
    pinned = set(int(p) for p in pinned)
    where = {}            # expert -> slot
    holder = [None] * n_slots
    last = [0] * n_slots
    clock = 0
    st = dict(requests=0, hits=0, misses=0, inflight_reuses=0, evictions=0)
    trace = [int(t) for t in trace]
    for r0 in range(0, len(trace), request_size):
        req = trace[r0:r0 + request_size]
        protected = {where[e] for e in req if e in where}
        brought = set()
        for e in req:
            st["requests"] += 1
            clock += 1
            if e in where:
                s = where[e]
                st["inflight_reuses" if s in brought else "hits"] += 1
                last[s] = clock
                continue
            empty = [s for s in range(n_slots) if holder[s] is None]
            if empty:
                s = empty[0]
            else:
                cands = [s for s in range(n_slots)
                         if s not in protected and holder[s] not in pinned]
                s = min(cands, key=lambda j: last[j])
                del where[holder[s]]
                st["evictions"] += 1
            holder[s] = e
            where[e] = s
            last[s] = clock
            protected.add(s)
            brought.add(s)
            st["misses"] += 1
    return st


def replay(trace, n_experts, n_slots, pinned=(), request_size=1):
    st = K.k3_cache_replay(trace, n_experts, n_slots, pinned, request_size)
    assert st["bytes_copied"] == 0  # the replay copies nothing
    assert st["requests"] == len(trace)
    assert st["hits"] + st["misses"] + st["inflight_reuses"] == st["requests"]
    return st


def test_cyclic_scan_defeats_lru():
    # 90 slots over a 93-key cycle: every request misses, forever
    trace = np.tile(np.arange(93), 50)
    st = replay(trace, 93, 90)
    assert st["hits"] == 0 and st["misses"] == len(trace)
    assert st["evictions"] == len(trace) - 90


def test_pinned_prefix_plus_one_ring_slot():
    # 90 pinned of 93 plus one rotating slot: hit rate 90/93 after warm-up
    cycles = 40
    trace = np.tile(np.arange(93), cycles)
    st = replay(trace, 93, 91, pinned=np.arange(90))
    assert st["hits"] == 90 * (cycles - 1)
    assert st["misses"] == 93 + 3 * (cycles - 1)
    steady = 90 / 93
    assert abs(steady - 0.968) < 5e-4  # the pages' 96.8%


def test_one_request_of_distinct_misses_takes_distinct_slots():
    ids = np.array([5, 17, 2, 40, 33, 8, 21, 11], np.int32)
    st = replay(ids, 48, 8, request_size=8)
    assert st == dict(requests=8, hits=0, misses=8, inflight_reuses=0, evictions=0,
                      bytes_copied=0)
    # a second request for the same ids hits every one
    st = replay(np.concatenate([ids, ids[::-1]]), 48, 8, request_size=8)
    assert st["hits"] == 8 and st["misses"] == 8 and st["evictions"] == 0


def test_repeat_inside_one_request_is_an_inflight_reuse():
    st = replay(np.array([3, 3, 4, 3], np.int32), 10, 2, request_size=4)
    assert st["misses"] == 2 and st["inflight_reuses"] == 2 and st["hits"] == 0


def test_whole_pool_resident_only_cold_misses():
    rng = np.random.default_rng(3)
    trace = rng.integers(0, 64, 16 * 200).astype(np.int32)
    st = replay(trace, 64, 64, request_size=16)
    assert st["misses"] == len(np.unique(trace)) and st["evictions"] == 0


def skewed_trace(rng, n, k, tokens, alpha):
    """Requests of k distinct experts drawn with Zipf-like popularity."""
    p = 1.0 / np.arange(1, n + 1) ** alpha
    p /= p.sum()
    perm = rng.permutation(n)
    return np.concatenate([perm[rng.choice(n, k, replace=False, p=p)]
                           for _ in range(tokens)]).astype(np.int32)


@pytest.mark.parametrize("n,k,slots,alpha,npin", [
    (896, 16, 64, 0.0, 0), (896, 16, 128, 0.8, 0), (896, 16, 300, 1.1, 8),
    (96, 8, 8, 0.5, 0), (96, 8, 20, 0.9, 12), (40, 1, 3, 0.7, 2)])
def test_policy_matches_independent_lru_model(n, k, slots, alpha, npin):
    rng = np.random.default_rng(n * 1000 + slots)
    trace = skewed_trace(rng, n, k, 150, alpha)
    pinned = rng.choice(n, npin, replace=False)
    got = replay(trace, n, slots, pinned, request_size=k)
    want = lru_model(trace, slots, pinned, request_size=k)
    got.pop("bytes_copied")
    assert got == want


def test_requests_with_repeats_match_the_model():
    rng = np.random.default_rng(9)
    trace = rng.integers(0, 30, 6 * 120).astype(np.int32)  # repeats inside requests
    got = replay(trace, 30, 9, pinned=[1, 2], request_size=6)
    got.pop("bytes_copied")
    assert got == lru_model(trace, 9, [1, 2], request_size=6)


def test_replay_refusals():
    with pytest.raises(K.K3Error) as e:  # 4 distinct misses, 3 slots
        K.k3_cache_replay([1, 2, 3, 4], 10, 3, (), 4)
    assert e.value.status == K.K3_ERR_MEMORY
    with pytest.raises(K.K3Error) as e:  # pinned residents leave 1 slot for 2 misses
        K.k3_cache_replay([0, 1, 2, 3], 10, 3, (0, 1), 2)
    assert e.value.status == K.K3_ERR_MEMORY
    with pytest.raises(K.K3Error) as e:
        K.k3_cache_replay([0, 10], 10, 3, (), 1)
    assert e.value.status == K.K3_ERR_ARG
    with pytest.raises(K.K3Error) as e:
        K.k3_cache_replay([0], 10, 11, (), 1)
    assert e.value.status == K.K3_ERR_CONFIG
    with pytest.raises(K.K3Error) as e:
        K.k3_cache_replay([0], 10, 3, (12,), 1)
    assert e.value.status == K.K3_ERR_ARG


def opt_model(trace, n_slots, pinned=(), request_size=1):
    """Belady's rule written from its definition: on a miss with no empty
    slot, evict the resident expert (not pinned, not named by the current
    request, so not referenced again before the request ends) whose next
    reference is farthest ahead (never again = farthest); ties to the lowest
    slot."""
    pinned = set(int(p) for p in pinned)
    trace = [int(t) for t in trace]
    holder = [None] * n_slots
    st = dict(requests=0, hits=0, misses=0, inflight_reuses=0, evictions=0)
    for r0 in range(0, len(trace), request_size):
        req = trace[r0:r0 + request_size]
        r1 = r0 + len(req)
        protected = {holder.index(e) for e in req if e in holder}
        brought = set()
        for pos, e in enumerate(req, start=r0):
            st["requests"] += 1
            if e in holder:
                s = holder.index(e)
                st["inflight_reuses" if s in brought else "hits"] += 1
                continue
            if None in holder:
                s = holder.index(None)
            else:
                def next_ref(x):
                    # x's own reference inside this request (if any) was
                    # already passed; look from the position after it
                    start = pos + 1
                    for q in range(start, len(trace)):
                        if trace[q] == x:
                            return q
                    return len(trace) + 1
                cands = [j for j in range(n_slots)
                         if j not in protected and holder[j] not in pinned]
                s = max(cands, key=lambda j: (next_ref(holder[j]), -j))
                st["evictions"] += 1
            holder[s] = e
            protected.add(s)
            brought.add(s)
            st["misses"] += 1
    return st


def min_misses_bruteforce(trace, n_slots):
    """Fewest misses over every possible eviction choice (one id per
    request): the optimum Belady's rule must reach."""
    from functools import lru_cache

    @lru_cache(maxsize=None)
    def go(i, cache):
        if i == len(trace):
            return 0
        e = trace[i]
        if e in cache:
            return go(i + 1, cache)
        if len(cache) < n_slots:
            return 1 + go(i + 1, tuple(sorted(cache + (e,))))
        return 1 + min(go(i + 1, tuple(sorted(tuple(c for c in cache if c != v) + (e,))))
                       for v in cache)
    return go(0, ())


def test_opt_reaches_the_bruteforce_optimum():
    rng = np.random.default_rng(41)
    for _ in range(60):
        n = int(rng.integers(3, 6))
        slots = int(rng.integers(1, n))
        trace = rng.integers(0, n, int(rng.integers(4, 11))).astype(np.int32)
        st = K.k3_cache_replay_opt(trace, n, slots)
        assert st["misses"] == min_misses_bruteforce(tuple(trace.tolist()), slots), trace


@pytest.mark.parametrize("n,k,slots,alpha,npin", [
    (896, 16, 64, 0.0, 0), (896, 16, 200, 1.0, 4), (96, 8, 12, 0.6, 2), (40, 1, 5, 0.8, 1)])
def test_opt_matches_independent_model_and_beats_lru(n, k, slots, alpha, npin):
    rng = np.random.default_rng(7 * n + slots)
    trace = skewed_trace(rng, n, k, 80, alpha)
    pinned = rng.choice(n, npin, replace=False)
    got = K.k3_cache_replay_opt(trace, n, slots, pinned, k)
    assert got.pop("bytes_copied") == 0
    assert got == opt_model(trace, slots, pinned, k)
    lru = K.k3_cache_replay(trace, n, slots, pinned, k)
    assert got["misses"] <= lru["misses"]


def test_opt_on_a_cyclic_scan():
    # 93 keys through 90 slots: LRU never hits, the optimum misses 3 per cycle
    trace = np.tile(np.arange(93), 40).astype(np.int32)
    lru = K.k3_cache_replay(trace, 93, 90)
    opt = K.k3_cache_replay_opt(trace, 93, 90)
    assert lru["hits"] == 0
    assert opt["misses"] == 93 + 3 * 39
    # everything fits: only cold misses
    assert K.k3_cache_replay_opt(trace, 93, 93)["misses"] == 93
