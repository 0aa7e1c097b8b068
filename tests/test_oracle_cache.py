"""Pins of the cache policy oracle (oracle/cache.py), and the library's host
planner (k3g_cache_plan: host code, no GPU) against it.

"kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM", section "The
cache the project exists for": LRU with pinning, a linear-scan victim, a third
slot state (in flight) so that one batch never hands a slot to two reads, a
request histogram."""
import numpy as np
import pytest

from oracle.cache import CacheRefused, LruSlots


@pytest.fixture(scope="module")
def k3g():
    """The library (its host planner runs without a GPU)."""
    import mxfp4_moe_expert_amd as k3g
    k3g.lib()
    return k3g


def test_hand_sequence_lru_order():
    c = LruSlots(3, 10)
    assert c.request([[0, 1]]) == ([[0, 1]], [(0, 0), (1, 1)])   # empty slots, in order
    assert c.request([[2]]) == ([[2]], [(2, 2)])
    assert c.request([[0, 3]]) == ([[0, 1]], [(3, 1)])           # 0 hits; 1 (oldest) goes
    # 1 and 4 both miss: 2 (age 2) goes first, then the tie of ages 3 to the lower slot
    assert c.request([[4, 1]]) == ([[0, 2]], [(1, 2), (4, 0)])
    assert (c.hits, c.misses, c.evictions) == (1, 6, 3)


def test_pinned_expert_is_never_evicted_and_a_full_step_is_refused():
    c = LruSlots(2, 10)
    c.pinned.add(0)
    c.request([[0]])
    c.request([[1]])
    assert c.request([[2]]) == ([[1]], [(2, 1)])   # the pinned 0 stays; 1 goes
    c.finish_batch()
    before = (list(c.state), dict(c.where), list(c.hist), c.step)
    with pytest.raises(CacheRefused):
        c.request([[2, 3]])                         # 2 uses the only unpinned slot
    assert (list(c.state), dict(c.where), list(c.hist), c.step) == before


def test_one_batch_never_gets_one_slot_twice():
    # the pages' bug: a batch's misses were each handed the first empty slot
    c = LruSlots(4, 10)
    slots, copies = c.request([[3, 1], [2, 4]])
    assert sorted(s for _, s in copies) == [0, 1, 2, 3]
    assert all(st == "inflight" for st in c.state)  # until the batch finishes
    c.finish_batch()
    assert c.state == [1, 2, 3, 4]
    assert slots == [[2, 0], [1, 3]]


def test_histogram_and_dropped_entries():
    c = LruSlots(4, 8)
    slots, copies = c.request([[5, -1, 2], [5, 7, -1]])
    assert c.hist == [0, 0, 1, 0, 0, 2, 0, 1]
    assert slots == [[1, -1, 0], [1, 2, -1]]
    assert copies == [(2, 0), (5, 1), (7, 2)]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_library_planner_matches_the_oracle(k3g, seed):
    rng = np.random.default_rng(seed)
    n_total, n_slots, T, K = 40, 12, 2, 3
    arena = k3g.ExpertBank()
    arena.base = None
    arena.stride = 4096
    arena.n_experts = n_slots
    cache = k3g.ExpertCache(None, n_total, arena)
    ref = LruSlots(n_slots, n_total)
    for e in rng.choice(n_total, 3, replace=False):
        cache.pin(int(e))
        ref.pinned.add(int(e))
    hot = rng.choice(n_total, 8, replace=False)  # a skewed pool: some steps hit
    for step in range(60):
        pool = hot if rng.random() < 0.6 else np.arange(n_total)
        idx = np.stack([rng.choice(pool, K, replace=False) for _ in range(T)]).astype(np.int32)
        if rng.random() < 0.2:
            idx[0, -1] = -1
        try:
            want = ref.request(idx.tolist())
        except CacheRefused:
            with pytest.raises(k3g.K3GError):
                cache.plan(idx)
            continue
        got = cache.plan(idx)
        assert got[0].tolist() == want[0] and got[1] == want[1], f"step {step}"
    stats, slot_of, hist = cache.query()
    assert (stats["hits"], stats["misses"], stats["evictions"]) == (ref.hits, ref.misses, ref.evictions)
    assert hist.tolist() == ref.hist
    assert slot_of.tolist() == [ref.where.get(e, -1) for e in range(n_total)]
    assert stats["misses"] > 0 and stats["hits"] > 0 and stats["evictions"] > 0
    cache.close()


def test_decode_step_refuses_on_the_host(k3g):
    # no cache, or a plan-only cache (no host bank to copy from): K3G_EINVAL
    # before any device work, and nothing planned
    L = k3g.lib()
    fake = k3g.C.c_void_p(4096)
    idx = np.array([0, 1], np.int32)
    assert L.k3g_cache_decode_step(None, fake, fake, idx.ctypes.data, fake, 2, 0, fake, 1 << 20, None, None) == -1
    arena = k3g.ExpertBank()
    arena.base = None
    arena.stride = 4096
    arena.n_experts = 4
    cache = k3g.ExpertCache(None, 8, arena)
    assert L.k3g_cache_decode_step(cache._c, fake, fake, idx.ctypes.data, fake, 2, 0, fake, 1 << 20, None,
                                   None) == -1
    assert cache.query()[0]["steps"] == 0
    cache.close()
