"""Host logic of the partial-residency cache (planning mode: no device work).

A plain Python model of the eviction rule stated in include/moe_layer.h (fewest
uses, then oldest last use, then lower (layer, id); empty slots first, lowest
first; blobs of the current call and of unreleased calls are never victims)
is replayed beside the library on random call sequences, and every slot
assignment and counter must agree.  The pages name the policy only as
frequency plus recency (linlog.top article, core design 3, the expert cache
pool; Swiftlet README translation, "How it works"), so this pins our stated
reading, not the pages.
"""

import numpy as np
import pytest

import int4_quantized_expert_amd as M


class PolicyModel:
    def __init__(self, n_slots, n_layers, n_experts, keep_counts=False):
        self.keep_counts = keep_counts
        self.count = {}
        self.slots = [dict(layer=-1, id=-1, uses=0, last=-1, held=0) for _ in range(n_slots)]
        self.where = {}
        self.tick = 0
        self.hits = self.misses = self.evictions = 0
        self.pending = {l: [] for l in range(n_layers)}

    def _key(self, s):
        x = self.slots[s]
        return (0 if x["layer"] < 0 else 1, x["uses"], x["last"], x["layer"], x["id"], s)

    def acquire(self, layer, ids):
        need = sorted(set(int(e) for e in ids))
        now = self.tick
        self.tick += 1
        table, held = {}, []
        for e in need:
            s = self.where.get((layer, e))
            if s is not None:
                x = self.slots[s]
                x["held"] += 1
                self.count[(layer, e)] = self.count.get((layer, e), 0) + 1
                x["uses"] = self.count[(layer, e)] if self.keep_counts else x["uses"] + 1
                x["last"] = now
                table[e] = s
                held.append(s)
                self.hits += 1
        for e in need:
            if e in table:
                continue
            free = [s for s in range(len(self.slots)) if self.slots[s]["held"] == 0]
            s = min(free, key=self._key)
            x = self.slots[s]
            if x["layer"] >= 0:
                del self.where[(x["layer"], x["id"])]
                self.evictions += 1
            self.count[(layer, e)] = self.count.get((layer, e), 0) + 1
            x.update(layer=layer, id=e, uses=self.count[(layer, e)] if self.keep_counts else 1, last=now)
            x["held"] += 1
            self.where[(layer, e)] = s
            table[e] = s
            held.append(s)
            self.misses += 1
        self.pending[layer].append(held)
        return table

    def release(self, layer):
        for s in self.pending[layer].pop(0):
            self.slots[s]["held"] -= 1


def _run(seed, n_slots, n_layers, n_experts, n_calls, k, depth, keep_counts=False):
    rng = np.random.default_rng(seed)
    stride = 4096
    cache = M.ExpertCache(n_slots, stride, None, None, n_layers, n_experts)
    cache.set_policy(keep_counts)
    model = PolicyModel(n_slots, n_layers, n_experts, keep_counts)
    popularity = 1.0 / np.arange(1, n_experts + 1) ** 1.1
    popularity /= popularity.sum()
    inflight = []
    for c in range(n_calls):
        layer = int(rng.integers(n_layers))
        perm = rng.permutation(n_experts)
        tokens = int(rng.integers(1, 6))
        ids = np.concatenate([perm[rng.choice(n_experts, size=k, replace=False, p=popularity)]
                              for _ in range(tokens)]).astype(np.int32)
        table = np.full(n_experts, -1, dtype=np.int64)
        expect = model.acquire(layer, ids)
        cache.acquire(layer, ids, table)
        for e, s in expect.items():
            assert table[e] == s * stride, (c, e)
            assert cache.slot_of(layer, e) == s
        assert cache.stats() == (model.hits, model.misses, model.evictions)
        inflight.append(layer)
        while len(inflight) > depth:
            l0 = inflight.pop(0)
            model.release(l0)
            cache.release(l0)
    cache.close()
    return model


@pytest.mark.parametrize("seed,depth,keep", [(1, 0, False), (2, 1, False), (3, 2, False), (4, 0, True),
                                             (5, 2, True)])
def test_policy_matches_model(seed, depth, keep):
    m = _run(seed, n_slots=48, n_layers=3, n_experts=40, n_calls=300, k=4, depth=depth, keep_counts=keep)
    assert m.evictions > 50 and m.hits > 50


def test_kept_counts_bring_a_hot_expert_back_for_good():
    """A hot expert pushed out by a burst of others comes back.  With counts
    restarting at eviction it returns with one use and is the next victim
    every time; with counts kept it returns with its history and stays."""
    def run(keep):
        cache = M.ExpertCache(3, 256, None, None, 1, 32)
        cache.set_policy(keep)
        t = np.zeros(32, dtype=np.int64)

        def call(ids):
            cache.acquire(0, ids, t)
            cache.release(0)
        for _ in range(10):                      # expert 0 is hot
            call([0])
        for _ in range(3):                       # a burst that needs every slot
            call([1, 2, 3])
        assert cache.slot_of(0, 0) == -1
        hits0 = cache.stats()[0]
        for j in range(10):                      # 0 between cold experts
            call([0])
            call([4 + j])
        return cache.stats()[0] - hits0
    assert run(False) == 0
    assert run(True) == 9                        # a miss on its return, then a hit every time


def test_injected_copy_failure_leaves_nothing_of_the_call_resident():
    """A copy that fails (injected; MOE_EHIP) rolls its call back: none of the
    experts it missed is resident, its hits are released, counters are those
    before the call, and the cache keeps working."""
    cache = M.ExpertCache(6, 256, None, None, 2, 16)
    t = np.zeros(16, dtype=np.int64)
    cache.acquire(0, [1, 2, 3], t)               # held (not released)
    before = cache.stats()
    cache.inject_fault(1)                        # the second copy from now fails
    with pytest.raises(M.MoeError) as ei:
        cache.acquire(0, [3, 4, 5, 6], t)        # hit 3; misses 4, 5, 6
    assert ei.value.code == -3
    assert [cache.slot_of(0, e) for e in (4, 5, 6)] == [-1, -1, -1]
    assert all(cache.slot_of(0, e) >= 0 for e in (1, 2, 3))
    assert cache.stats() == before
    cache.acquire(0, [3, 4, 5, 6], t)            # the same call now goes through
    assert all(cache.slot_of(0, e) >= 0 for e in (3, 4, 5, 6))
    cache.release(0)
    cache.release(0)
    with pytest.raises(M.MoeError):
        cache.release(0)                         # the failed call left no pending hold
    cache.inject_fault(0)
    with pytest.raises(M.MoeError):
        cache.acquire(1, [7], t)
    cache.inject_fault(-1)
    cache.acquire(1, [7], t)
    assert cache.slot_of(1, 7) >= 0


def test_hot_experts_stay_resident():
    """Under a skewed load the most used experts are the last to go."""
    cache = M.ExpertCache(4, 256, None, None, 1, 16)
    t = np.zeros(16, dtype=np.int64)
    for _ in range(5):
        cache.acquire(0, [0, 1], t)
        cache.release(0)
    for e in range(2, 12):
        cache.acquire(0, [e], t)
        cache.release(0)
    assert cache.slot_of(0, 0) >= 0 and cache.slot_of(0, 1) >= 0
    h, m, ev = cache.stats()
    assert (h, m, ev) == (8, 12, 8)


def test_errors():
    cache = M.ExpertCache(3, 256, None, None, 2, 8)
    t = np.zeros(8, dtype=np.int64)
    with pytest.raises(M.MoeError) as ei:
        cache.acquire(0, [0, 1, 2, 3], t)           # four distinct experts, three slots
    assert ei.value.code == -6
    with pytest.raises(M.MoeError) as ei:
        cache.acquire(0, [9], t)
    assert ei.value.code == -1
    with pytest.raises(M.MoeError):
        cache.release(1)                             # nothing acquired for layer 1
    cache.acquire(0, [0, 1], t)                      # held until released
    with pytest.raises(M.MoeError) as ei:
        cache.acquire(1, [4, 5], t)                  # only one slot is free of held blobs
    assert ei.value.code == -6
    cache.acquire(1, [4], t)
    cache.release(0)
    cache.release(1)
    cache.acquire(1, [5, 6, 7], t)                   # everything evictable again
    assert cache.stats()[2] == 3
    with pytest.raises(M.MoeError):
        M.ExpertCache(0, 256, None, None, 1, 8)
    with pytest.raises(M.MoeError):
        M.ExpertCache(4, 100, None, None, 1, 8)      # stride not a multiple of 256
