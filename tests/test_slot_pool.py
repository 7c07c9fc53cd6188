"""Host tests of the streaming-replay slot pool (hstu_pool_*): targeted cases of its
policy (freshness at the TTL boundary, room for the new events, least-recently-committed
eviction that spares the batch and uncommitted batches, abort), error paths that change
nothing, and long random request streams against an independent Python model of the
same policy. Nothing here touches a GPU."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa

OK, ERR_NULL, ERR_SHAPE, ERR_CAPACITY = 0, 1, 2, 4


class PolicyModel:
    """The pool's documented policy, written independently: per user a slot, a committed
    row count and the time and order of its last commit."""

    def __init__(self, slots, capacity, ttl):
        self.slots, self.capacity, self.ttl = slots, capacity, ttl
        self.owner = [None] * slots          # user per slot
        self.rows = [0] * slots
        self.last = [0] * slots
        self.order = [0] * slots             # commit counter value of the last commit
        self.pending = [False] * slots
        self.counter = 0
        self.stats = dict.fromkeys(hsa.POOL_STATS, 0)

    def assign(self, users, new, now):
        out = []
        held = {self.owner.index(u) for u in users if u in self.owner}
        for u, n in zip(users, new):
            if u in self.owner:
                s = self.owner.index(u)
                fresh = now - self.last[s] <= self.ttl
                if fresh and self.rows[s] + n <= self.capacity:
                    out.append((s, self.rows[s], 0))
                    self.stats["hits"] += 1
                else:
                    out.append((s, 0, 1))
                    self.stats["rebuild_full" if fresh else "rebuild_stale"] += 1
            else:
                out.append(None)
        for i, u in enumerate(users):
            if out[i] is not None:
                continue
            cands = [s for s in range(self.slots) if s not in held and not self.pending[s]]
            free = [s for s in cands if self.owner[s] is None]
            s = free[0] if free else min(cands, key=lambda s: self.order[s])
            if self.owner[s] is not None:
                self.stats["evictions"] += 1
            self.owner[s], self.rows[s], self.last[s], self.order[s] = u, 0, 0, 0
            held.add(s)
            out[i] = (s, 0, 1)
            self.stats["rebuild_new"] += 1
        for s, _, rb in out:
            self.pending[s] = True
            if rb:
                self.rows[s] = 0
        return out

    def commit(self, users, total, now):
        for u, t in zip(users, total):
            s = self.owner.index(u)
            self.counter += 1
            self.rows[s], self.last[s], self.order[s], self.pending[s] = t, now, self.counter, False


def test_fresh_cache_is_extended_until_ttl():
    pool = hsa.SlotPool(slots=2, capacity=100, ttl=10)
    slot, cached, rebuild = pool.assign([5], [30], now=0)
    assert rebuild.tolist() == [1] and cached.tolist() == [0]
    pool.commit([5], [30], now=0)
    # exactly ttl later: still fresh
    slot2, cached, rebuild = pool.assign([5], [20], now=10)
    assert slot2.tolist() == slot.tolist() and cached.tolist() == [30] and rebuild.tolist() == [0]
    pool.commit([5], [50], now=10)
    # ttl + 1 after the last commit: stale, encoded again in the same slot
    slot3, cached, rebuild = pool.assign([5], [1], now=21)
    assert slot3.tolist() == slot.tolist() and cached.tolist() == [0] and rebuild.tolist() == [1]
    pool.commit([5], [40], now=21)
    assert pool.lookup(5) == (int(slot[0]), 40)
    assert pool.stats() == {"hits": 1, "rebuild_new": 1, "rebuild_stale": 1, "rebuild_full": 0, "evictions": 0}


def test_no_room_means_encode_again():
    pool = hsa.SlotPool(slots=1, capacity=64, ttl=1000)
    pool.assign([1], [60], 0)
    pool.commit([1], [60], 0)
    _, cached, rebuild = pool.assign([1], [4], 1)          # 60 + 4 fits exactly
    assert cached.tolist() == [60] and rebuild.tolist() == [0]
    pool.commit([1], [64], 1)
    _, cached, rebuild = pool.assign([1], [1], 2)          # 64 + 1 does not
    assert cached.tolist() == [0] and rebuild.tolist() == [1]
    assert pool.stats()["rebuild_full"] == 1


def test_eviction_is_least_recently_committed_and_spares_the_batch():
    pool = hsa.SlotPool(slots=3, capacity=50, ttl=100)
    for t, u in enumerate([10, 11, 12]):
        pool.assign([u], [5], t)
        pool.commit([u], [5], t)
    pool.assign([10], [1], 3)                              # 10 becomes the most recent
    pool.commit([10], [6], 3)
    s11 = pool.lookup(11)[0]
    slot, _, _ = pool.assign([13], [2], 4)                 # evicts 11 (oldest commit)
    assert slot.tolist() == [s11] and pool.lookup(11) == (-1, 0)
    pool.commit([13], [2], 4)
    # 12 is now the oldest, but it is in the batch: 10 goes instead
    s10 = pool.lookup(10)[0]
    slot, cached, rebuild = pool.assign([12, 14], [1, 1], 5)
    assert slot.tolist()[1] == s10 and cached.tolist() == [5, 0] and rebuild.tolist() == [0, 1]
    assert pool.stats()["evictions"] == 2


def test_uncommitted_batches_hold_their_slots():
    pool = hsa.SlotPool(slots=2, capacity=50, ttl=100)
    pool.assign([1], [5], 0)                               # pending
    pool.assign([2], [5], 0)                               # pending, the other slot
    st, *_ = pool.assign_raw([3], [5], 1)                  # no slot that is not pending
    assert st == ERR_CAPACITY
    st, *_ = pool.assign_raw([1], [5], 1)                  # a pending user again
    assert st == ERR_SHAPE
    pool.commit([1], [5], 1)
    slot, _, _ = pool.assign([3], [5], 2)                  # now 1 can be evicted, 2 cannot
    assert slot.tolist() == [0] and pool.lookup(1) == (-1, 0)


def test_abort_frees_the_users():
    pool = hsa.SlotPool(slots=2, capacity=50, ttl=100)
    pool.assign([1, 2], [5, 6], 0)
    pool.commit([1, 2], [5, 6], 0)
    pool.assign([1], [3], 1)
    pool.abort([1])
    assert pool.lookup(1) == (-1, 0) and pool.lookup(2)[1] == 6
    _, cached, rebuild = pool.assign([1], [3], 2)
    assert cached.tolist() == [0] and rebuild.tolist() == [1]


@pytest.mark.parametrize("users,new,want", [
    ([1, 1], [1, 1], ERR_SHAPE),          # repeated user
    ([-1], [1], ERR_SHAPE),               # negative id
    ([1], [-1], ERR_CAPACITY),
    ([1], [51], ERR_CAPACITY),            # more new events than a slot holds
    ([1, 2, 3, 4], [1] * 4, ERR_CAPACITY),   # more users than slots
])
def test_assign_errors_change_nothing(users, new, want):
    pool = hsa.SlotPool(slots=3, capacity=50, ttl=100)
    pool.assign([9], [5], 0)
    pool.commit([9], [5], 0)
    before = (pool.stats(), pool.lookup(9))
    st, slot, cached, rebuild = pool.assign_raw(users, new, 1)
    assert st == want
    assert (slot == -7).all() and (cached == -7).all() and (rebuild == -7).all()   # outputs untouched
    assert (pool.stats(), pool.lookup(9)) == before


def test_commit_errors():
    pool = hsa.SlotPool(slots=2, capacity=50, ttl=100)
    pool.assign([1], [5], 0)
    assert pool.commit_raw([2], [5], 0) == ERR_SHAPE        # not assigned
    assert pool.commit_raw([1], [51], 0) == ERR_CAPACITY    # above capacity
    pool.commit([1], [5], 0)
    assert pool.commit_raw([1], [5], 0) == ERR_SHAPE        # no longer pending
    pool.assign([1], [5], 1)                                # cached 5
    assert pool.commit_raw([1], [4], 1) == ERR_CAPACITY     # below the cached rows


def test_create_errors():
    lib = hsa.load_library()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.hstu_pool_create(0, 10, 5, ctypes.byref(h)) == ERR_SHAPE
    assert lib.hstu_pool_create(2, 0, 5, ctypes.byref(h)) == ERR_SHAPE
    assert lib.hstu_pool_create(2, 10, -1, ctypes.byref(h)) == ERR_SHAPE
    assert lib.hstu_pool_create(2, 10, 5, None) == ERR_NULL


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_streams_match_the_policy_model(seed):
    rng = np.random.default_rng(seed)
    slots, cap, ttl = 6, 200, 25
    pool, model = hsa.SlotPool(slots, cap, ttl), PolicyModel(slots, cap, ttl)
    now = 0
    for _ in range(400):
        now += int(rng.integers(0, 6))
        B = int(rng.integers(1, slots + 1))
        users = [int(u) for u in rng.choice(20, size=B, replace=False)]
        new = [int(n) for n in rng.integers(0, 80, size=B)]
        slot, cached, rebuild = pool.assign(users, new, now)
        want = model.assign(users, new, now)
        assert list(zip(slot.tolist(), cached.tolist(), rebuild.tolist())) == want
        # rows after the encode: cached + the new events, or a window of the history
        total = [int(c) + n if not r else min(cap, n + int(rng.integers(0, 150)))
                 for c, n, r in zip(cached, new, rebuild)]
        pool.commit(users, total, now)
        model.commit(users, total, now)
        assert pool.stats() == model.stats
