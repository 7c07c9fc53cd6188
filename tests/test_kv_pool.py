"""Host tests of the streaming-replay page pool (hstu_pool_*): targeted cases of its
policy (freshness at the TTL boundary, room under max_rows, pages that follow a user's
rows, least-recently-committed eviction that spares the batch and uncommitted batches,
abort), error paths that change nothing, and long random request streams against an
independent Python model of the same policy. Nothing here touches a GPU."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa

OK, ERR_NULL, ERR_SHAPE, ERR_CAPACITY = 0, 1, 2, 4
PPU = 8   # pages_per_user in these tests


def npages(rows):
    return (rows + 63) // 64


class PolicyModel:
    """The pool's documented policy, written independently: per user its pages in position
    order, its committed rows, and the time and order of its last commit; a stack of free
    pages (a fresh pool hands out 0, 1, 2, ...)."""

    def __init__(self, pages, max_rows, ttl):
        self.max_rows, self.ttl = max_rows, ttl
        self.free = list(range(pages - 1, -1, -1))     # top of the stack last
        self.user = {}                                 # id -> dict(pages, len, last, order, pending)
        self.counter = 0
        self.stats = dict.fromkeys(hsa.POOL_STATS, 0)

    def fits(self, users, new, window, now):
        """Whether the batch fits (after evicting every user it may evict)."""
        dec = self._decide(users, new, window, now)
        demand = sum(npages(rows) - (len(self.user[u]["pages"]) if u in self.user else 0)
                     for u, (_, _, rows) in zip(users, dec))
        evictable = sum(len(e["pages"]) for u, e in self.user.items() if not e["pending"] and u not in users)
        return demand <= len(self.free) + evictable

    def _decide(self, users, new, window, now):
        dec = []
        for u, n, w in zip(users, new, window):
            e = self.user.get(u)
            if e is not None and now - e["last"] <= self.ttl and e["len"] + n <= self.max_rows:
                dec.append((e["len"], 0, e["len"] + n))
            else:
                dec.append((0, 1, w))
        return dec

    def assign(self, users, new, window, now):
        dec = []
        for u, n, w in zip(users, new, window):
            e = self.user.get(u)
            if e is not None and now - e["last"] <= self.ttl and e["len"] + n <= self.max_rows:
                dec.append((e["len"], 0, e["len"] + n))
            else:
                dec.append((0, 1, w))
        demand = sum(npages(rows) - (len(self.user[u]["pages"]) if u in self.user else 0)
                     for u, (_, _, rows) in zip(users, dec))
        lru = sorted((e["order"], u) for u, e in self.user.items() if not e["pending"] and u not in users)
        avail, evict = len(self.free), []
        for _, u in lru:
            if avail >= demand:
                break
            evict.append(u)
            avail += len(self.user[u]["pages"])
        for u in evict:
            self.free += self.user.pop(u)["pages"]
            self.stats["evictions"] += 1
        for u, (c, rb, rows) in zip(users, dec):
            e = self.user.get(u)
            if e is None:
                e = self.user[u] = dict(pages=[], len=0, last=0, order=0, pending=False)
                self.stats["rebuild_new"] += 1
            else:
                self.stats["hits" if not rb else "rebuild_full" if now - e["last"] <= self.ttl else "rebuild_stale"] += 1
            while len(e["pages"]) > npages(rows):
                self.free.append(e["pages"].pop())
        for u, (c, rb, rows) in zip(users, dec):
            e = self.user[u]
            while len(e["pages"]) < npages(rows):
                e["pages"].append(self.free.pop())
            e["pending"] = True
            if rb:
                e["len"] = 0
        self.stats["pages_in_use"] = sum(len(e["pages"]) for e in self.user.values())
        self.stats["pages_peak"] = max(self.stats["pages_peak"], self.stats["pages_in_use"])
        return [(list(self.user[u]["pages"]), c, rb) for u, (c, rb, _) in zip(users, dec)]

    def abort(self, users):
        for u in users:
            e = self.user.pop(u, None)
            if e is not None:
                self.free += e["pages"]
        self.stats["pages_in_use"] = sum(len(e["pages"]) for e in self.user.values())

    def commit(self, users, total, now):
        for u, t in zip(users, total):
            e = self.user[u]
            while len(e["pages"]) > npages(t):
                self.free.append(e["pages"].pop())
            self.counter += 1
            e.update(len=t, last=now, order=self.counter, pending=False)
        self.stats["pages_in_use"] = sum(len(e["pages"]) for e in self.user.values())


def rows_of(table):
    return [[int(p) for p in row if p >= 0] for row in table]


def test_fresh_cache_is_extended_until_ttl():
    pool = hsa.KvPool(pages=16, max_rows=500, ttl=10)
    table, cached, rebuild = pool.assign([5], [30], [30], now=0, pages_per_user=PPU)
    assert rebuild.tolist() == [1] and cached.tolist() == [0] and rows_of(table) == [[0]]
    assert (table[0, 1:] == -1).all()
    pool.commit([5], [30], now=0)
    # exactly ttl later: still fresh; 30 + 70 rows need a second page
    table, cached, rebuild = pool.assign([5], [70], [100], now=10, pages_per_user=PPU)
    assert cached.tolist() == [30] and rebuild.tolist() == [0] and rows_of(table) == [[0, 1]]
    pool.commit([5], [100], now=10)
    assert pool.lookup(5) == (100, 2)
    # ttl + 1 after the last commit: stale, encoded again in the user's own first page
    table, cached, rebuild = pool.assign([5], [1], [40], now=21, pages_per_user=PPU)
    assert cached.tolist() == [0] and rebuild.tolist() == [1] and rows_of(table) == [[0]]
    pool.commit([5], [40], now=21)
    assert pool.lookup(5) == (40, 1)
    assert pool.stats() == {"hits": 1, "rebuild_new": 1, "rebuild_stale": 1, "rebuild_full": 0, "evictions": 0,
                            "pages_in_use": 1, "pages_peak": 2}


def test_pages_follow_the_rows_held():
    """A user holds ceil(rows / 64) pages: memory in proportion to its history."""
    pool = hsa.KvPool(pages=64, max_rows=PPU * 64, ttl=1000)
    lens = {1: 1, 2: 64, 3: 65, 4: 300, 5: 512}
    pool.assign(list(lens), list(lens.values()), list(lens.values()), 0, PPU)
    pool.commit(list(lens), list(lens.values()), 0)
    for u, n in lens.items():
        assert pool.lookup(u) == (n, npages(n))
    assert pool.stats()["pages_in_use"] == sum(npages(n) for n in lens.values())


def test_no_room_means_encode_again():
    pool = hsa.KvPool(pages=8, max_rows=128, ttl=1000)
    pool.assign([1], [120], [120], 0, PPU)
    pool.commit([1], [120], 0)
    _, cached, rebuild = pool.assign([1], [8], [128], 1, PPU)        # 120 + 8 fits exactly
    assert cached.tolist() == [120] and rebuild.tolist() == [0]
    pool.commit([1], [128], 1)
    _, cached, rebuild = pool.assign([1], [1], [100], 2, PPU)        # 128 + 1 does not
    assert cached.tolist() == [0] and rebuild.tolist() == [1]
    assert pool.stats()["rebuild_full"] == 1


def test_eviction_is_least_recently_committed_and_spares_the_batch():
    pool = hsa.KvPool(pages=3, max_rows=192, ttl=100)
    for t, u in enumerate([10, 11, 12]):          # one page each
        pool.assign([u], [5], [5], t, PPU)
        pool.commit([u], [5], t)
    pool.assign([10], [1], [6], 3, PPU)            # 10 becomes the most recent
    pool.commit([10], [6], 3)
    p11 = 1
    table, _, _ = pool.assign([13], [2], [2], 4, PPU)   # evicts 11 (oldest commit)
    assert rows_of(table) == [[p11]] and pool.lookup(11) == (0, 0)
    pool.commit([13], [2], 4)
    # 12 is now the oldest, but it is in the batch: 10 goes instead
    table, cached, rebuild = pool.assign([12, 14], [1, 1], [6, 1], 5, PPU)
    assert rows_of(table)[1] == [0] and cached.tolist() == [5, 0] and rebuild.tolist() == [0, 1]
    assert pool.stats()["evictions"] == 2


def test_a_long_history_evicts_several_users():
    pool = hsa.KvPool(pages=4, max_rows=4 * 64, ttl=100)
    for t, u in enumerate([1, 2, 3, 4]):
        pool.assign([u], [10], [10], t, PPU)
        pool.commit([u], [10], t)
    table, _, _ = pool.assign([9], [150], [150], 9, PPU)     # three pages: the three oldest go
    assert len(rows_of(table)[0]) == 3 and [pool.lookup(u)[1] for u in (1, 2, 3, 4)] == [0, 0, 0, 1]
    assert pool.stats()["evictions"] == 3


def test_uncommitted_batches_hold_their_pages():
    pool = hsa.KvPool(pages=2, max_rows=64, ttl=100)
    pool.assign([1], [5], [5], 0, PPU)                       # pending
    pool.assign([2], [5], [5], 0, PPU)                       # pending, the other page
    st, *_ = pool.assign_raw([3], [5], [5], 1, PPU)          # no page that is not pending
    assert st == ERR_CAPACITY
    st, *_ = pool.assign_raw([1], [5], [5], 1, PPU)          # a pending user again
    assert st == ERR_SHAPE
    pool.commit([1], [5], 1)
    table, _, _ = pool.assign([3], [5], [5], 2, PPU)         # now 1 can be evicted, 2 cannot
    assert rows_of(table) == [[0]] and pool.lookup(1) == (0, 0)


def test_abort_frees_the_users():
    pool = hsa.KvPool(pages=4, max_rows=100, ttl=100)
    pool.assign([1, 2], [5, 6], [5, 6], 0, PPU)
    pool.commit([1, 2], [5, 6], 0)
    pool.assign([1], [3], [8], 1, PPU)
    pool.abort([1])
    assert pool.lookup(1) == (0, 0) and pool.lookup(2) == (6, 1)
    assert pool.stats()["pages_in_use"] == 1
    _, cached, rebuild = pool.assign([1], [3], [8], 2, PPU)
    assert cached.tolist() == [0] and rebuild.tolist() == [1]


def test_commit_frees_pages_beyond_the_rows_sent():
    pool = hsa.KvPool(pages=8, max_rows=400, ttl=100)
    table, _, _ = pool.assign([1], [300], [300], 0, PPU)     # 5 pages reserved
    assert len(rows_of(table)[0]) == 5
    pool.commit([1], [100], 0)                               # only 100 rows were sent
    assert pool.lookup(1) == (100, 2) and pool.stats()["pages_in_use"] == 2


@pytest.mark.parametrize("users,new,window,ppu,want", [
    ([1, 1], [1, 1], [1, 1], PPU, ERR_SHAPE),        # repeated user
    ([-1], [1], [1], PPU, ERR_SHAPE),                # negative id
    ([1], [-1], [1], PPU, ERR_SHAPE),
    ([1], [1], [201], PPU, ERR_SHAPE),               # window beyond max_rows
    ([1], [1], [1], 0, ERR_SHAPE),                   # no pages per user
    ([1], [1], [200], 3, ERR_CAPACITY),              # 200 rows need 4 pages
    ([1, 2, 3], [1] * 3, [200, 200, 200], PPU, ERR_CAPACITY),   # 12 pages from a pool of 10
])
def test_assign_errors_change_nothing(users, new, window, ppu, want):
    pool = hsa.KvPool(pages=10, max_rows=200, ttl=100)
    pool.assign([9], [5], [5], 0, PPU)
    pool.commit([9], [5], 0)
    before = (pool.stats(), pool.lookup(9))
    st, table, cached, rebuild = pool.assign_raw(users, new, window, 1, ppu)
    assert st == want
    assert (table == -7).all() and (cached == -7).all() and (rebuild == -7).all()   # outputs untouched
    assert (pool.stats(), pool.lookup(9)) == before


def test_commit_errors():
    pool = hsa.KvPool(pages=4, max_rows=100, ttl=100)
    pool.assign([1], [5], [5], 0, PPU)
    assert pool.commit_raw([2], [5], 0) == ERR_SHAPE        # not assigned
    assert pool.commit_raw([1], [101], 0) == ERR_CAPACITY   # above max_rows
    assert pool.commit_raw([1], [65], 0) == ERR_CAPACITY    # beyond its one page
    pool.commit([1], [5], 0)
    assert pool.commit_raw([1], [5], 0) == ERR_SHAPE        # no longer pending
    pool.assign([1], [5], [5], 1, PPU)                      # cached 5
    assert pool.commit_raw([1], [4], 1) == ERR_CAPACITY     # below the cached rows


def test_create_errors():
    lib = hsa.load_library()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.hstu_pool_create(0, 10, 5, ctypes.byref(h)) == ERR_SHAPE
    assert lib.hstu_pool_create(2, 0, 5, ctypes.byref(h)) == ERR_SHAPE
    assert lib.hstu_pool_create(2, 10, -1, ctypes.byref(h)) == ERR_SHAPE
    assert lib.hstu_pool_create(2, 10, 5, None) == ERR_NULL


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_streams_match_the_policy_model(seed):
    """400 random batches; about a third stay pending until the next batch and are then
    committed or aborted, so batches meet pages held by uncommitted users (and fail for want
    of pages, which must change nothing), stale users, full users and evictions."""
    rng = np.random.default_rng(seed)
    pages, max_rows, ttl = 24, 300, 12
    pool, model = hsa.KvPool(pages, max_rows, ttl), PolicyModel(pages, max_rows, ttl)
    now, held = 0, None          # held: (users, totals) of a batch left pending
    seen = set()
    for _ in range(400):
        now += int(rng.integers(0, 9))
        B = int(rng.integers(1, 5))
        pending = set(held[0]) if held else set()
        users = [int(u) for u in rng.choice([u for u in range(16) if u not in pending], size=B, replace=False)]
        new = [int(n) for n in rng.integers(0, 80, size=B)]
        window = [int(w) for w in rng.integers(0, max_rows + 1, size=B)]
        st, table, cached, rebuild = pool.assign_raw(users, new, window, now, PPU)
        assert (st == OK) == model.fits(users, new, window, now)
        if st == OK:
            want = model.assign(users, new, window, now)
            assert [(p, c, r) for p, c, r in zip(rows_of(table), cached.tolist(), rebuild.tolist())] == want
            # rows after the encode: cached + the new events, or the window sent again
            total = [int(c) + n if not r else w for c, n, w, r in zip(cached, new, window, rebuild)]
        else:
            seen.add("capacity")
        if held:                   # resolve the batch left pending before
            if rng.random() < 0.5:
                pool.commit(*held, now)
                model.commit(*held, now)
            else:
                pool.abort(held[0])
                model.abort(held[0])
                seen.add("abort")
            held = None
        if st == OK:
            if rng.random() < 0.35:
                held = (users, total)
            else:
                pool.commit(users, total, now)
                model.commit(users, total, now)
        assert pool.stats() == model.stats
        all_pages = [p for e in model.user.values() for p in e["pages"]]
        assert len(all_pages) == len(set(all_pages)) == model.stats["pages_in_use"]
        for u in range(16):
            e = model.user.get(u)
            if e is not None and not e["pending"]:
                assert pool.lookup(u) == (e["len"], len(e["pages"]))
    stats = pool.stats()
    assert all(stats[k] > 0 for k in ("hits", "rebuild_new", "rebuild_stale", "rebuild_full", "evictions"))
    assert seen == {"capacity", "abort"}
