// Host-side manager of the streaming key/value cache's user slots, for time-ordered
// request replay (the DLRMv3 page, section "Dataset selection": requests replayed in
// time order; section "Model selection": a user's history key/value state reused across
// consecutive timestamps). Cached user state goes stale: the multi-stage sequence model
// page's limitations section names staleness, and invalidation and TTL design, as a
// deciding factor. The pool decides, per request, whether a user's cached rows can be
// extended or the history must be encoded again, and which slot a user gets.
//
// Policy:
//  - a resident user whose cache is fresh (now - last use <= ttl) and has room for the
//    request's new events (cached + new <= capacity) keeps its slot and cached rows;
//  - otherwise the user's history is encoded again (cached length 0) in its own slot
//    if it has one, else in a free slot, else in the least recently used slot that no
//    other user of the same batch holds (its user is evicted);
//  - assignments take effect at once but stay pending until commit (the encode
//    succeeded: lengths and times recorded) or abort (the users' slots are freed).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "hstu.h"

struct hstu_slot_pool {
  int32_t slots = 0, capacity = 0;
  int64_t ttl = 0;
  struct Slot {
    int64_t user = -1;   // -1: free
    int32_t len = 0;     // cached rows (committed)
    int64_t last = 0;    // time of the last committed use
    uint64_t seq = 0;    // commit order, for least-recently-used eviction
    bool pending = false;
  };
  std::vector<Slot> slot;
  std::unordered_map<int64_t, int32_t> where;
  uint64_t seq = 0;
  int64_t stats[HSTU_POOL_STATS] = {};
};

namespace {

// A free slot if there is one, else the least recently committed one; never a slot
// held by this batch or by a batch that has not been committed yet.
int32_t free_or_lru(const hstu_slot_pool* p, const std::vector<char>& taken) {
  int32_t best = -1;
  for (int32_t s = 0; s < p->slots; ++s) {
    if (taken[s] || p->slot[s].pending) continue;
    if (p->slot[s].user < 0) return s;
    if (best < 0 || p->slot[s].seq < p->slot[best].seq) best = s;
  }
  return best;
}

}  // namespace

extern "C" {

hstu_status hstu_pool_create(int32_t slots, int32_t capacity, int64_t ttl, hstu_slot_pool** pool) {
  if (!pool) return HSTU_ERR_NULL;
  if (slots < 1 || capacity < 1 || ttl < 0) return HSTU_ERR_SHAPE;
  hstu_slot_pool* p = new (std::nothrow) hstu_slot_pool;
  if (!p) return HSTU_ERR_HIP;
  p->slots = slots;
  p->capacity = capacity;
  p->ttl = ttl;
  p->slot.resize(slots);
  *pool = p;
  return HSTU_OK;
}

void hstu_pool_destroy(hstu_slot_pool* pool) { delete pool; }

hstu_status hstu_pool_assign(hstu_slot_pool* p, int32_t B, const int64_t* user, const int32_t* new_events,
                             int64_t now, int32_t* slot_of_user, int32_t* cached_len, int32_t* rebuild) {
  if (!p) return HSTU_ERR_NULL;
  if (B < 0) return HSTU_ERR_SHAPE;
  if (B == 0) return HSTU_OK;
  if (!user || !new_events || !slot_of_user || !cached_len || !rebuild) return HSTU_ERR_NULL;
  if (B > p->slots) return HSTU_ERR_CAPACITY;
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < B; ++b) {
    if (user[b] < 0 || !seen.insert(user[b]).second) return HSTU_ERR_SHAPE;   // ids >= 0, distinct
    if (new_events[b] < 0 || new_events[b] > p->capacity) return HSTU_ERR_CAPACITY;
    auto it = p->where.find(user[b]);
    if (it != p->where.end() && p->slot[it->second].pending) return HSTU_ERR_SHAPE;   // not committed
  }
  // Decisions for resident users first (nothing is changed until every user has a slot),
  // so that a slot another user of this batch keeps is never chosen for eviction. The
  // caller's arrays are written only on success.
  std::vector<int32_t> so(B), cl(B), rb(B);
  std::vector<char> taken(p->slots, 0);
  int32_t newcomers = 0;
  for (int32_t b = 0; b < B; ++b) {
    auto it = p->where.find(user[b]);
    so[b] = -1;
    if (it == p->where.end()) {
      ++newcomers;
      continue;
    }
    const int32_t s = it->second;
    const hstu_slot_pool::Slot& e = p->slot[s];
    taken[s] = 1;
    so[b] = s;
    const bool fresh = now - e.last <= p->ttl;
    const bool room = (int64_t)e.len + new_events[b] <= p->capacity;
    cl[b] = fresh && room ? e.len : 0;
    rb[b] = fresh && room ? 0 : 1;
  }
  int32_t available = 0;
  for (int32_t s = 0; s < p->slots; ++s) available += !taken[s] && !p->slot[s].pending;
  if (newcomers > available) return HSTU_ERR_CAPACITY;   // slots held by uncommitted batches
  for (int32_t b = 0; b < B; ++b) {
    if (so[b] < 0) continue;
    const hstu_slot_pool::Slot& e = p->slot[so[b]];
    ++p->stats[!rb[b] ? HSTU_POOL_HITS
               : now - e.last <= p->ttl ? HSTU_POOL_REBUILD_FULL : HSTU_POOL_REBUILD_STALE];
  }
  for (int32_t b = 0; b < B; ++b) {
    if (so[b] >= 0) continue;
    const int32_t s = free_or_lru(p, taken);   // exists: counted above
    hstu_slot_pool::Slot& e = p->slot[s];
    if (e.user >= 0) {
      p->where.erase(e.user);
      ++p->stats[HSTU_POOL_EVICTIONS];
    }
    e = hstu_slot_pool::Slot{};
    e.user = user[b];
    p->where[user[b]] = s;
    taken[s] = 1;
    so[b] = s;
    cl[b] = 0;
    rb[b] = 1;
    ++p->stats[HSTU_POOL_REBUILD_NEW];
  }
  for (int32_t b = 0; b < B; ++b) {
    hstu_slot_pool::Slot& e = p->slot[so[b]];
    e.pending = true;
    if (rb[b]) e.len = 0;   // the old rows are no longer valid
    slot_of_user[b] = so[b];
    cached_len[b] = cl[b];
    rebuild[b] = rb[b];
  }
  return HSTU_OK;
}

hstu_status hstu_pool_commit(hstu_slot_pool* p, int32_t B, const int64_t* user, const int32_t* total_len,
                             int64_t now) {
  if (!p) return HSTU_ERR_NULL;
  if (B < 0) return HSTU_ERR_SHAPE;
  if (B == 0) return HSTU_OK;
  if (!user || !total_len) return HSTU_ERR_NULL;
  for (int32_t b = 0; b < B; ++b) {
    auto it = p->where.find(user[b]);
    if (it == p->where.end() || !p->slot[it->second].pending) return HSTU_ERR_SHAPE;
    if (total_len[b] < p->slot[it->second].len || total_len[b] > p->capacity) return HSTU_ERR_CAPACITY;
  }
  for (int32_t b = 0; b < B; ++b) {
    hstu_slot_pool::Slot& e = p->slot[p->where[user[b]]];
    e.len = total_len[b];
    e.last = now;
    e.seq = ++p->seq;
    e.pending = false;
  }
  return HSTU_OK;
}

hstu_status hstu_pool_abort(hstu_slot_pool* p, int32_t B, const int64_t* user) {
  if (!p) return HSTU_ERR_NULL;
  if (B < 0) return HSTU_ERR_SHAPE;
  if (B > 0 && !user) return HSTU_ERR_NULL;
  for (int32_t b = 0; b < B; ++b) {
    auto it = p->where.find(user[b]);
    if (it == p->where.end()) continue;
    p->slot[it->second] = hstu_slot_pool::Slot{};
    p->where.erase(it);
  }
  return HSTU_OK;
}

hstu_status hstu_pool_stats(const hstu_slot_pool* p, int64_t* stats, int32_t n) {
  if (!p || !stats) return HSTU_ERR_NULL;
  if (n < 0) return HSTU_ERR_SHAPE;
  for (int32_t k = 0; k < n; ++k) stats[k] = k < HSTU_POOL_STATS ? p->stats[k] : 0;
  return HSTU_OK;
}

hstu_status hstu_pool_lookup(const hstu_slot_pool* p, int64_t user, int32_t* slot, int32_t* len) {
  if (!p || !slot || !len) return HSTU_ERR_NULL;
  auto it = p->where.find(user);
  if (it == p->where.end()) {
    *slot = -1;
    *len = 0;
  } else {
    *slot = it->second;
    *len = p->slot[it->second].len;
  }
  return HSTU_OK;
}

}  // extern "C"
