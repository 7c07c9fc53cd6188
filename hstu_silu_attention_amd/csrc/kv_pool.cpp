// Host-side manager of a paged key/value cache, for time-ordered request replay (the
// DLRMv3 page, section "Dataset selection": requests replayed in time order; section
// "Model selection": a user's history key/value state reused across consecutive
// timestamps). Cached user state goes stale: the multi-stage sequence model page's
// limitations section names staleness, and invalidation and TTL design, as a deciding
// factor. Per request the pool decides whether a user's cached rows are extended or its
// history is encoded again, and which pages of the cache hold the user's rows: a user
// holds ceil(rows / 64) pages, so the cache memory a user takes follows its history.
//
// Policy:
//  - a resident user whose rows are fresh (now - last commit <= ttl) and can take the
//    request's new events (rows + new <= max_rows) keeps its rows and pages, and gets
//    more pages for the new rows;
//  - otherwise its history is encoded again from position 0 (the caller resends its
//    latest `window` events), reusing the user's pages;
//  - pages come from the free list; when too few are free, the least recently committed
//    users outside the batch and not pending are evicted whole, oldest first;
//  - assignments take effect at once but stay pending until commit (the encode
//    succeeded: lengths and times recorded, pages beyond the rows freed) or abort (the
//    users' pages are freed and the users forgotten).
#include <algorithm>
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "hstu.h"

namespace {
constexpr int32_t kRows = 64;   // rows per page (hstu_kv_cache's page_rows)
int32_t pages_for(int64_t rows) { return (int32_t)((rows + kRows - 1) / kRows); }
}  // namespace

struct hstu_kv_pool {
  int32_t pages = 0, max_rows = 0;
  int64_t ttl = 0;
  struct User {
    std::vector<int32_t> pages;   // in position order: pages[i] holds rows 64i .. 64i+63
    int32_t len = 0;              // committed rows
    int64_t last = 0;             // time of the last commit
    uint64_t seq = 0;             // commit order (least recently committed first)
    bool pending = false;
  };
  std::unordered_map<int64_t, User> users;
  std::set<std::pair<uint64_t, int64_t>> lru;   // (seq, user) of committed, not pending users
  std::vector<int32_t> free_pages;              // a stack
  uint64_t seq = 0;
  int64_t stats[HSTU_POOL_STATS] = {};

  int32_t in_use() const { return pages - (int32_t)free_pages.size(); }
  void note_use() { stats[HSTU_POOL_PAGES_PEAK] = std::max<int64_t>(stats[HSTU_POOL_PAGES_PEAK], in_use()); }
  void release(User& u) {
    for (int32_t p : u.pages) free_pages.push_back(p);
    u.pages.clear();
  }
};

extern "C" {

hstu_status hstu_pool_create(int32_t pages, int32_t max_rows, int64_t ttl, hstu_kv_pool** pool) {
  if (!pool) return HSTU_ERR_NULL;
  if (pages < 1 || max_rows < 1 || ttl < 0) return HSTU_ERR_SHAPE;
  hstu_kv_pool* p = new (std::nothrow) hstu_kv_pool;
  if (!p) return HSTU_ERR_HIP;
  p->pages = pages;
  p->max_rows = max_rows;
  p->ttl = ttl;
  try {
    p->free_pages.reserve((size_t)pages);
    // lowest ids on top of the stack: a fresh pool hands out pages 0, 1, 2, ...
    for (int32_t i = pages - 1; i >= 0; --i) p->free_pages.push_back(i);
  } catch (...) {
    delete p;
    return HSTU_ERR_HIP;
  }
  *pool = p;
  return HSTU_OK;
}

void hstu_pool_destroy(hstu_kv_pool* pool) { delete pool; }

hstu_status hstu_pool_assign(hstu_kv_pool* p, int32_t B, const int64_t* user, const int32_t* new_events,
                             const int32_t* window, int64_t now, int32_t pages_per_user, int32_t* page_table,
                             int32_t* cached_len, int32_t* rebuild) {
  if (!p) return HSTU_ERR_NULL;
  if (B < 0 || pages_per_user < 1) return HSTU_ERR_SHAPE;
  if (B == 0) return HSTU_OK;
  if (!user || !new_events || !window || !page_table || !cached_len || !rebuild) return HSTU_ERR_NULL;
  // Decide every user's rows first (nothing changes until the whole batch fits).
  std::unordered_set<int64_t> seen;
  std::vector<int32_t> cl(B), rb(B), need(B), held(B);
  int64_t demand = 0;   // pages the batch takes beyond what its users hold
  for (int32_t b = 0; b < B; ++b) {
    if (user[b] < 0 || !seen.insert(user[b]).second) return HSTU_ERR_SHAPE;   // ids >= 0, distinct
    if (new_events[b] < 0 || window[b] < 0 || window[b] > p->max_rows) return HSTU_ERR_SHAPE;
    auto it = p->users.find(user[b]);
    int64_t rows = window[b];
    cl[b] = 0;
    rb[b] = 1;
    held[b] = 0;
    if (it != p->users.end()) {
      const hstu_kv_pool::User& u = it->second;
      if (u.pending) return HSTU_ERR_SHAPE;   // not committed yet
      held[b] = (int32_t)u.pages.size();
      const bool fresh = now - u.last <= p->ttl;
      if (fresh && (int64_t)u.len + new_events[b] <= p->max_rows) {
        cl[b] = u.len;
        rb[b] = 0;
        rows = (int64_t)u.len + new_events[b];
      }
    }
    need[b] = pages_for(rows);
    if (need[b] > pages_per_user) return HSTU_ERR_CAPACITY;
    demand += need[b] - held[b];
  }
  // Users to evict, least recently committed first, until the batch fits.
  std::vector<int64_t> evict;
  int64_t avail = (int64_t)p->free_pages.size();
  for (auto it = p->lru.begin(); avail < demand && it != p->lru.end(); ++it) {
    if (seen.count(it->second)) continue;
    evict.push_back(it->second);
    avail += (int64_t)p->users[it->second].pages.size();
  }
  if (avail < demand) return HSTU_ERR_CAPACITY;
  // Apply.
  for (int64_t v : evict) {
    hstu_kv_pool::User& u = p->users[v];
    p->lru.erase({u.seq, v});
    p->release(u);
    p->users.erase(v);
    ++p->stats[HSTU_POOL_EVICTIONS];
  }
  for (int32_t b = 0; b < B; ++b) {
    auto it = p->users.find(user[b]);
    if (it == p->users.end()) {
      it = p->users.emplace(user[b], hstu_kv_pool::User{}).first;
      ++p->stats[HSTU_POOL_REBUILD_NEW];
    } else {
      hstu_kv_pool::User& u = it->second;
      p->lru.erase({u.seq, user[b]});
      ++p->stats[!rb[b] ? HSTU_POOL_HITS : now - u.last <= p->ttl ? HSTU_POOL_REBUILD_FULL : HSTU_POOL_REBUILD_STALE];
    }
    hstu_kv_pool::User& u = it->second;
    // a rebuild keeps the user's pages for its new rows (positions restart at 0)
    while ((int32_t)u.pages.size() > need[b]) {
      p->free_pages.push_back(u.pages.back());
      u.pages.pop_back();
    }
  }
  for (int32_t b = 0; b < B; ++b) {
    hstu_kv_pool::User& u = p->users[user[b]];
    while ((int32_t)u.pages.size() < need[b]) {
      u.pages.push_back(p->free_pages.back());
      p->free_pages.pop_back();
    }
    u.pending = true;
    if (rb[b]) u.len = 0;   // the old rows are no longer valid
    int32_t* row = page_table + (size_t)b * pages_per_user;
    for (int32_t i = 0; i < pages_per_user; ++i) row[i] = i < (int32_t)u.pages.size() ? u.pages[i] : -1;
    cached_len[b] = cl[b];
    rebuild[b] = rb[b];
  }
  p->note_use();
  return HSTU_OK;
}

hstu_status hstu_pool_commit(hstu_kv_pool* p, int32_t B, const int64_t* user, const int32_t* total_len,
                             int64_t now) {
  if (!p) return HSTU_ERR_NULL;
  if (B < 0) return HSTU_ERR_SHAPE;
  if (B == 0) return HSTU_OK;
  if (!user || !total_len) return HSTU_ERR_NULL;
  for (int32_t b = 0; b < B; ++b) {
    auto it = p->users.find(user[b]);
    if (it == p->users.end() || !it->second.pending) return HSTU_ERR_SHAPE;
    const hstu_kv_pool::User& u = it->second;
    if (total_len[b] < u.len || total_len[b] > p->max_rows || pages_for(total_len[b]) > (int32_t)u.pages.size())
      return HSTU_ERR_CAPACITY;
  }
  for (int32_t b = 0; b < B; ++b) {
    hstu_kv_pool::User& u = p->users[user[b]];
    while ((int32_t)u.pages.size() > pages_for(total_len[b])) {   // pages beyond the rows sent
      p->free_pages.push_back(u.pages.back());
      u.pages.pop_back();
    }
    u.len = total_len[b];
    u.last = now;
    u.seq = ++p->seq;
    u.pending = false;
    p->lru.insert({u.seq, user[b]});
  }
  return HSTU_OK;
}

hstu_status hstu_pool_abort(hstu_kv_pool* p, int32_t B, const int64_t* user) {
  if (!p) return HSTU_ERR_NULL;
  if (B < 0) return HSTU_ERR_SHAPE;
  if (B > 0 && !user) return HSTU_ERR_NULL;
  for (int32_t b = 0; b < B; ++b) {
    auto it = p->users.find(user[b]);
    if (it == p->users.end()) continue;
    if (!it->second.pending) p->lru.erase({it->second.seq, user[b]});
    p->release(it->second);
    p->users.erase(it);
  }
  return HSTU_OK;
}

hstu_status hstu_pool_stats(const hstu_kv_pool* p, int64_t* stats, int32_t n) {
  if (!p || !stats) return HSTU_ERR_NULL;
  if (n < 0) return HSTU_ERR_SHAPE;
  for (int32_t k = 0; k < n; ++k)
    stats[k] = k == HSTU_POOL_PAGES_IN_USE ? p->in_use() : k < HSTU_POOL_STATS ? p->stats[k] : 0;
  return HSTU_OK;
}

hstu_status hstu_pool_lookup(const hstu_kv_pool* p, int64_t user, int32_t* len, int32_t* pages) {
  if (!p || !len || !pages) return HSTU_ERR_NULL;
  auto it = p->users.find(user);
  *len = it == p->users.end() ? 0 : it->second.len;
  *pages = it == p->users.end() ? 0 : (int32_t)it->second.pages.size();
  return HSTU_OK;
}

}  // extern "C"
