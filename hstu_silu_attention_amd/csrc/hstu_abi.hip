// Host side of the C ABI declared in include/hstu.h: argument validation, the
// jagged work planner, the pinned staging ring and the per-layer launch sequence.
//
// Validation is complete before anything is enqueued, so every error except
// HSTU_ERR_HIP leaves the device and every host array untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <numeric>
#include <unordered_map>
#include <vector>

#include "hstu.h"
#include "hstu_internal.h"

namespace {

using hstu::UserRec;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

hstu_status check_dims(const hstu_dims* d) {
  if (!d) return HSTU_ERR_NULL;
  if (d->layers < 1 || d->d_model <= 0 || d->heads <= 0 || d->max_len < 1) return HSTU_ERR_SHAPE;
  if (d->d_model % d->heads) return HSTU_ERR_SHAPE;
  // a position table holds fewer than 2^31 elements (the kernels index it in 32 bits)
  if ((int64_t)d->max_len * 3 * d->d_model >= ((int64_t)1 << 31)) return HSTU_ERR_SHAPE;
  const int dh = d->d_model / d->heads;
  if (d->dtype == HSTU_F32) {
    if (d->d_model % 64 || (dh != 32 && dh != 64 && dh != 128)) return HSTU_ERR_SHAPE;
  } else if (d->dtype == HSTU_BF16) {
    if (d->d_model % 128 || (dh != 64 && dh != 128)) return HSTU_ERR_SHAPE;
  } else {
    return HSTU_ERR_SHAPE;
  }
  return HSTU_OK;
}

// Offsets are the exclusive running sum of per-user lengths: start at 0, never decrease.
hstu_status check_offsets(int32_t B, const int32_t* uo, const int32_t* co) {
  if (B < 0) return HSTU_ERR_SHAPE;
  if (B == 0) return HSTU_OK;
  if (!uo || !co) return HSTU_ERR_NULL;
  if (uo[0] != 0 || co[0] != 0) return HSTU_ERR_OFFSETS;
  for (int32_t b = 0; b < B; ++b)
    if (uo[b + 1] < uo[b] || co[b + 1] < co[b]) return HSTU_ERR_OFFSETS;
  if ((int64_t)uo[B] + (int64_t)co[B] > INT32_MAX) return HSTU_ERR_SHAPE;
  return HSTU_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Layout {
  int32_t Nu = 0, Nc = 0, T = 0;
  int64_t ntiles = 0;
  size_t users = 0, wptr = 0, items = 0, rows = 0, xn = 0, cs = 0, st = 0, vqk = 0, aout = 0, x = 0, total = 0;
  size_t staged = 0;  // host-planned part: users table, W1 pointers, attention items (copied up to the grid)
};

Layout make_layout(const hstu_dims* d, int32_t B, const int32_t* uo, const int32_t* co) {
  Layout L;
  if (B > 0) {
    L.Nu = uo[B];
    L.Nc = co[B];
  }
  L.T = L.Nu + L.Nc;
  const int bm = hstu::attn_block_rows(d->dtype);
  for (int32_t b = 0; b < B; ++b)
    L.ntiles += d->heads * (cdiv(uo[b + 1] - uo[b], bm) + cdiv(co[b + 1] - co[b], bm));
  const size_t es = d->dtype == HSTU_F32 ? 4 : 2;
  const size_t D = (size_t)d->d_model, T = (size_t)L.T;
  // GEMM operands (xn, vqk, aout) are padded to whole 256-row tiles.
  const size_t Tp = (size_t)cdiv(L.T, hstu::kRowPad) * hstu::kRowPad;
  size_t off = 0;
  L.users = off; off += align_up((size_t)B * sizeof(UserRec));
  L.wptr = off; off += align_up((size_t)d->layers * sizeof(void*));
  // one item per attention workgroup: kXcds bins of at most ntiles items each
  L.items = off; off += align_up((size_t)hstu::kXcds * L.ntiles * sizeof(hstu::AttnItem));
  L.staged = off;
  L.rows = off; off += align_up(T * 8);
  // float32 models normalise into xn; bfloat16 models normalise inside the projection
  // and need the column sums of W1 instead
  L.xn = off; off += d->dtype == HSTU_F32 ? align_up(Tp * D * es) : 0;
  L.cs = off; off += d->dtype == HSTU_F32 ? 0 : align_up((size_t)d->layers * 4 * D * sizeof(float));
  L.st = off; off += d->dtype == HSTU_F32 ? 0 : align_up(T * (D / 128) * 2 * sizeof(float));
  L.vqk = off; off += align_up(Tp * 3 * D * es);
  L.aout = off; off += align_up(Tp * 3 * D * es);
  L.x = off; off += d->layers > 1 ? align_up(T * D * es) : 0;
  L.total = L.T == 0 ? 0 : off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// ---------------------------------------------------------------- pinned staging ring
// The plan (users table + tile list) is written into pinned host memory and copied
// asynchronously into the workspace. A ring slot is reused only after the copy that
// last read it has completed (its event), so a call never waits for the device
// unless more than kRing calls are in flight on the device.
constexpr int kRing = 4;
struct StageSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
struct DeviceStage {
  StageSlot slot[kRing];
  int next = 0;
};
std::mutex g_stage_mu;
std::unordered_map<int, DeviceStage> g_stage;

hstu_status stage_and_copy(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HSTU_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_stage_mu);
  DeviceStage& ds = g_stage[dev];
  StageSlot& s = ds.slot[ds.next];
  ds.next = (ds.next + 1) % kRing;
  if (s.pending) {
    if (hipEventSynchronize(s.ev) != hipSuccess) return HSTU_ERR_HIP;
    s.pending = false;
  }
  if (s.cap < bytes) {
    if (s.host && hipHostFree(s.host) != hipSuccess) return HSTU_ERR_HIP;
    s.host = nullptr;
    s.cap = 0;
    size_t cap = std::max<size_t>(bytes, 64 * 1024);
    if (hipHostMalloc(&s.host, cap, hipHostMallocDefault) != hipSuccess) return HSTU_ERR_HIP;
    s.cap = cap;
  }
  if (!s.ev && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) return HSTU_ERR_HIP;
  std::memcpy(s.host, src, bytes);
  if (hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
    return HSTU_ERR_HIP;
  if (hipEventRecord(s.ev, stream) != hipSuccess) return HSTU_ERR_HIP;
  s.pending = true;
  return HSTU_OK;
}

// ---------------------------------------------------------------- per-kernel timing
struct Timing {
  std::mutex mu;
  bool on = false;
  uint32_t mask = 0xffffffffu;   // kernel kinds that get events while timing is on
  struct Rec { int kind; hipEvent_t a, b; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  double ms[HSTU_KERNEL_KINDS] = {};
  int64_t n[HSTU_KERNEL_KINDS] = {};
};
Timing g_timing;

hipEvent_t timing_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch through `f`, bracketed by events on `s` while timing is on.
template <typename F>
hipError_t timed_launch(int kind, hipStream_t s, F&& f) {
  std::unique_lock<std::mutex> lock(g_timing.mu);
  if (!g_timing.on || !((g_timing.mask >> kind) & 1u)) {
    lock.unlock();
    return f();
  }
  hipEvent_t a = timing_event(), b = timing_event();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = f();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  g_timing.recs.push_back({kind, a, b});
  return hipSuccess;
}

}  // namespace

extern "C" {

hstu_status hstu_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (enable) {
    for (auto& r : g_timing.recs) {
      if (hipEventSynchronize(r.b) != hipSuccess) return HSTU_ERR_HIP;
      g_timing.pool.push_back(r.a);
      g_timing.pool.push_back(r.b);
    }
    g_timing.recs.clear();
    for (int k = 0; k < HSTU_KERNEL_KINDS; ++k) {
      g_timing.ms[k] = 0.0;
      g_timing.n[k] = 0;
    }
  }
  g_timing.on = enable != 0;
  return HSTU_OK;
}

hstu_status hstu_timing_select(uint32_t kinds_mask) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  g_timing.mask = kinds_mask;
  return HSTU_OK;
}

hstu_status hstu_timing_read(double* total_ms, int64_t* launches, int32_t kinds) {
  if (!total_ms || !launches) return HSTU_ERR_NULL;
  if (kinds < 0) return HSTU_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  for (auto& r : g_timing.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return HSTU_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return HSTU_ERR_HIP;
    g_timing.ms[r.kind] += ms;
    g_timing.n[r.kind] += 1;
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.recs.clear();
  for (int k = 0; k < kinds; ++k) {
    total_ms[k] = k < HSTU_KERNEL_KINDS ? g_timing.ms[k] : 0.0;
    launches[k] = k < HSTU_KERNEL_KINDS ? g_timing.n[k] : 0;
  }
  for (int k = 0; k < HSTU_KERNEL_KINDS; ++k) {
    g_timing.ms[k] = 0.0;
    g_timing.n[k] = 0;
  }
  return HSTU_OK;
}

int32_t hstu_abi_version(void) { return HSTU_ABI_VERSION; }

const char* hstu_status_string(hstu_status s) {
  switch (s) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_NULL: return "a required pointer is NULL";
    case HSTU_ERR_SHAPE: return "unsupported dimensions, dtype or batch size";
    case HSTU_ERR_OFFSETS: return "offsets must start at 0 and never decrease";
    case HSTU_ERR_CAPACITY: return "history exceeds max_len or cache capacity, or a bad cache slot";
    case HSTU_ERR_WORKSPACE: return "workspace missing or smaller than hstu_workspace_size()";
    case HSTU_ERR_HIP: return "a HIP runtime call failed";
    case HSTU_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    default: return "unknown status";
  }
}

hstu_status hstu_workspace_size(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                                const int32_t* cand_offsets, size_t* bytes) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  if (!bytes) return HSTU_ERR_NULL;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  *bytes = make_layout(d, B, uih_offsets, cand_offsets).total;
  return HSTU_OK;
}

hstu_status hstu_flops(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                       const int32_t* cand_offsets, const int32_t* cached_len,
                       uint64_t* algorithmic_flops, uint64_t* formula_flops) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  const uint64_t D = (uint64_t)d->d_model, L = (uint64_t)d->layers;
  uint64_t alg = 0, form = 0;
  for (int32_t b = 0; b < B; ++b) {
    const uint64_t n = (uint64_t)(uih_offsets[b + 1] - uih_offsets[b]);
    const uint64_t c = (uint64_t)(cand_offsets[b + 1] - cand_offsets[b]);
    int32_t mm = cached_len ? cached_len[b] : 0;
    if (mm < 0) return HSTU_ERR_CAPACITY;
    const uint64_t m = (uint64_t)mm;
    // masked (query, key) pairs: history row i sees m+i+1 keys, a candidate m+n keys + itself
    const uint64_t pairs = n * m + n * (n + 1) / 2 + c * (m + n + 1);
    alg += L * (14 * (n + c) * D * D + 4 * D * pairs);
    const uint64_t N = m + n;
    form += 2 * L * (N * N * D / 2 + N * D * D * 4 + N * D * D * 3);
  }
  if (algorithmic_flops) *algorithmic_flops = alg;
  if (formula_flops) *formula_flops = form;
  return HSTU_OK;
}

hstu_status hstu_encode(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                        const int32_t* cand_offsets, const void* uih, const void* cand,
                        const hstu_layer_weights* w, hstu_kv_cache* kv, void* uih_out,
                        void* cand_out, void* workspace, size_t workspace_bytes, void* stream) {
  // ------------------------------------------------------------ validation (host only)
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  if (!w) return HSTU_ERR_NULL;
  const Layout lay = make_layout(d, B, uih_offsets, cand_offsets);
  if (lay.T == 0) return HSTU_OK;  // nothing to encode; no history appended
  const int32_t L = d->layers, D = d->d_model;
  for (int32_t l = 0; l < L; ++l) {
    if (!w[l].w_uvqk || !w[l].w_out) return HSTU_ERR_NULL;
    if (!aligned16(w[l].w_uvqk) || !aligned16(w[l].w_out) || !aligned16(w[l].pos_bias) ||
        !aligned16(w[l].rel_bias))
      return HSTU_ERR_ALIGN;
    if (w[l].rel_bias && d->dtype == HSTU_BF16 && d->max_len > hstu::kRelMaxLen) return HSTU_ERR_SHAPE;
  }
  if ((lay.Nu > 0 && (!uih || !uih_out)) || (lay.Nc > 0 && (!cand || !cand_out))) return HSTU_ERR_NULL;
  if ((lay.Nu > 0 && (!aligned16(uih) || !aligned16(uih_out))) ||
      (lay.Nc > 0 && (!aligned16(cand) || !aligned16(cand_out))))
    return HSTU_ERR_ALIGN;
  if (kv) {
    if (!kv->k || !kv->v || !kv->slot_of_user || !kv->cached_len) return HSTU_ERR_NULL;
    if (!aligned16(kv->k) || !aligned16(kv->v)) return HSTU_ERR_ALIGN;
    if (kv->slots <= 0 || kv->capacity <= 0) return HSTU_ERR_CAPACITY;
  }
  std::vector<char> slot_used(kv ? (size_t)kv->slots : 0, 0);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = uih_offsets[b + 1] - uih_offsets[b];
    int64_t m = 0;
    if (kv) {
      m = kv->cached_len[b];
      const int32_t slot = kv->slot_of_user[b];
      if (m < 0 || slot < 0 || slot >= kv->slots || slot_used[slot]) return HSTU_ERR_CAPACITY;
      slot_used[slot] = 1;
      if (m + n > kv->capacity) return HSTU_ERR_CAPACITY;
    }
    if (m + n + 1 > d->max_len) return HSTU_ERR_CAPACITY;
    // the attention kernel addresses one user's key rows with 32-bit byte offsets
    if ((m + n) * (int64_t)(kv ? d->d_model : 3 * d->d_model) * (d->dtype == HSTU_F32 ? 4 : 2) > INT32_MAX)
      return HSTU_ERR_CAPACITY;
  }
  if (!workspace || workspace_bytes < lay.total) return HSTU_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return HSTU_ERR_ALIGN;

  // ------------------------------------------------------------ plan (host)
  const int bm = hstu::attn_block_rows(d->dtype);
  std::vector<char> staged(lay.staged, 0);
  UserRec* users = reinterpret_cast<UserRec*>(staged.data() + lay.users);
  for (int32_t b = 0; b < B; ++b) {
    UserRec& u = users[b];
    u.uoff = uih_offsets[b];
    u.n = uih_offsets[b + 1] - uih_offsets[b];
    u.coff = cand_offsets[b];
    u.c = cand_offsets[b + 1] - cand_offsets[b];
    u.m = kv ? kv->cached_len[b] : 0;
    u.key_row = kv ? kv->slot_of_user[b] * kv->capacity : u.uoff;
    u.pad0 = u.pad1 = 0;
  }
  // Attention work items, grouped per (user, head). Each group goes whole to one of
  // the kXcds bins (one bin per XCD), so a user's keys and values are read into one
  // L2 only; groups are placed largest first on the least loaded bin. The order never
  // changes any result: each item writes its own rows, with a fixed key order inside.
  struct Item { int32_t user, hk, q0, nq; int64_t cost; };
  struct Group { std::vector<Item> items; int64_t cost = 0; };
  std::vector<Group> groups;
  groups.reserve((size_t)B * d->heads);
  for (int32_t b = 0; b < B; ++b) {
    const UserRec& u = users[b];
    for (int32_t h = 0; h < d->heads; ++h) {
      Group g;
      // cost ~ key blocks swept, plus a fixed per-item overhead
      for (int32_t q0 = 0; q0 < u.n; q0 += bm) {
        const int32_t nq = std::min(bm, u.n - q0);
        g.items.push_back({b, h << 1, q0, nq, cdiv((int64_t)u.m + q0 + nq, 64) + 2});
      }
      for (int32_t q0 = 0; q0 < u.c; q0 += bm)
        g.items.push_back({b, (h << 1) | 1, q0, std::min(bm, u.c - q0), cdiv((int64_t)u.m + u.n, 64) + 2});
      if (g.items.empty()) continue;
      std::stable_sort(g.items.begin(), g.items.end(),
                       [](const Item& x, const Item& y) { return x.cost > y.cost; });
      for (const Item& it : g.items) g.cost += it.cost;
      groups.push_back(std::move(g));
    }
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group& x, const Group& y) { return x.cost > y.cost; });
  std::vector<std::vector<const Item*>> bin_items(hstu::kXcds);
  int64_t bin_cost[hstu::kXcds] = {};
  for (const Group& g : groups) {
    const int x = (int)(std::min_element(bin_cost, bin_cost + hstu::kXcds) - bin_cost);
    bin_cost[x] += g.cost;
    for (const Item& it : g.items) bin_items[x].push_back(&it);
  }
  // Inside a bin, items run longest first (workgroups take them in order as CUs free
  // up), so the bin ends on short items instead of one user's long tail.
  for (int x = 0; x < hstu::kXcds; ++x)
    std::stable_sort(bin_items[x].begin(), bin_items[x].end(),
                     [](const Item* p, const Item* q) { return p->cost > q->cost; });
  size_t longest = 0;
  for (int x = 0; x < hstu::kXcds; ++x) longest = std::max(longest, bin_items[x].size());
  const int attn_grid = hstu::kXcds * (int)longest;
  // workgroup w runs on XCD w % kXcds: it takes position w / kXcds of that XCD's bin
  // (nq = 0 past the bin's end)
  hstu::AttnItem* items = reinterpret_cast<hstu::AttnItem*>(staged.data() + lay.items);
  for (int w = 0; w < attn_grid; ++w) {
    const std::vector<const Item*>& bin = bin_items[w % hstu::kXcds];
    const size_t j = (size_t)(w / hstu::kXcds);
    hstu::AttnItem& a = items[w];
    a = hstu::AttnItem{0, 0, 0, 0, 0, 0, 0, 0};
    if (j >= bin.size()) continue;
    const Item& it = *bin[j];
    const UserRec& u = users[it.user];
    const bool is_cand = (it.hk & 1) != 0;
    a.hk = it.hk;
    a.q0 = it.q0;
    a.nq = it.nq;
    a.m = u.m;
    a.rbase = (is_cand ? lay.Nu + u.coff : u.uoff) + it.q0;
    a.key_end = is_cand ? u.m + u.n : u.m + it.q0 + it.nq;
    a.key_row = u.key_row;
  }
  const size_t staged_bytes = lay.items + (size_t)attn_grid * sizeof(hstu::AttnItem);
  const void** wptr = reinterpret_cast<const void**>(staged.data() + lay.wptr);
  for (int32_t l = 0; l < L; ++l) wptr[l] = w[l].w_uvqk;

  // ------------------------------------------------------------ enqueue
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  st = stage_and_copy(staged.data(), staged_bytes, ws, s);
  if (st != HSTU_OK) return st;
  const UserRec* d_users = reinterpret_cast<const UserRec*>(ws + lay.users);
  const hstu::AttnItem* d_items = reinterpret_cast<const hstu::AttnItem*>(ws + lay.items);
  int2* d_rows = reinterpret_cast<int2*>(ws + lay.rows);
  char* xn = ws + lay.xn;
  float* cs = reinterpret_cast<float*>(ws + lay.cs);
  float2* rstat = reinterpret_cast<float2*>(ws + lay.st);
  const size_t es = d->dtype == HSTU_F32 ? 4 : 2;
  char* vqk = ws + lay.vqk;
  char* aout = ws + lay.aout;
  char* xbuf = ws + lay.x;
  const size_t nu_bytes = (size_t)lay.Nu * D * es;

  hstu::PlanArgs pa{d_users, B, lay.Nu, lay.T, d_rows};
  if (timed_launch(HSTU_KERNEL_PLAN, s, [&] { return hstu::launch_plan(pa, s); }) != hipSuccess)
    return HSTU_ERR_HIP;

  if (d->dtype != HSTU_F32) {
    hstu::ColsumArgs ca{reinterpret_cast<const void* const*>(ws + lay.wptr), L, D, cs};
    if (timed_launch(HSTU_KERNEL_NORM, s, [&] { return hstu::launch_colsum(ca, s); }) != hipSuccess)
      return HSTU_ERR_HIP;
    if (timed_launch(HSTU_KERNEL_NORM, s,
                     [&] { return hstu::launch_rowstats(uih, cand, lay.Nu, lay.T, D, rstat, s); }) != hipSuccess)
      return HSTU_ERR_HIP;
  }

  const int dh = D / d->heads;
  const size_t layer_cache = kv ? (size_t)kv->slots * kv->capacity * D * es : 0;
  for (int32_t l = 0; l < L; ++l) {
    const void* x_lo = l == 0 ? uih : xbuf;
    const void* x_hi = l == 0 ? cand : (const void*)(xbuf + nu_bytes);
    void* y_lo = l == L - 1 ? uih_out : (void*)xbuf;
    void* y_hi = l == L - 1 ? cand_out : (void*)(xbuf + nu_bytes);
    void* ck = kv ? (void*)((char*)kv->k + l * layer_cache) : nullptr;
    void* cv = kv ? (void*)((char*)kv->v + l * layer_cache) : nullptr;

    if (d->dtype == HSTU_F32) {
      hstu::NormArgs na{x_lo, x_hi, lay.Nu, lay.T, D, xn};
      if (timed_launch(HSTU_KERNEL_NORM, s, [&] { return hstu::launch_norm(d->dtype, na, s); }) != hipSuccess)
        return HSTU_ERR_HIP;
    }
    hstu::UvqkArgs ua{xn, x_lo, x_hi, cs + (size_t)l * 4 * D, rstat, lay.Nu, lay.T, D, w[l].w_uvqk, w[l].pos_bias, d_rows, d_users,
                      vqk, aout, ck, cv};
    if (timed_launch(HSTU_KERNEL_UVQK, s, [&] { return hstu::launch_uvqk(d->dtype, ua, s); }) != hipSuccess)
      return HSTU_ERR_HIP;

    hstu::AttnArgs aa{};
    aa.items = d_items;
    aa.Nu = lay.Nu;
    aa.D = D;
    aa.inv = 1.0f / (float)d->max_len;
    aa.vqk = vqk;
    if (kv) {
      aa.kbase = ck;
      aa.vbase = cv;
      aa.ld = D;
    } else {
      aa.kbase = vqk + 2 * (size_t)D * es;
      aa.vbase = vqk;
      aa.ld = 3 * (int64_t)D;
    }
    aa.aout = aout;
    aa.rel = w[l].rel_bias;
    aa.max_len = d->max_len;
    if (timed_launch(HSTU_KERNEL_ATTENTION, s,
                     [&] { return hstu::launch_attn(d->dtype, dh, aa, attn_grid, s); }) != hipSuccess)
      return HSTU_ERR_HIP;

    // the output GEMM also leaves the next layer's row statistics (bfloat16 path)
    hstu::OutArgs oa{aout, w[l].w_out, x_lo, x_hi, y_lo, y_hi,
                     d->dtype == HSTU_F32 || l == L - 1 ? nullptr : rstat, lay.Nu, lay.T, D};
    if (timed_launch(HSTU_KERNEL_OUT, s, [&] { return hstu::launch_out(d->dtype, oa, s); }) != hipSuccess)
      return HSTU_ERR_HIP;
  }
  if (kv)
    for (int32_t b = 0; b < B; ++b) kv->cached_len[b] += uih_offsets[b + 1] - uih_offsets[b];
  return HSTU_OK;
}

hstu_status hstu_pack_uih(const hstu_dims* d, int32_t events, int32_t mode, const void* context,
                          const void* action, void* uih, void* stream) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  if (events < 0 || (mode != HSTU_PACK_SUM && mode != HSTU_PACK_INTERLEAVE)) return HSTU_ERR_SHAPE;
  const int64_t esize = d->dtype == HSTU_BF16 ? 2 : 4;
  const int64_t cpr = d->d_model * esize / 16;   // D is a multiple of 64, so rows are whole chunks
  const int64_t rows = mode == HSTU_PACK_INTERLEAVE ? 2 * (int64_t)events : events;
  if (rows * cpr >= ((int64_t)1 << 31)) return HSTU_ERR_SHAPE;
  if (events == 0) return HSTU_OK;
  if (!context || !action || !uih) return HSTU_ERR_NULL;
  if (!aligned16(context) || !aligned16(action) || !aligned16(uih)) return HSTU_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const hstu::PackArgs pa{context, action, uih, (int32_t)(rows * cpr), (int32_t)cpr,
                          mode == HSTU_PACK_INTERLEAVE, d->dtype == HSTU_BF16};
  if (timed_launch(HSTU_KERNEL_PACK, s, [&] { return hstu::launch_pack(pa, s); }) != hipSuccess)
    return HSTU_ERR_HIP;
  return HSTU_OK;
}

hstu_status hstu_score(const hstu_dims* d, int32_t rows, const void* x, const hstu_head_layer* head,
                       int32_t head_layers, float* prob, void* stream) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  if (!head) return HSTU_ERR_NULL;
  if (head_layers < 1 || head_layers > hstu::kMaxHeadLayers || rows < 0) return HSTU_ERR_SHAPE;
  if (d->d_model > hstu::kMaxHeadWidth) return HSTU_ERR_SHAPE;
  for (int32_t l = 0; l + 1 < head_layers; ++l) {
    const int32_t n = head[l].out_features;
    if (n < 128 || n > hstu::kMaxHeadWidth || n % 128) return HSTU_ERR_SHAPE;
  }
  const int32_t outcomes = head[head_layers - 1].out_features;
  if (outcomes < 1 || outcomes > hstu::kMaxOutcomes) return HSTU_ERR_SHAPE;
  if (rows == 0) return HSTU_OK;
  if (!x || !prob) return HSTU_ERR_NULL;
  for (int32_t l = 0; l < head_layers; ++l)
    if (!head[l].weight || !head[l].bias) return HSTU_ERR_NULL;
  if (!aligned16(x) || !aligned16(prob)) return HSTU_ERR_ALIGN;
  for (int32_t l = 0; l < head_layers; ++l)
    if (!aligned16(head[l].weight) || !aligned16(head[l].bias)) return HSTU_ERR_ALIGN;
  hstu::ScoreArgs sa{};
  sa.x = x;
  sa.prob = prob;
  sa.rows = rows;
  sa.D = d->d_model;
  sa.layers = head_layers;
  sa.outcomes = outcomes;
  for (int32_t l = 0; l < head_layers; ++l) {
    sa.w[l] = head[l].weight;
    sa.b[l] = head[l].bias;
    sa.width[l] = head[l].out_features;
  }
  hipStream_t s = (hipStream_t)stream;
  if (timed_launch(HSTU_KERNEL_SCORE, s, [&] { return hstu::launch_score(d->dtype, sa, s); }) != hipSuccess)
    return HSTU_ERR_HIP;
  return HSTU_OK;
}

}  // extern "C"
