// Host side of the C ABI declared in include/hstu.h: argument validation, the
// jagged work planner, the plan's transfer to the device and the per-layer launch
// sequence.
//
// Validation is complete before anything is enqueued, so every error except
// HSTU_ERR_HIP leaves the device and every host array untouched. The planner works
// in host memory its caller provides and the plan reaches the device inside kernel
// arguments, so a call allocates no device or pinned memory and never waits for the
// device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <numeric>
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
  if (d->heads > 127) return HSTU_ERR_SHAPE;   // the planner's item codes hold a head in 7 bits
  if (d->weight_layout != HSTU_WEIGHTS_PREPARED && d->weight_layout != HSTU_WEIGHTS_MATH) return HSTU_ERR_SHAPE;
  if (d->d_model % d->heads) return HSTU_ERR_SHAPE;
  // a position table holds fewer than 2^31 elements (the kernels index it in 32 bits)
  if ((int64_t)d->max_len * 3 * d->d_model >= ((int64_t)1 << 31)) return HSTU_ERR_SHAPE;
  const int dh = d->d_model / d->heads;
  if (d->dtype == HSTU_F32) {
    if (d->d_model % 64 || (dh != 32 && dh != 64 && dh != 128)) return HSTU_ERR_SHAPE;
  } else if (d->dtype == HSTU_BF16) {
    if (d->d_model % 128 || (dh != 32 && dh != 64 && dh != 128)) return HSTU_ERR_SHAPE;
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
  int32_t B = 0, Nu = 0, Nc = 0, T = 0;
  int64_t ntiles = 0, groups = 0;
  size_t users = 0, wptr = 0, codes = 0, items = 0, rows = 0, xn = 0, cs = 0, st = 0, vqk = 0, aout = 0, x = 0,
         wt = 0, relf = 0, total = 0;
  size_t staged = 0;  // host-planned part: users table, W1 pointers, item codes (sent up to the grid)
};

Layout make_layout(const hstu_dims* d, int32_t B, const int32_t* uo, const int32_t* co) {
  Layout L;
  L.B = B;
  if (B > 0) {
    L.Nu = uo[B];
    L.Nc = co[B];
  }
  L.T = L.Nu + L.Nc;
  const int bm = hstu::attn_block_rows(d->dtype);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t per_head = cdiv(uo[b + 1] - uo[b], bm) + cdiv(co[b + 1] - co[b], bm);
    L.ntiles += d->heads * per_head;
    L.groups += per_head > 0 ? d->heads : 0;
  }
  const size_t es = d->dtype == HSTU_F32 ? 4 : 2;
  const size_t D = (size_t)d->d_model, T = (size_t)L.T;
  // GEMM operands (xn, vqk, aout) are padded to whole 256-row tiles.
  const size_t Tp = (size_t)cdiv(L.T, hstu::kRowPad) * hstu::kRowPad;
  size_t off = 0;
  L.users = off; off += align_up((size_t)B * sizeof(UserRec));
  L.wptr = off; off += align_up((size_t)d->layers * sizeof(void*));
  // one item per attention workgroup: kXcds bins of at most ntiles items each
  L.codes = off; off += align_up((size_t)hstu::kXcds * L.ntiles * sizeof(hstu::ItemCode));
  L.staged = off;
  L.items = off; off += align_up((size_t)hstu::kXcds * L.ntiles * sizeof(hstu::AttnItem));
  L.rows = off; off += align_up(T * 8);
  // float32 models normalise into xn; bfloat16 models normalise inside the projection
  // and need the column sums of W1 instead
  L.xn = off; off += d->dtype == HSTU_F32 ? align_up(Tp * D * es) : 0;
  L.cs = off; off += d->dtype == HSTU_F32 ? 0 : align_up((size_t)d->layers * 4 * D * sizeof(float));
  L.st = off; off += d->dtype == HSTU_F32 ? 0 : align_up(T * (D / 128) * 2 * sizeof(float));
  L.vqk = off; off += align_up(Tp * 3 * D * es);
  L.aout = off; off += align_up(Tp * 3 * D * es);
  L.x = off; off += d->layers > 1 ? align_up(T * D * es) : 0;
  // weights given in the math layout: each layer's W1 [D][4D] and W2 [3D][D], transposed
  // into [4D][D] and [D][3D] at the start of the call
  L.wt = off; off += d->weight_layout == HSTU_WEIGHTS_MATH ? align_up((size_t)d->layers * 7 * D * D * es) : 0;
  // bfloat16 models: the current layer's relative table widened to float32 (the attention
  // adds its entries to float32 weights; reused by every layer)
  L.relf = off; off += d->dtype == HSTU_F32 ? 0 : align_up((size_t)d->heads * d->max_len * sizeof(float));
  L.total = L.T == 0 ? 0 : off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// ---------------------------------------------------------------- attention planner
// Attention work items, grouped per (user, head). Each group goes whole to one of the
// kXcds bins (one bin per XCD), so a user's keys and values are read into one L2 only;
// groups are placed largest first on the least loaded bin. Inside a bin the items run
// longest first (workgroups take them in order as CUs free up), so the bin ends on
// short items instead of one user's long tail. The order never changes any result:
// each item writes its own rows, with a fixed key order inside.
//
// The planner allocates nothing: its caller provides the group and item records. Every
// sort key is a total order (ties broken by a sequence number), so std::sort gives the
// same order on every call.
struct PlanItem {
  int64_t cost;           // key blocks swept, plus a fixed per-item overhead (below)
  int32_t user, code;     // code as in hstu::ItemCode
  int32_t seq, bin;       // push order inside the group, then append order inside the bin
};
struct PlanGroup {
  int64_t cost;
  int32_t first, count;   // its items
  int32_t index, pad;
};

// Fills codes[0, grid) and returns grid, the attention's workgroup count: workgroup w
// runs on XCD w % kXcds and takes position w / kXcds of that XCD's bin (user -1 past
// the bin's end).
// An item's cost is in key blocks: the blocks it sweeps, plus its fixed work (Q and first
// K/V loads, the diagonal pass of a history item, a candidate's own key, the stores)
// as measured on MI355X at dh = 128: about 13 blocks' time for a history item and 22
// for a candidate item.
constexpr int64_t kHistoryItemFixed = 13, kCandidateItemFixed = 22;

int plan_attention(const UserRec* users, int32_t B, int32_t heads, int bm, PlanGroup* groups, PlanItem* items,
                   hstu::ItemCode* codes) {
  int32_t G = 0, N = 0;
  for (int32_t b = 0; b < B; ++b) {
    const UserRec& u = users[b];
    for (int32_t h = 0; h < heads; ++h) {
      const int32_t first = N;
      for (int32_t q0 = 0; q0 < u.n; q0 += bm) {
        const int32_t nq = std::min(bm, u.n - q0);
        items[N] = {cdiv((int64_t)u.m + q0 + nq, 64) + kHistoryItemFixed, b, ((q0 / bm) << 8) | (h << 1), N - first, -1};
        ++N;
      }
      for (int32_t q0 = 0; q0 < u.c; q0 += bm) {
        items[N] = {cdiv((int64_t)u.m + u.n, 64) + kCandidateItemFixed, b, ((q0 / bm) << 8) | (h << 1) | 1, N - first, -1};
        ++N;
      }
      if (N == first) continue;
      // the group's items, longest first (ties in push order)
      std::sort(items + first, items + N, [](const PlanItem& x, const PlanItem& y) {
        return x.cost != y.cost ? x.cost > y.cost : x.seq < y.seq;
      });
      int64_t cost = 0;
      for (int32_t i = first; i < N; ++i) cost += items[i].cost;
      groups[G] = {cost, first, N - first, G, 0};
      ++G;
    }
  }
  std::sort(groups, groups + G, [](const PlanGroup& x, const PlanGroup& y) {
    return x.cost != y.cost ? x.cost > y.cost : x.index < y.index;
  });
  int64_t bin_cost[hstu::kXcds] = {};
  int32_t bin_n[hstu::kXcds] = {};
  for (int32_t g = 0; g < G; ++g) {
    const int x = (int)(std::min_element(bin_cost, bin_cost + hstu::kXcds) - bin_cost);
    bin_cost[x] += groups[g].cost;
    for (int32_t i = groups[g].first; i < groups[g].first + groups[g].count; ++i) {
      items[i].bin = x;
      items[i].seq = bin_n[x]++;
    }
  }
  std::sort(items, items + N, [](const PlanItem& x, const PlanItem& y) {
    if (x.bin != y.bin) return x.bin < y.bin;
    return x.cost != y.cost ? x.cost > y.cost : x.seq < y.seq;
  });
  int32_t start[hstu::kXcds] = {}, longest = 0;
  for (int x = 0, acc = 0; x < hstu::kXcds; ++x) {
    start[x] = acc;
    acc += bin_n[x];
    longest = std::max(longest, bin_n[x]);
  }
  const int grid = hstu::kXcds * longest;
  for (int w = 0; w < grid; ++w) {
    const int x = w % hstu::kXcds, j = w / hstu::kXcds;
    codes[w] = j < bin_n[x] ? hstu::ItemCode{items[start[x] + j].user, items[start[x] + j].code}
                            : hstu::ItemCode{-1, 0};
  }
  return grid;
}

// Host memory the planner of one call works in.
struct PlanSpace {
  PlanGroup* groups = nullptr;
  PlanItem* items = nullptr;
  unsigned char* image = nullptr;   // the upload image: users | W1 pointers | item codes
  int32_t* keys = nullptr;          // validation scratch: one entry per user
};

// The calling thread's planner memory for a layout, grown when a larger plan comes
// (host memory only; steady-state calls of one shape reuse it).
PlanSpace thread_plan_space(const Layout& lay) {
  thread_local std::vector<PlanGroup> groups;
  thread_local std::vector<PlanItem> items;
  thread_local std::vector<unsigned char> image;
  thread_local std::vector<int32_t> keys;
  if (groups.size() < (size_t)lay.groups) groups.resize((size_t)lay.groups);
  if (items.size() < (size_t)lay.ntiles) items.resize((size_t)lay.ntiles);
  if (image.size() < lay.staged) image.resize(lay.staged);
  if (keys.size() < (size_t)lay.B) keys.resize((size_t)lay.B);
  return PlanSpace{groups.data(), items.data(), image.data(), keys.data()};
}

// Copies `bytes` (a multiple of 4) from host memory to device memory dst on `stream`
// inside the arguments of upload kernels.
hipError_t upload(const unsigned char* src, size_t bytes, char* dst, hipStream_t stream) {
  constexpr size_t kChunk = sizeof(uint32_t) * hstu::kUploadWords;
  for (size_t off = 0; off < bytes; off += kChunk) {
    hstu::UploadArgs ua;
    ua.dst = reinterpret_cast<uint32_t*>(dst + off);
    ua.words = (int32_t)(std::min(kChunk, bytes - off) / sizeof(uint32_t));
    ua.pad = 0;
    std::memcpy(ua.w, src + off, (size_t)ua.words * sizeof(uint32_t));
    const hipError_t e = hstu::launch_upload(ua, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

// ---------------------------------------------------------------- hstu_encode's steps
struct EncodeCall {
  const hstu_dims* d;
  int32_t B;
  const int32_t* uo;
  const int32_t* co;
  const void* uih;
  const void* cand;
  const hstu_layer_weights* w;
  hstu_kv_cache* kv;
  void* uih_out;
  void* cand_out;
  Layout lay;
};

// Every argument but the workspace (host only; nothing is enqueued, nothing written
// but `keys`, int32 scratch of at least B entries). c.lay must be make_layout's.
hstu_status validate_encode(EncodeCall& c, int32_t* keys) {
  const hstu_dims* d = c.d;
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  st = check_offsets(c.B, c.uo, c.co);
  if (st != HSTU_OK) return st;
  if (!c.w) return HSTU_ERR_NULL;
  if (c.lay.T == 0) return HSTU_OK;
  for (int32_t l = 0; l < d->layers; ++l) {
    const hstu_layer_weights& w = c.w[l];
    if (!w.w_uvqk || !w.w_out) return HSTU_ERR_NULL;
    if (!aligned16(w.w_uvqk) || !aligned16(w.w_out) || !aligned16(w.pos_bias) || !aligned16(w.rel_bias))
      return HSTU_ERR_ALIGN;
  }
  const Layout& lay = c.lay;
  if ((lay.Nu > 0 && (!c.uih || !c.uih_out)) || (lay.Nc > 0 && (!c.cand || !c.cand_out))) return HSTU_ERR_NULL;
  if ((lay.Nu > 0 && (!aligned16(c.uih) || !aligned16(c.uih_out))) ||
      (lay.Nc > 0 && (!aligned16(c.cand) || !aligned16(c.cand_out))))
    return HSTU_ERR_ALIGN;
  const hstu_kv_cache* kv = c.kv;
  const int64_t es = d->dtype == HSTU_F32 ? 4 : 2;
  const bool paged = kv && kv->page_rows != 0;
  if (kv) {
    if (!kv->k || !kv->v || !kv->cached_len) return HSTU_ERR_NULL;
    if (!aligned16(kv->k) || !aligned16(kv->v)) return HSTU_ERR_ALIGN;
    if (!paged) {
      if (!kv->slot_of_user) return HSTU_ERR_NULL;
      if (kv->slots <= 0 || kv->capacity <= 0) return HSTU_ERR_CAPACITY;
    } else {
      if (kv->page_rows != hstu::kPageRows || kv->pages <= 0 || kv->pages_per_user <= 0) return HSTU_ERR_CAPACITY;
      if (!kv->page_table) return HSTU_ERR_NULL;
      if (((uintptr_t)kv->page_table & 3) != 0) return HSTU_ERR_ALIGN;
      // the kernels address a layer's pool with 32-bit byte offsets and the page table
      // with 32-bit indices
      if ((int64_t)kv->pages * hstu::kPageRows * d->d_model * es > INT32_MAX) return HSTU_ERR_CAPACITY;
      if ((int64_t)c.B * kv->pages_per_user > INT32_MAX) return HSTU_ERR_CAPACITY;
    }
  }
  for (int32_t b = 0; b < c.B; ++b) {
    const int64_t n = c.uo[b + 1] - c.uo[b];
    // the planner's item codes hold a query block index in 23 bits
    if (n >= ((int64_t)1 << 30) || c.co[b + 1] - c.co[b] >= ((int64_t)1 << 30)) return HSTU_ERR_SHAPE;
    int64_t m = 0;
    if (kv) {
      m = kv->cached_len[b];
      if (m < 0) return HSTU_ERR_CAPACITY;
      if (paged) {
        if ((m + n + hstu::kPageRows - 1) / hstu::kPageRows > kv->pages_per_user) return HSTU_ERR_CAPACITY;
      } else {
        const int32_t slot = kv->slot_of_user[b];
        if (slot < 0 || slot >= kv->slots) return HSTU_ERR_CAPACITY;
        if (m + n > kv->capacity) return HSTU_ERR_CAPACITY;
      }
    }
    if (m + n + 1 > d->max_len) return HSTU_ERR_CAPACITY;
    // the attention kernel addresses one user's key rows with 32-bit byte offsets
    if (!paged && (m + n) * (int64_t)(kv ? d->d_model : 3 * d->d_model) * es > INT32_MAX) return HSTU_ERR_CAPACITY;
  }
  // distinct slots: no two users of the call may write the same cache rows
  if (kv && !paged && c.B > 1) {
    std::copy(kv->slot_of_user, kv->slot_of_user + c.B, keys);
    std::sort(keys, keys + c.B);
    if (std::adjacent_find(keys, keys + c.B) != keys + c.B) return HSTU_ERR_CAPACITY;
  }
  return HSTU_OK;
}

// Plans the call in `ps` and enqueues it on stream s with workspace ws (a validated call
// with T > 0 and a workspace of c.lay.total bytes). With `timed` false the timing aid is
// bypassed (it creates events while it is on).
hstu_status run_encode(const EncodeCall& c, const PlanSpace& ps, char* ws, hipStream_t s, bool timed = true) {
  auto timed_launch = [timed](int kind, hipStream_t st, auto&& f) -> hipError_t {
    return timed ? ::timed_launch(kind, st, f) : f();
  };
  const hstu_dims* d = c.d;
  const Layout& lay = c.lay;
  const hstu_kv_cache* kv = c.kv;
  const int32_t B = c.B, L = d->layers, D = d->d_model;
  const bool paged = kv && kv->page_rows != 0;
  const int32_t* pages = paged ? kv->page_table : nullptr;
  const int32_t npages = paged ? kv->pages : 0;

  // ------------------------------------------------------------ plan (host)
  const int bm = hstu::attn_block_rows(d->dtype);
  std::memset(ps.image, 0, lay.codes);
  UserRec* users = reinterpret_cast<UserRec*>(ps.image + lay.users);
  for (int32_t b = 0; b < B; ++b) {
    UserRec& u = users[b];
    u.uoff = c.uo[b];
    u.n = c.uo[b + 1] - c.uo[b];
    u.coff = c.co[b];
    u.c = c.co[b + 1] - c.co[b];
    u.m = kv ? kv->cached_len[b] : 0;
    u.key_row = !kv ? u.uoff : paged ? b * kv->pages_per_user : kv->slot_of_user[b] * kv->capacity;
    u.pad0 = u.pad1 = 0;
  }
  // the layers' W1 [4D][D] and W2 [D][3D] as the GEMMs read them: the caller's, or their
  // transposes in the workspace (math layout)
  const size_t esz = d->dtype == HSTU_F32 ? 4 : 2;
  const bool math = d->weight_layout == HSTU_WEIGHTS_MATH;
  auto w1 = [&](int32_t l) -> const void* {
    return math ? ws + lay.wt + (size_t)l * 7 * D * D * esz : c.w[l].w_uvqk;
  };
  auto w2 = [&](int32_t l) -> const void* {
    return math ? ws + lay.wt + ((size_t)l * 7 + 4) * D * D * esz : c.w[l].w_out;
  };
  const void** wptr = reinterpret_cast<const void**>(ps.image + lay.wptr);
  for (int32_t l = 0; l < L; ++l) wptr[l] = w1(l);
  hstu::ItemCode* codes = reinterpret_cast<hstu::ItemCode*>(ps.image + lay.codes);
  const int attn_grid = plan_attention(users, B, d->heads, bm, ps.groups, ps.items, codes);

  // ------------------------------------------------------------ enqueue
  if (timed_launch(HSTU_KERNEL_PLAN, s, [&] {
        return upload(ps.image, lay.codes + (size_t)attn_grid * sizeof(hstu::ItemCode), ws, s);
      }) != hipSuccess)
    return HSTU_ERR_HIP;
  const UserRec* d_users = reinterpret_cast<const UserRec*>(ws + lay.users);
  hstu::AttnItem* d_items = reinterpret_cast<hstu::AttnItem*>(ws + lay.items);
  int2* d_rows = reinterpret_cast<int2*>(ws + lay.rows);
  char* xn = ws + lay.xn;
  float* cs = reinterpret_cast<float*>(ws + lay.cs);
  float2* rstat = reinterpret_cast<float2*>(ws + lay.st);
  const size_t es = d->dtype == HSTU_F32 ? 4 : 2;
  char* vqk = ws + lay.vqk;
  char* aout = ws + lay.aout;
  char* xbuf = ws + lay.x;
  const size_t nu_bytes = (size_t)lay.Nu * D * es;

  hstu::PlanArgs pa{d_users, B, lay.Nu, lay.T, d_rows,
                    reinterpret_cast<const hstu::ItemCode*>(ws + lay.codes), d_items, attn_grid, bm};
  if (timed_launch(HSTU_KERNEL_PLAN, s, [&] { return hstu::launch_plan(pa, s); }) != hipSuccess)
    return HSTU_ERR_HIP;

  // math layout: every layer's W1 [D][4D] and W2 [3D][D] transposed into the workspace,
  // up to kTransposeList layers a launch
  for (int32_t l0 = 0; math && l0 < L; l0 += hstu::kTransposeList) {
    hstu::TransposeList t1{}, t2{};
    t1.count = t2.count = std::min(L - l0, hstu::kTransposeList);
    t1.rows = D, t1.cols = 4 * D;
    t2.rows = 3 * D, t2.cols = D;
    for (int32_t i = 0; i < t1.count; ++i) {
      t1.src[i] = c.w[l0 + i].w_uvqk;
      t1.dst[i] = const_cast<void*>(w1(l0 + i));
      t2.src[i] = c.w[l0 + i].w_out;
      t2.dst[i] = const_cast<void*>(w2(l0 + i));
    }
    if (timed_launch(HSTU_KERNEL_NORM, s, [&] {
          const hipError_t e = hstu::launch_transpose_list((int)esz, t1, s);
          return e != hipSuccess ? e : hstu::launch_transpose_list((int)esz, t2, s);
        }) != hipSuccess)
      return HSTU_ERR_HIP;
  }
  if (d->dtype != HSTU_F32) {
    hstu::ColsumArgs ca{reinterpret_cast<const void* const*>(ws + lay.wptr), L, D, cs};
    if (timed_launch(HSTU_KERNEL_NORM, s, [&] { return hstu::launch_colsum(ca, s); }) != hipSuccess)
      return HSTU_ERR_HIP;
    if (timed_launch(HSTU_KERNEL_NORM, s,
                     [&] { return hstu::launch_rowstats(c.uih, c.cand, lay.Nu, lay.T, D, rstat, s); }) != hipSuccess)
      return HSTU_ERR_HIP;
  }

  const int dh = D / d->heads;
  const size_t layer_cache = !kv ? 0 : paged ? (size_t)kv->pages * hstu::kPageRows * D * es
                                            : (size_t)kv->slots * kv->capacity * D * es;
  for (int32_t l = 0; l < L; ++l) {
    const void* x_lo = l == 0 ? c.uih : xbuf;
    const void* x_hi = l == 0 ? c.cand : (const void*)(xbuf + nu_bytes);
    void* y_lo = l == L - 1 ? c.uih_out : (void*)xbuf;
    void* y_hi = l == L - 1 ? c.cand_out : (void*)(xbuf + nu_bytes);
    void* ck = kv ? (void*)((char*)kv->k + l * layer_cache) : nullptr;
    void* cv = kv ? (void*)((char*)kv->v + l * layer_cache) : nullptr;

    if (d->dtype == HSTU_F32) {
      hstu::NormArgs na{x_lo, x_hi, lay.Nu, lay.T, D, xn};
      if (timed_launch(HSTU_KERNEL_NORM, s, [&] { return hstu::launch_norm(d->dtype, na, s); }) != hipSuccess)
        return HSTU_ERR_HIP;
    }
    hstu::UvqkArgs ua{xn, x_lo, x_hi, cs + (size_t)l * 4 * D, rstat, lay.Nu, lay.T, D, w1(l),
                      c.w[l].pos_bias, d_rows, d_users, vqk, aout, ck, cv, pages, npages};
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
    aa.pages = pages;
    aa.npages = npages;
    aa.aout = aout;
    aa.rel = c.w[l].rel_bias;
    if (aa.rel && d->dtype != HSTU_F32) {
      float* relf = reinterpret_cast<float*>(ws + lay.relf);
      if (timed_launch(HSTU_KERNEL_NORM, s, [&] {
            return hstu::launch_widen_bf16(c.w[l].rel_bias, relf, (int64_t)d->heads * d->max_len, s);
          }) != hipSuccess)
        return HSTU_ERR_HIP;
      aa.rel = relf;
    }
    aa.max_len = d->max_len;
    if (timed_launch(HSTU_KERNEL_ATTENTION, s,
                     [&] { return hstu::launch_attn(d->dtype, dh, aa, attn_grid, s); }) != hipSuccess)
      return HSTU_ERR_HIP;

    // the output GEMM also leaves the next layer's row statistics (bfloat16 path)
    hstu::OutArgs oa{aout, w2(l), x_lo, x_hi, y_lo, y_hi,
                     d->dtype == HSTU_F32 || l == L - 1 ? nullptr : rstat, lay.Nu, lay.T, D};
    if (timed_launch(HSTU_KERNEL_OUT, s, [&] { return hstu::launch_out(d->dtype, oa, s); }) != hipSuccess)
      return HSTU_ERR_HIP;
  }
  if (kv)
    for (int32_t b = 0; b < B; ++b) kv->cached_len[b] += c.uo[b + 1] - c.uo[b];
  return HSTU_OK;
}

// ---------------------------------------------------------------- no-allocation entry point
// hstu_encode_static: hstu_encode with the workspace in a fixed device array and the
// planner in fixed host arrays, for callers that cannot allocate. The array is a
// file-scope device variable: each GPU that runs the entry point holds its own copy
// until the process ends. Its device address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current; host code uses
// only that address (the variable's name in host code is a host-side stand-in).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
constexpr int32_t kStaticMaxUsers = 1024;
constexpr int64_t kStaticMaxItems = 16384;       // attention work items (and so groups)
constexpr size_t kStaticImageBytes = 256 * 1024 + (size_t)hstu::kXcds * kStaticMaxItems * sizeof(hstu::ItemCode);
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_static_mu;                          // the host arrays below and g_scratch_ptr
void* g_scratch_ptr[kMaxDevices] = {};
PlanGroup g_static_groups[kStaticMaxItems];
PlanItem g_static_items[kStaticMaxItems];
alignas(256) unsigned char g_static_image[kStaticImageBytes];
int32_t g_static_keys[kStaticMaxUsers];

// The current device's copy of `scratch` (looked up on the device's first call).
hstu_status static_scratch(char** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HSTU_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HSTU_ERR_HIP;
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HSTU_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = static_cast<char*>(g_scratch_ptr[dev]);
  return HSTU_OK;
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
    case HSTU_ERR_TOO_LARGE: return "batch too large for hstu_encode_static's fixed scratch (use hstu_encode)";
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

hstu_status hstu_attention_plan(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                                const int32_t* cand_offsets, const int32_t* cached_len, int32_t* grid,
                                int64_t* codes, int64_t capacity) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  if (!grid) return HSTU_ERR_NULL;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  const Layout lay = make_layout(d, B, uih_offsets, cand_offsets);
  std::vector<UserRec> users((size_t)B);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t m = cached_len ? cached_len[b] : 0;
    if (m < 0) return HSTU_ERR_CAPACITY;
    users[b] = UserRec{uih_offsets[b], uih_offsets[b + 1] - uih_offsets[b], cand_offsets[b],
                       cand_offsets[b + 1] - cand_offsets[b], m, 0, 0, 0};
  }
  std::vector<PlanGroup> groups((size_t)lay.groups);
  std::vector<PlanItem> items((size_t)lay.ntiles);
  std::vector<hstu::ItemCode> out((size_t)hstu::kXcds * lay.ntiles);
  const int g = plan_attention(users.data(), B, d->heads, hstu::attn_block_rows(d->dtype), groups.data(),
                               items.data(), out.data());
  *grid = g;
  if (!codes) return HSTU_OK;
  if (capacity < g) return HSTU_ERR_WORKSPACE;
  for (int w = 0; w < g; ++w)
    codes[w] = out[w].user < 0 ? -1 : ((int64_t)out[w].user << 32) | (uint32_t)out[w].code;
  return HSTU_OK;
}

hstu_status hstu_flops(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                       const int32_t* cand_offsets, const int32_t* cached_len,
                       uint64_t* algorithmic_flops, uint64_t* formula_flops) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  // 128-bit sums: with n, c, m < 2^31, D < 2^14 (at most 127 heads of 128) and layers
  // < 2^31, each user adds under 2^112, so a running total checked after every user
  // cannot wrap
  typedef unsigned __int128 u128;
  const u128 D = (u128)d->d_model, L = (u128)d->layers, lim = (u128)UINT64_MAX;
  u128 alg = 0, form = 0;
  for (int32_t b = 0; b < B; ++b) {
    const u128 n = (u128)(uih_offsets[b + 1] - uih_offsets[b]);
    const u128 c = (u128)(cand_offsets[b + 1] - cand_offsets[b]);
    const int32_t mm = cached_len ? cached_len[b] : 0;
    if (mm < 0) return HSTU_ERR_CAPACITY;
    const u128 m = (u128)mm;
    // masked (query, key) pairs: history row i sees m+i+1 keys, a candidate m+n keys + itself
    const u128 pairs = n * m + n * (n + 1) / 2 + c * (m + n + 1);
    alg += L * (14 * (n + c) * D * D + 4 * D * pairs);
    const u128 N = m + n;
    form += 2 * L * (N * N * D / 2 + N * D * D * 4 + N * D * D * 3);
    if (alg > lim || form > lim) return HSTU_ERR_SHAPE;
  }
  if (algorithmic_flops) *algorithmic_flops = (uint64_t)alg;
  if (formula_flops) *formula_flops = (uint64_t)form;
  return HSTU_OK;
}

hstu_status hstu_encode(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                        const int32_t* cand_offsets, const void* uih, const void* cand,
                        const hstu_layer_weights* w, hstu_kv_cache* kv, void* uih_out,
                        void* cand_out, void* workspace, size_t workspace_bytes, void* stream) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  EncodeCall c{d, B, uih_offsets, cand_offsets, uih, cand, w, kv, uih_out, cand_out,
               make_layout(d, B, uih_offsets, cand_offsets)};
  const PlanSpace ps = thread_plan_space(c.lay);
  st = validate_encode(c, ps.keys);
  if (st != HSTU_OK || c.lay.T == 0) return st;   // T = 0: nothing to encode, no history appended
  if (!workspace || workspace_bytes < c.lay.total) return HSTU_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return HSTU_ERR_ALIGN;
  return run_encode(c, ps, static_cast<char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

hstu_status hstu_encode_static(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                               const int32_t* cand_offsets, const void* uih, const void* cand,
                               const hstu_layer_weights* w, hstu_kv_cache* kv, void* uih_out, void* cand_out,
                               void* stream) {
  hstu_status st = check_dims(d);
  if (st != HSTU_OK) return st;
  st = check_offsets(B, uih_offsets, cand_offsets);
  if (st != HSTU_OK) return st;
  EncodeCall c{d, B, uih_offsets, cand_offsets, uih, cand, w, kv, uih_out, cand_out,
               make_layout(d, B, uih_offsets, cand_offsets)};
  if (B > kStaticMaxUsers || c.lay.ntiles > kStaticMaxItems || c.lay.staged > kStaticImageBytes ||
      c.lay.total > kStaticScratchBytes)
    return HSTU_ERR_TOO_LARGE;
  std::lock_guard<std::mutex> lock(g_static_mu);
  st = validate_encode(c, g_static_keys);
  if (st != HSTU_OK || c.lay.T == 0) return st;
  char* ws = nullptr;
  st = static_scratch(&ws);
  if (st != HSTU_OK) return st;
  return run_encode(c, PlanSpace{g_static_groups, g_static_items, g_static_image, g_static_keys}, ws,
                    reinterpret_cast<hipStream_t>(stream), false);
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

hstu_status hstu_transpose_weights(int32_t dtype, int32_t rows, int32_t cols, const void* src, void* dst,
                                   void* stream) {
  if (dtype != HSTU_F32 && dtype != HSTU_BF16) return HSTU_ERR_SHAPE;
  if (rows < 0 || cols < 0 || (int64_t)rows * cols >= ((int64_t)1 << 31)) return HSTU_ERR_SHAPE;
  if ((int64_t)rows * cols == 0) return HSTU_OK;
  if (!src || !dst) return HSTU_ERR_NULL;
  const size_t esize = dtype == HSTU_BF16 ? 2 : 4;
  if ((uintptr_t)src % esize || (uintptr_t)dst % esize) return HSTU_ERR_ALIGN;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst, n = (uintptr_t)rows * cols * esize;
  if (s0 < d0 + n && d0 < s0 + n) return HSTU_ERR_SHAPE;   // the two matrices overlap
  if (hstu::launch_transpose((int)esize, src, dst, rows, cols, (hipStream_t)stream) != hipSuccess)
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
