// Jagged target-aware causal SiLU attention on gfx950 (bf16 MFMA 32x32x16, float32
// accumulation). Scores never pass through a softmax: each history row sums
// SiLU(q.k) v over the keys at or before its position, each candidate over every
// history key plus itself, and the 1/max_len scale is applied once at the end.
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// One work item = (user, head, up to 128 query rows of one kind): four waves of QB
// blocks of 32 query rows each; two work items share a CU, so every SIMD runs two
// independent waves that hide each other's stalls.
//
// Keys advance 64 at a time (a "block"). K and V blocks go from global memory straight
// into LDS (buffer loads with the LDS destination; their range check returns zero for
// keys outside the user's [0, key_end)), each into a ring of two slots. A slot holds
// its 64 rows unpadded, with the 16-byte chunks of a row permuted by an XOR of the row
// index (k_swz, v_swz) so the fragment reads below hit distinct banks. Each block has
// one barrier, after its first step; right after it a wave requests K of block b+2 and
// V of block b+1 (into the slots of K(b) and V(b-1), whose last reads came before the
// barrier) and waits for them at the next block's barrier, two steps later. The slots
// are separate arrays and the block loop is unrolled by two, so every access names its
// slot statically and the compiler never stalls an LDS read on an unrelated load.
//
// Per 32-key "half" h a wave computes, for each of its query blocks, S^T = K Q^T
// (queries along lanes), the bf16 weights a = SiLU(s), and O^T += V^T A^T; every K
// and V fragment read from LDS feeds all QB blocks. The V^T operand comes from the
// row-major V slot by the LDS transpose read: in each 16-lane group, lanes 4r..4r+3
// address 16 consecutive columns of key row r and lane i receives column i of those
// four rows. The key order inside the PV contraction is permuted to match the layout
// in which S^T's accumulators hold the weights; both operands use it.
//
// Software pipeline: step h issues the score MFMAs of half h + 1 and the PV MFMAs of
// half h - 1 while the VALU turns the scores of half h (finished in step h - 1) into
// weights, so no instruction of a step waits for another of the same step and the
// matrix and SiLU streams interleave. The loop body has no branches (a branch makes
// the register allocator copy the accumulators): every step of every wave does the
// same work, and masking is a wave-uniform bias inside the SiLU,
// SiLU(x) = x / (1 + 2^(x * -log2(e) + bias)), which is exactly x * sigmoid(x) for
// bias 0 and exactly 0 for bias +inf.
//
// History rows: keys are numbered from a shifted origin kappa = key + s with
// s = (-m) mod 32, so every wave's first query sits at a multiple of 32 and each
// query block meets the causal diagonal in exactly one half. Halves wholly before a
// block get bias 0; the diagonal half and every later one get +inf inside the loop,
// and a short pass after it adds the diagonal halves with a per-element mask.
// Candidate rows take bias 0 everywhere (keys past the last history key are zero, and
// SiLU(0) = 0) and add their own key in the same short pass, masked to j == i.
template <int DH>
struct AttnTile {
  static constexpr int WAVES = 4, NT = 64 * WAVES, QB = 1;
  static constexpr int BM = WAVES * QB * 32;     // query rows per work item
  static constexpr int KB = 64;                  // keys per block
  static constexpr int SLOT = KB * DH;           // elements of one K or V slot
  static constexpr int CPR = DH / 8;             // 16-byte chunks per key row
  static constexpr int RPI = 64 / CPR;           // rows one 64-lane LDS load covers
  static constexpr int IPW = KB / RPI / WAVES;   // such loads per wave per matrix and block
  static constexpr int KK = DH / 16, MB = DH / 32;
};

constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer, 32-bit data format

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Raw buffer descriptor: base address, no stride, num_records bytes (loads at or past
// it return zero).
__device__ __forceinline__ i32x4 buffer_desc(const void* base, int num_records) {
  const uint64_t a = (uint64_t)base;
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xffff, num_records, (int)kBufferWord3};
}

// One 64-lane load of 16 bytes per lane from the buffer at byte offset voff into LDS
// at lds_addr + 16 * lane. Written out so the compiler does not track it: it would
// otherwise make LDS reads of other slots wait for it. The kernel waits for these loads
// itself (vmcnt, then a barrier) before any wave reads the rows they bring. M0 holds
// the LDS address and needs one wait state before the load reads it.
__device__ __forceinline__ void lds_load16(const i32x4& desc, uint32_t lds_addr, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(desc)
      : "memory", "m0");
}

// Chunk permutations of the slots. gfx950's LDS has 64 four-byte banks; a 16-byte read
// is served 16 lanes at a time (16 consecutive K rows of one fragment) and a transpose
// read 32 lanes at a time (4 V rows x 4 chunks), so each group must cover distinct
// 16-byte bank groups. At dh = 32 a row is 64 bytes: K rows 4 apart start on the same
// bank and get distinct slots from bits 2-3 of the row; the 4 V rows of a transpose
// read are 256 consecutive bytes, all 64 banks once, so V needs no permutation.
template <int DH>
__device__ __forceinline__ int k_swz(int r) { return DH == 128 ? (r & 15) : DH == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
template <int DH>
__device__ __forceinline__ int v_swz(int r) { return DH == 128 ? 4 * (r & 3) : DH == 64 ? 4 * ((r >> 1) & 1) : 0; }

__device__ __forceinline__ float silu_bias(float x, float nlog2e, float bias) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(x, nlog2e, bias)));
}

// Relative bias (REL): each weight gains rel[h][pos_i - pos_j] after its SiLU. The kernel
// reads a float32 copy of the layer's table (widened before the launch, so the entries
// add to the float32 weights with no conversion), from the 16-byte-aligned address at or
// before the head's row (mis entries early). LDS holds a static part, kTabPad zero
// entries and then the row's first entries (entry d at tab[kTabPad + mis + d], for the
// diagonal pass and a candidate's own key), and per wave a ring of three slices of
// kSlice entries: for key block b a wave's weights only need the 96 consecutive entries
// d in [q - 64b - 63, q + 31 - 64b] (q: the wave's first query position), and the slice
// of block b + 2 (one 64-lane load of 16 bytes a lane) is loaded beside K(b + 2), into
// the slot of block b - 1. A lane reads its 16 weights' entries there; wholly masked
// halves read the zero pad instead, so every step stays branch-free. Any max_len works.
constexpr int kTabPad = 64, kSlice = 256, kRing = 3, kTabStatic = kTabPad + kSlice;

// dh = 64 fits three waves per SIMD (under 168 registers; 32 KB of K/V slots, 48 KB with
// a relative table, per workgroup), which hides more of each wave's latency; dh = 128
// needs two (233 registers, 64 KB); dh = 32 fits four (under 128 registers, 16 KB).
//
// Paged cache (PAGED): key r of the user lives in row r % 64 of page pages[key_row + r / 64]
// of the layer's pool. The buffer range is then the whole pool, and each DMA lane takes its
// row's page from the pair of page ids that a block of 64 consecutive keys can touch; the
// pair is read (wave-uniform) one block ahead. A key outside [0, key_end), or an id
// outside the pool, gets an offset past the range and reads as zero.
template <int DH>
constexpr int attn_waves_per_eu() { return DH == 32 ? 4 : DH == 64 ? 3 : 2; }

template <int DH, bool REL, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<DH>(), attn_waves_per_eu<DH>())))
void attn_kernel(AttnArgs a) {
  using C = AttnTile<DH>;
  __shared__ __attribute__((aligned(16))) u16 ks0[C::SLOT], ks1[C::SLOT], vs0[C::SLOT], vs1[C::SLOT];
  __shared__ __attribute__((aligned(16))) float tab[REL ? kTabStatic + C::WAVES * kRing * kSlice : 4];

  const AttnItem it = a.items[blockIdx.x];
  if (it.nq <= 0) return;
  const int head = it.hk >> 1, q0 = it.q0, nq = it.nq;
  const bool cand = (it.hk & 1) != 0;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so are the biases
  const int D = a.D;
  const size_t ld3 = 3 * (size_t)D;

  // this lane's query rows (one per query block)
  bool qok[C::QB];
  size_t row[C::QB];
  bf16x8 qf[C::QB][C::KK];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int qloc = wv * 32 * C::QB + qb * 32 + l32;
    qok[qb] = qloc < nq;
    row[qb] = (size_t)it.rbase + (qok[qb] ? qloc : 0);
    const u16* qrow = (const u16*)a.vqk + row[qb] * ld3 + D + head * DH;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
      qf[qb][kk] = as_bf16x8(qok[qb] ? *reinterpret_cast<const uint4*>(qrow + kk * 16 + hi * 8) : make_uint4(0, 0, 0, 0));
  }

  const int key_end = it.key_end;                         // keys [0, key_end)
  const int shift = cand ? 0 : (-it.m) & 31;              // kappa = key + shift
  const int nblk = (key_end + shift + C::KB - 1) / C::KB;
  const int wf = it.m + q0 + wv * 32 * C::QB + shift;     // kappa of this wave's first row (history)

  f32x16 oacc[C::QB][C::MB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qb][mb][e] = 0.0f;

  // key row r of this user and head at byte offset 2 * (r * ld + col) of the resource;
  // rows outside [0, key_end) read as zero
  const int ld = (int)a.ld;
  const int nbytes = PAGED ? a.npages * kPageRows * ld * 2 : key_end * ld * 2;
  const size_t row0 = PAGED ? 0 : (size_t)it.key_row;
  const i32x4 rk_src = buffer_desc((const u16*)a.kbase + row0 * a.ld + head * DH, nbytes);
  const i32x4 rv_src = buffer_desc((const u16*)a.vbase + row0 * a.ld + head * DH, nbytes);
  // PAGED: the ids of the pages holding keys key0 .. key0 + 63 (the 64-row chunks
  // floor(key0 / 64) and the next, clamped to the user's npg pages). Branch-free: a user
  // with no keys reads entry 0 of its table row (in bounds; every key is masked anyway).
  // The table is read through the constant address space: wave-uniform addresses there
  // become scalar loads, which count on lgkmcnt. (Vector loads would count on vmcnt, and
  // the wait for them would also wait for the K/V loads meant to stay in flight until
  // the block's barrier.)
  const int last_pg = max((key_end + kPageRows - 1) / kPageRows - 1, 0);
  const const_i32* tbl = (const const_i32*)(a.pages + it.key_row);
  auto page_pair = [&](int key0) -> int2 {
    if (!PAGED) return make_int2(-1, -1);
    const int c0 = key0 >> 6;
    return make_int2(tbl[min(max(c0, 0), last_pg)], tbl[min(max(c0 + 1, 0), last_pg)]);
  };
  // relative bias table of this head, read from the 16-byte-aligned address at or before it
  // (offsets before it, or past the whole table, read as zero)
  int mis = 0;
  i32x4 rel_src = {0, 0, 0, 0};
  if (REL) {
    const uintptr_t hb = (uintptr_t)((const float*)a.rel + (size_t)head * a.max_len);
    const uintptr_t ab = hb & ~(uintptr_t)15;
    const uintptr_t end = (uintptr_t)((const float*)a.rel + (size_t)(D / DH) * a.max_len);
    mis = (int)((hb - ab) / 4);
    // The range ends at the table's end: a load returns zero for each 4-byte word past
    // it, and every entry is one whole word.
    rel_src = buffer_desc((const void*)ab, (int)(end - ab));
  }

  // 64-lane LDS loads: load j of a region covers rows RPI*j.. of it; lane i brings the
  // global chunk that belongs at row RPI*j + i/CPR, slot i%CPR
  auto lds_rows = [&](const i32x4& src, u16* dst, int key0, int j, bool is_v, int2 pp) {
    const int r = C::RPI * j + lane / C::CPR, slot = lane % C::CPR;
    const int chunk = slot ^ (is_v ? v_swz<DH>(r) : k_swz<DH>(r));
    const uint32_t addr = (uint32_t)(uintptr_t)(lds_void*)(dst + j * 512);
    int voff = ((key0 + r) * ld + chunk * 8) * 2;
    if (PAGED) {
      // branch-free (a branch here would split the loop body): unsigned arithmetic, and a
      // mask instead of a short-circuit test; an invalid key or page gets offset 2^31,
      // past any pool of under 2 GiB
      const int key = key0 + r;
      const unsigned pg = (unsigned)((key >> 6) == (key0 >> 6) ? pp.x : pp.y);
      const unsigned ok = (unsigned)((unsigned)key < (unsigned)key_end) & (unsigned)(pg < (unsigned)a.npages);
      const unsigned off = ((pg * kPageRows + ((unsigned)key & (kPageRows - 1))) * (unsigned)ld + chunk * 8u) * 2u;
      voff = (int)((off & (0u - ok)) | ((ok ^ 1u) << 31));
    }
    lds_load16(src, __builtin_amdgcn_readfirstlane(addr), voff);
  };
  auto load_k = [&](u16* slot, int blk, int2 pp) {
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) lds_rows(rk_src, slot, blk * C::KB - shift, wv + C::WAVES * i, false, pp);
  };
  auto load_v = [&](u16* slot, int blk, int2 pp) {
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) lds_rows(rv_src, slot, blk * C::KB - shift, wv + C::WAVES * i, true, pp);
  };
  auto block_pages = [&](int blk) { return page_pair(blk * C::KB - shift); };
  // every LDS load of this wave has landed
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // LDS fragments: K rows for the scores, V^T columns for PV (weight chunk c, element
  // e <-> key 16c + 8*(e/4) + 4*hi + e%4 of the half; the transpose reads fetch V rows
  // 16c + 4*hi + r and + 8)
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1), tr_off = 4 * (lane & 1);
  auto read_k_at = [&](const u16* rows, bf16x8 (&kf)[C::KK]) {   // rows: key row 0 of the half
    const u16* sk = rows + l32 * DH;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
      kf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(sk + (((2 * kk + hi) ^ k_swz<DH>(l32)) * 8)));
  };
  auto read_v_at = [&](const u16* rows, bf16x8 (&vf)[2][C::MB]) {
    const int sw = v_swz<DH>(tr_row);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const u16* p = rows + (16 * c + tr_row) * DH + ((tr_chunk + 4 * mb) ^ sw) * 8 + tr_off;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 8 * DH));
        vf[c][mb] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };

  // S^T = K Q^T for query block qb; s[4*i + j] = q . k(key 8*i + 4*hi + j of the half)
  auto score_mfma = [&](const bf16x8 (&kf)[C::KK], int qb, f32x16& s) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) s = mfma32(kf[kk], qf[qb][kk], s);
  };
  auto pv_mfma = [&](const bf16x8 (&vf)[2][C::MB], int qb, const bf16x8 (&w)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) oacc[qb][mb] = mfma32(vf[c][mb], w[c], oacc[qb][mb]);
  };

  const float nlog2e = -1.4426950408889634f;
  const float kInf = __builtin_huge_valf();
  // bias of query block qb in half h: 0 for halves wholly before the block's first row
  auto bias = [&](int h, int qb) { return cand || wf + 32 * qb - 32 * h > 0 ? 0.0f : kInf; };
  // Relative bias of the weights of query block qb in half h, elements e0 .. e0 + 7
  // (element e <-> key 8*(e/4) + 4*hi + e%4 of the half, query row l32): pos_q - pos_k is
  // wf + 32*qb - 32*h + l32 - key for history rows, key_end - 32*h - key for candidates.
  // slice of key block b: the 16-byte chunk of the aligned row where it starts (floor
  // division: negative chunks read as zero), and its slot in this wave's ring
  const int qfirst = cand ? key_end : wf;
  auto slice_chunk = [&](int b) { return (mis + qfirst - 64 * b - 63) >> 2; };
  const int ring = kTabStatic + wv * kRing * kSlice;   // this wave's ring, in entries of tab
  auto slice_slot = [&](int b) { return ring + (b % kRing) * kSlice; };
  auto load_slice = [&](int b) {
    if (REL)
      lds_load16(rel_src, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(tab + slice_slot(b))),
                 (slice_chunk(b) + lane) * 16);
  };
  const int lane_off = (cand ? 0 : l32) - 4 * hi;
  auto rel_bias = [&](int h, int qb, int e0, float (&r)[8]) {
    if (!REL) return;
    const int d0 = cand ? key_end - 32 * h : wf + 32 * qb - 32 * h;
    const int b = h >> 1;
    // an integer select (a pointer select became a branch): masked halves read the zero pad
    const int at = bias(h, qb) == 0.0f ? slice_slot(b) + d0 + mis - 4 * slice_chunk(b) : 31;
    const float* tl = tab + at + lane_off;
#pragma unroll
    for (int e = e0; e < e0 + 8; ++e) r[e - e0] = tl[-(8 * (e >> 2) + (e & 3))];
  };

  // Step h: (si, wi) = scores of half h, weights of half h - 1 -> (so, wo) = scores of
  // half h + 1, weights of half h.
  // krows / vrows: the 32 K rows of half h + 1 and the 32 V rows of half h - 1
  // after_reads runs once the step's K fragment reads are issued. The V fragments are
  // read after the score MFMAs have consumed the K fragments, so the two sets never
  // occupy registers at the same time.
  auto body = [&](int h, const u16* krows, const u16* vrows, const f32x16 (&si)[C::QB], const bf16x8 (&wi)[C::QB][2],
                  f32x16 (&so)[C::QB], bf16x8 (&wo)[C::QB][2], auto after_reads) {
    bf16x8 kf[C::KK];
    read_k_at(krows, kf);
    __builtin_amdgcn_sched_barrier(0);
    after_reads();
    __builtin_amdgcn_sched_barrier(0);
    // score MFMAs with the first half of the SiLU work (the compiler interleaves the two
    // streams itself; pinning a fixed interleave measured 2% slower)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) score_mfma(kf, qb, so[qb]);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const float b = bias(h, qb);
      float r[8] = {};
      rel_bias(h, qb, 0, r);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = silu_bias(si[qb][e], nlog2e, b);
        wo[qb][e >> 3][e & 7] = (__bf16)(REL ? x + r[e] : x);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 vf[2][C::MB];
    read_v_at(vrows, vf);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) pv_mfma(vf, qb, wi[qb]);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const float b = bias(h, qb);
      float r[8] = {};
      rel_bias(h, qb, 8, r);
#pragma unroll
      for (int e = 8; e < 16; ++e) {
        const float x = silu_bias(si[qb][e], nlog2e, b);
        wo[qb][e >> 3][e & 7] = (__bf16)(REL ? x + r[e - 8] : x);
      }
    }
  };

  // V rows of "half -1" (V slot 1, rows 32..63) are multiplied by the zero weights of
  // the first step: make them finite
  for (int i = tid; i < 32 * DH / 8; i += C::NT)
    *reinterpret_cast<uint4*>(vs1 + 32 * DH + 8 * i) = make_uint4(0, 0, 0, 0);
  {
    const int2 p0 = block_pages(0), p1 = block_pages(1);
    load_k(ks0, 0, p0);
    load_k(ks1, 1, p1);
    load_v(vs0, 0, p0);
  }
  if (REL) {
    if (tid < kTabPad / 4) *reinterpret_cast<uint4*>(tab + 4 * tid) = make_uint4(0, 0, 0, 0);
    // the static part: 64 chunks = the row's first 256 - mis entries
    if (wv == 0)
      lds_load16(rel_src, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(tab + kTabPad)), lane * 16);
    load_slice(0);
    load_slice(1);
  }
  wait_loads();
  __syncthreads();
  // ping-pong state: (sA, wA) enters the even steps, (sB, wB) the odd ones
  f32x16 sA[C::QB], sB[C::QB];
  bf16x8 wA[C::QB][2], wB[C::QB][2];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) wA[qb][0] = wA[qb][1] = as_bf16x8(make_uint4(0, 0, 0, 0));
  {
    bf16x8 kf[C::KK];
    read_k_at(ks0, kf);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) score_mfma(kf, qb, sA[qb]);
  }
  // Block b with its K in kb (the other K slot holds block b + 1) and its V in vb (the
  // other V slot holds block b - 1).
  auto block = [&](int b, u16* kb, u16* kn, u16* vb, u16* vp) {
    const int2 pk = block_pages(b + 2), pv = block_pages(b + 1);   // read here, used after the wait
    body(2 * b, kb + 32 * DH, vp + 32 * DH, sA, wA, sB, wB, [] {});   // K rows of half 2b+1, V of half 2b-1
    wait_loads();                      // this wave's K(b + 1) and V(b) have landed
    __syncthreads();                   // ... everyone's; K(b) and V(b - 1) are no longer read
    body(2 * b + 1, kn, vb, sB, wB, sA, wA, [&] {                  // K rows of half 2b+2, V of half 2b
      load_k(kb, b + 2, pk);           // past the last block these rows read as zero
      load_v(vp, b + 1, pv);
      load_slice(b + 2);               // into the slot of block b - 1, last read in step 2b
    });
  };
  int b = 0;
  for (; b + 1 < nblk; b += 2) {
    block(b, ks0, ks1, vs0, vs1);
    block(b + 1, ks1, ks0, vs1, vs0);
  }
  if (b < nblk) block(b, ks0, ks1, vs0, vs1);
  if (nblk > 0) {
    // PV of the last half (its weights are in wA): V of block nblk - 1, rows 32..
    bf16x8 vf[2][C::MB];
    read_v_at(((nblk - 1) & 1 ? vs1 : vs0) + 32 * DH, vf);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) pv_mfma(vf, qb, wA[qb]);
  }

  // The diagonal pass, in a private LDS area per wave (32 K rows, then 32 V rows, laid
  // out like the slots). History rows: the diagonal half of each query block, key offset
  // j visible to row offset i when j <= i. Candidates: each row's own key (j == i), whose
  // K and V rows sit in the candidate rows of the V | Q | K buffer (rows past the item
  // read as zero).
  static_assert(C::WAVES == 4 && 64 * DH == C::SLOT, "one slot per wave for the diagonal pass");
  u16* dk = wv == 0 ? ks0 : wv == 1 ? ks1 : wv == 2 ? vs0 : vs1;
  u16* dv = dk + 32 * DH;
  const u16* own = (const u16*)a.vqk + (size_t)it.rbase * ld3 + head * DH;   // V of the item's first row
  const int own_bytes = ((nq - 1) * (int)ld3 + DH) * 2;
  const i32x4 own_v = buffer_desc(own, own_bytes), own_k = buffer_desc(own + 2 * D, own_bytes);
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    wait_loads();
    __syncthreads();   // the slots (or the previous block's area) are free
    if (cand) {
      const int r0 = wv * 32 * C::QB + qb * 32;   // the block's first row in the item
#pragma unroll
      for (int j = 0; j < 32 / C::RPI; ++j) {
        const int r = C::RPI * j + lane / C::CPR, slot = lane % C::CPR;
        const int roff = (r0 + r) * (int)ld3;
        lds_load16(own_k, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(dk + j * 512)),
                   (roff + 8 * (slot ^ k_swz<DH>(r))) * 2);
        lds_load16(own_v, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(dv + j * 512)),
                   (roff + 8 * (slot ^ v_swz<DH>(r))) * 2);
      }
    } else {
      const int k0 = wf + 32 * qb - shift;   // key of the half's first row
      const int2 pp = page_pair(k0);
#pragma unroll
      for (int j = 0; j < 32 / C::RPI; ++j) {
        lds_rows(rk_src, dk, k0, j, false, pp);
        lds_rows(rv_src, dv, k0, j, true, pp);
      }
    }
    wait_loads();
    __syncthreads();
    bf16x8 kf[C::KK], vf[2][C::MB], w[2];
    f32x16 sd;
    read_k_at(dk, kf);
    score_mfma(kf, qb, sd);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = 8 * (e >> 2) + 4 * hi + (e & 3);
      const bool vis = cand ? j == l32 : j <= l32;
      // relative position l32 - j on the diagonal (0 for a candidate's own key)
      const float r = REL && vis ? tab[kTabPad + mis + l32 - j] : 0.0f;
      const float x = silu_bias(sd[e], nlog2e, vis ? 0.0f : kInf);
      w[e >> 3][e & 7] = (__bf16)(REL ? x + r : x);
    }
    read_v_at(dv, vf);
    pv_mfma(vf, qb, w);
  }

#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    if (qok[qb]) {
      // O = bf16(inv * acc) into columns [D, 2D) of the output GEMM's operand row
      u16* orow = (u16*)a.aout + row[qb] * ld3 + D + head * DH;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o0 = a.inv * oacc[qb][mb][4 * i + 0], o1 = a.inv * oacc[qb][mb][4 * i + 1];
          const float o2 = a.inv * oacc[qb][mb][4 * i + 2], o3 = a.inv * oacc[qb][mb][4 * i + 3];
          *reinterpret_cast<uint2*>(orow + mb * 32 + i * 8 + hi * 4) = make_uint2(pack2(o0, o1), pack2(o2, o3));
        }
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(int dh, const AttnArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const bool rel = a.rel != nullptr, paged = a.pages != nullptr;
  constexpr int NT = AttnTile<64>::NT;
  static_assert(AttnTile<128>::NT == NT, "one block size");
#define HSTU_ATTN_CASE(DH, REL, PAGED) \
  if (dh == DH && rel == REL && paged == PAGED) { attn_kernel<DH, REL, PAGED><<<grid, NT, 0, s>>>(a); return hipGetLastError(); }
  HSTU_ATTN_CASE(32, false, false)
  HSTU_ATTN_CASE(32, true, false)
  HSTU_ATTN_CASE(32, false, true)
  HSTU_ATTN_CASE(32, true, true)
  HSTU_ATTN_CASE(64, false, false)
  HSTU_ATTN_CASE(64, true, false)
  HSTU_ATTN_CASE(128, false, false)
  HSTU_ATTN_CASE(128, true, false)
  HSTU_ATTN_CASE(64, false, true)
  HSTU_ATTN_CASE(64, true, true)
  HSTU_ATTN_CASE(128, false, true)
  HSTU_ATTN_CASE(128, true, true)
#undef HSTU_ATTN_CASE
  return hipErrorInvalidValue;
}

int attn_block_rows_bf16() { return AttnTile<128>::BM; }

}  // namespace hstu
