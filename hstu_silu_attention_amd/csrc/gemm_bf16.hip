// bfloat16 GEMMs of the encoder layer on gfx950: the uvqk projection (layer input rows
// x W1 with the row normalisation applied to the product, SiLU + position bias +
// KV-cache append in the epilogue) and the
// output GEMM ([U | O | U*O] x W2 with the gate formed while staging, residual in the
// epilogue). bf16 MFMA 32x32x16 with
// float32 accumulation.
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {
namespace {

// C[M][N] = A[M][K] * W[N][K]^T on a BM x BN tile by WM x WN waves, each owning a
// (BM/WM) x (BN/WN) sub-tile of 32x32 accumulator blocks. The accumulators hold C^T
// blocks (the MFMA's A operand is a W row block), so a lane owns one output row and
// runs of 4 consecutive output columns.
//
// The output GEMM (gemm_tile) advances K 64 at a time through two LDS stages (rows
// padded to 72 elements, which makes the 16-byte fragment reads of 8 consecutive rows
// hit distinct banks). The next step's global loads are issued into registers before
// the current step's MFMAs and written to the other stage after them, so each step
// needs one barrier; staging through registers lets it form the gate columns of
// [U | O | U*O] from U and O on the way. The projection (gemm_tile_dma) loads its
// operands, the layer input rows as stored and W1, straight into LDS.
template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int STAGES_ = 2, int WPE_ = 0>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = 64 * WM * WN;          // threads
  static constexpr int BK = BK_, LDK = BK + 8;
  static constexpr int STAGES = STAGES_;           // LDS stages of the projection's ring
  static constexpr int TM = BM / WM, TN = BN / WN, MI = TM / 32, NI = TN / 32;
  static constexpr int RSTEP = NT / 8;             // rows between a thread's chunks
  static constexpr int AC = BM * BK / 8 / NT;      // 16-byte A chunks per thread per step
  static constexpr int BC = BN * BK / 8 / NT;      // 16-byte W chunks per thread per step
  static constexpr int STAGE = (BM + BN) * LDK;    // elements per LDS stage
  // 256 accumulators per lane leave room for one wave per SIMD only; WPE_ asks for more
  // waves per SIMD where the registers allow.
  static constexpr int WAVES_PER_EU = WPE_ ? WPE_ : MI * NI * 16 >= 256 ? 1 : 2;
};

// Thread t moves the chunks of rows t/8 + RSTEP*i (i < AC or BC), k offset (t%8)*8.

// A-operand loader of gemm_tile. A GEMM's K range is walked in steps of BK; a loader
// with PARTS parts visits step t as part t % PARTS of chunk t / PARTS and says which K
// offset of W that step multiplies (kw). GatedRows reads the output GEMM's operand rows
// [U | O | U*O]: part 0 is a chunk of U, part 1 the same chunk of O, and part 2 its gate
// U*O, formed from the two in registers and rounded to bfloat16.
template <int AC, int RSTEP>
struct GatedRows {
  static constexpr int PARTS = 3;
  const u16* p;
  size_t step;
  int D;
  uint4 u[AC], o[AC];
  __device__ __forceinline__ void init(const u16* base, int d, int row0, int tid) {
    D = d;
    p = base + (size_t)(row0 + (tid >> 3)) * 3 * d + (tid & 7) * 8;
    step = (size_t)RSTEP * 3 * d;
  }
  __device__ __forceinline__ void fetch(int part, int chunk) {
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < AC; ++i) u[i] = *reinterpret_cast<const uint4*>(p + i * step + chunk * 64);
    } else if (part == 1) {
#pragma unroll
      for (int i = 0; i < AC; ++i) o[i] = *reinterpret_cast<const uint4*>(p + i * step + D + chunk * 64);
    }
  }
  __device__ __forceinline__ uint4 get(int part, int i, float) const {
    if (part == 0) return u[i];
    if (part == 1) return o[i];
    const uint32_t uw[4] = {u[i].x, u[i].y, u[i].z, u[i].w}, ow[4] = {o[i].x, o[i].y, o[i].z, o[i].w};
    uint32_t g[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      g[e] = pack2(bf2f_lo(uw[e]) * bf2f_lo(ow[e]), bf2f_hi(uw[e]) * bf2f_hi(ow[e]));
    return make_uint4(g[0], g[1], g[2], g[3]);
  }
  __device__ __forceinline__ int kw(int part, int chunk) const { return part * D + chunk * 64; }
};

// Instruction order of one k step, pinned for the scheduler (which otherwise waits
// for each fragment read right before its MFMAs): the global loads, the initial
// fragment reads, then for each 16-wide sub-step but the last, the next sub-step's
// fragment reads interleaved one-to-one with this sub-step's MFMAs; the last
// sub-step's MFMAs are interleaved with the LDS writes of the next stage.
template <typename C>
__device__ __forceinline__ void schedule_step() {
  constexpr int kRead = C::MI + C::NI, kMfma = C::MI * C::NI, kWrite = C::AC + C::BC;
  constexpr unsigned MFMA = 0x008, VMEM_READ = 0x020, DS_READ = 0x100, DS_WRITE = 0x200;
  __builtin_amdgcn_sched_group_barrier(VMEM_READ, kWrite, 0);
  __builtin_amdgcn_sched_group_barrier(DS_READ, kRead, 0);
#pragma unroll
  for (int kk = 0; kk + 1 < C::BK / 16; ++kk) {
#pragma unroll
    for (int i = 0; i < (kMfma > kRead ? kMfma : kRead); ++i) {
      if (i < kRead) __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
      if (i < kMfma) __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < (kMfma > kWrite ? kMfma : kWrite); ++i) {
    if (i < kMfma) __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    if (i < kWrite) __builtin_amdgcn_sched_group_barrier(DS_WRITE, 1, 0);
  }
}

template <typename C, typename AL>
__device__ __forceinline__ void gemm_tile(AL& al, const u16* __restrict__ w, int K, int col0,
                                          f32x16 (&acc)[C::MI][C::NI], u16* smem) {
  constexpr int P = AL::PARTS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / C::WN, wn = wv % C::WN, l32 = lane & 31, hi = lane >> 5;
  const int r0 = tid >> 3, kc = (tid & 7) * 8;
  const u16* wp = w + (size_t)(col0 + r0) * K + kc;
  uint4 rb[C::BC];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto fetch = [&](int part, int chunk) {
    al.fetch(part, chunk);
    const int k0 = al.kw(part, chunk);
#pragma unroll
    for (int i = 0; i < C::BC; ++i) rb[i] = *reinterpret_cast<const uint4*>(wp + (size_t)C::RSTEP * i * K + k0);
  };
  auto store = [&](int stage, int part, float fresh) {
    u16* sa = smem + stage * C::STAGE;
    u16* sb = sa + C::BM * C::LDK;
#pragma unroll
    for (int i = 0; i < C::AC; ++i)
      *reinterpret_cast<uint4*>(sa + (r0 + C::RSTEP * i) * C::LDK + kc) = al.get(part, i, fresh);
#pragma unroll
    for (int i = 0; i < C::BC; ++i) *reinterpret_cast<uint4*>(sb + (r0 + C::RSTEP * i) * C::LDK + kc) = rb[i];
  };

  const int nchunk = K / C::BK / P;
  fetch(0, 0);
  store(0, 0, 1.0f);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
#pragma unroll
    for (int part = 0; part < P; ++part) {
      const int t = c * P + part;
      // The next step's operands: the next part of this chunk, or part 0 of the next
      // chunk (the last chunk's is fetched again into the idle stage, so every step
      // fetches and stores unconditionally and stays one basic block).
      const int np = part + 1 < P ? part + 1 : 0;
      const int nc = part + 1 < P ? c : min(c + 1, nchunk - 1);
      fetch(np, nc);
      const u16* sa = smem + (t & 1) * C::STAGE + (wm * C::TM + l32) * C::LDK + hi * 8;
      const u16* sb = smem + (t & 1) * C::STAGE + C::BM * C::LDK + (wn * C::TN + l32) * C::LDK + hi * 8;
      // Fragments double-buffered in registers: the LDS reads of sub-step kk+1 are in
      // flight while the MFMAs of sub-step kk run.
      bf16x8 af[2][C::MI], bw[2][C::NI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i) af[0][i] = as_bf16x8(*reinterpret_cast<const uint4*>(sa + i * 32 * C::LDK));
#pragma unroll
      for (int j = 0; j < C::NI; ++j) bw[0][j] = as_bf16x8(*reinterpret_cast<const uint4*>(sb + j * 32 * C::LDK));
#pragma unroll
      for (int kk = 0; kk < C::BK / 16; ++kk) {
        const int cur = kk & 1, nxt = cur ^ 1;
        if (kk + 1 < C::BK / 16) {
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
            af[nxt][i] = as_bf16x8(*reinterpret_cast<const uint4*>(sa + i * 32 * C::LDK + (kk + 1) * 16));
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
            bw[nxt][j] = as_bf16x8(*reinterpret_cast<const uint4*>(sb + j * 32 * C::LDK + (kk + 1) * 16));
        }
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j) acc[i][j] = mfma32(bw[cur][j], af[cur][i], acc[i][j]);
      }
      store((t + 1) & 1, np, part + 1 < P || c + 1 < nchunk ? 1.0f : 0.0f);
      schedule_step<C>();
      __syncthreads();
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One 64-lane load of 16 bytes per lane from global memory straight into LDS at
// lds_addr + 16 * lane (no register round trip). Written out so the compiler does not
// track it (it would make every later LDS read wait for it); the caller waits with
// vmcnt and a barrier before any wave reads the rows. M0 needs one wait state.
__device__ __forceinline__ void lds_load16(uint32_t lds_addr, const void* src) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds_addr), "v"(src)
      : "memory", "m0");
}

// The projection's main loop with its operands loaded straight into LDS. A stage holds
// BM A rows then BN W rows of BK elements (BK = 64 or 32), unpadded (RB = 2 * BK bytes a
// row). The 16-byte chunk c of row r sits at slot c ^ swz(r), swz(r) = (r / (256 / RB)) %
// (RB / 16): rows 256 / RB apart start on the same bank, and swz gives the RB / 16 such
// rows among any 16 consecutive ones distinct slots, so the fragment reads of 16
// consecutive rows hit distinct banks. Load j of a stage (64 lanes, 1 KB) fills its rows
// (1024 / RB) j .. (1024 / RB) (j + 1) - 1; wave w issues loads w, w + WAVES, ... The
// stages form a ring of STAGES: step t waits for its own stage (issued STAGES - 1 steps
// earlier; the loads of later steps stay in flight), synchronises, requests step
// t + STAGES - 1 into the stage step t - 1 used, then runs its MFMAs.
template <typename C>
__device__ __forceinline__ void gemm_tile_dma(const UvqkArgs& a, int row0, int col0, f32x16 (&acc)[C::MI][C::NI],
                                              u16* smem) {
  constexpr int BK = C::BK, S = C::STAGES, RB = 2 * BK, CPRW = RB / 16, RPL = 1024 / RB;
  constexpr int WAVES = C::NT / 64;
  static_assert((BK == 64 || BK == 32) && S >= 2 && (C::BM + C::BN) % (RPL * WAVES) == 0, "whole loads per wave");
  constexpr int LOADS = (C::BM + C::BN) / RPL / WAVES;   // per wave per stage
  constexpr int SROWS = C::BM + C::BN;                   // rows of a stage
  auto swz = [](int r) { return (r / (256 / RB)) & (CPRW - 1); };
  const int D = a.D, K = D;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / C::WN, wn = wv % C::WN, l32 = lane & 31, hi = lane >> 5;
  // this lane's source row of each of its loads, at k = 0
  const u16* src[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = RPL * (wv + WAVES * i) + lane / CPRW;    // row of the stage
    const int c = (lane % CPRW) ^ swz(r);                  // chunk that belongs in this slot
    if (r < C::BM) {
      const int row = min(row0 + r, a.T - 1);
      src[i] = (row < a.Nu ? (const u16*)a.x_lo + (size_t)row * D : (const u16*)a.x_hi + (size_t)(row - a.Nu) * D) + c * 8;
    } else {
      src[i] = (const u16*)a.w + (size_t)(col0 + r - C::BM) * K + c * 8;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      lds_load16(lds0 + stage * SROWS * RB + (wv + WAVES * i) * 1024, src[i] + k0);
  };
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int sw = swz(l32);                                   // this lane's rows' chunk swizzle
  const int nstep = K / BK;
#pragma unroll
  for (int t = 0; t + 1 < S; ++t)
    if (t < nstep) issue(t, t * BK);
  for (int t = 0; t < nstep; ++t) {
    // stage t has landed once at most the loads of the steps after it are outstanding
    if (S > 2 && t + 1 < nstep)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (S - 2)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                                          // stage t % S is complete; stage (t - 1) % S is free
    if (t + S - 1 < nstep) issue((t + S - 1) % S, (t + S - 1) * BK);
    const u16* sa = smem + (t % S) * SROWS * BK + (wm * C::TM + l32) * BK;
    const u16* sb = smem + (t % S) * SROWS * BK + (C::BM + wn * C::TN + l32) * BK;
    bf16x8 af[2][C::MI], bw[2][C::NI];
    auto rd = [&](const u16* p, int kk) { return as_bf16x8(*reinterpret_cast<const uint4*>(p + (((2 * kk + hi) ^ sw) * 8))); };
#pragma unroll
    for (int i = 0; i < C::MI; ++i) af[0][i] = rd(sa + i * 32 * BK, 0);
#pragma unroll
    for (int j = 0; j < C::NI; ++j) bw[0][j] = rd(sb + j * 32 * BK, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) af[nxt][i] = rd(sa + i * 32 * BK, kk + 1);
#pragma unroll
        for (int j = 0; j < C::NI; ++j) bw[nxt][j] = rd(sb + j * 32 * BK, kk + 1);
      }
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j) acc[i][j] = mfma32(bw[cur][j], af[cur][i], acc[i][j]);
    }
    {
      constexpr int kRead = C::MI + C::NI, kMfma = C::MI * C::NI;
      constexpr unsigned MFMA = 0x008, DS_READ = 0x100;
      __builtin_amdgcn_sched_group_barrier(DS_READ, kRead, 0);
#pragma unroll
      for (int kk = 0; kk + 1 < BK / 16; ++kk)
#pragma unroll
        for (int i = 0; i < (kMfma > kRead ? kMfma : kRead); ++i) {
          if (i < kRead) __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
          if (i < kMfma) __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        }
      __builtin_amdgcn_sched_group_barrier(MFMA, kMfma, 0);
    }
  }
  __syncthreads();                                            // the stages are free for the epilogue
}

template <typename C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
void uvqk_kernel(UvqkArgs a) {
  constexpr int RING = C::STAGES * (C::BM + C::BN) * C::BK, STAGED = C::BM * (C::BN + 8);
  constexpr int SMEM = RING > STAGED ? RING : STAGED;
  __shared__ __attribute__((aligned(1024))) u16 smem[SMEM];
  const int D = a.D, N = 4 * D, ncol = N / C::BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int row0 = (tile / ncol) * C::BM, col0 = (tile % ncol) * C::BN;
  __shared__ float row_mean[C::BM];
  __shared__ float2 row_scale[C::BM];                // {-log2(e) / sigma, sigma}, sigma = sqrt(var + eps)
  __shared__ int row_pos[C::BM];                     // position of each tile row (its bias row)
  __shared__ __attribute__((aligned(16))) float col_sum[256];   // W1 column sums of the tile's columns
  static_assert(C::BN <= 256 && C::NT >= C::BM, "one tile row per thread; one load of column sums");
  // The epilogue's inputs that depend only on the tile are requested before the main
  // loop, so their latency hides under it: the row's group statistics (the first four
  // groups in registers; a wider row reads the rest in the epilogue) and its position,
  // and the W1 column sums (one 64-lane LDS load by wave 0, issued ahead of its first
  // stage, whose wait then covers it).
  const int groups = D / 128;
  const bool has_row = threadIdx.x < C::BM;
  const int rr = min(row0 + (int)threadIdx.x, a.T - 1);
  float2 stp[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) stp[g] = has_row && g < groups ? a.st[(size_t)rr * groups + g] : make_float2(0.0f, 0.0f);
  const int posp = has_row ? a.row_info[rr].y : 0;
  if (threadIdx.x < 64)
    lds_load16((uint32_t)(uintptr_t)(lds_void*)col_sum, a.cs + col0 + min(4 * (int)threadIdx.x, C::BN - 4));
  f32x16 acc[C::MI][C::NI];
  gemm_tile_dma<C>(a, row0, col0, acc, smem);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv / C::WN, wn = wv % C::WN, l32 = lane & 31, hi = lane >> 5;
  // Row mean and variance from the per-128-column group statistics, merged in column
  // order (as merge_group_stats does).
  if (has_row) {
    float mean = stp[0].x, m2 = stp[0].y;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i < groups) merge_group_step(mean, m2, stp[i], i);
    for (int i = 4; i < groups; ++i) merge_group_step(mean, m2, a.st[(size_t)rr * groups + i], i);
    const float sigma = sqrtf(m2 / (float)(128 * groups) + kNormEps);
    row_mean[threadIdx.x] = mean;
    row_scale[threadIdx.x] = make_float2(-1.4426950408889634f / sigma, sigma);
    row_pos[threadIdx.x] = posp;
  }
  // Column sums of W1 for this lane's columns: the normalisation is applied to the
  // product, Xn W1 = (X W1 - mean * colsum(W1)) / sigma row by row, exactly; the mean
  // term is taken here, the 1 / sigma inside the SiLU below.
  float csum[C::NI][4][4];
#pragma unroll
  for (int j = 0; j < C::NI; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 c4 = *reinterpret_cast<const float4*>(col_sum + wn * C::TN + j * 32 + g * 8 + hi * 4);
      csum[j][g][0] = c4.x;
      csum[j][g][1] = c4.y;
      csum[j][g][2] = c4.z;
      csum[j][g][3] = c4.w;
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const float mean = row_mean[wm * C::TM + i * 32 + l32];
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][4 * g + e] = __builtin_fmaf(-mean, csum[j][g][e], acc[i][j][4 * g + e]);
  }
  // A tile lies inside one of the U, V, Q, K column blocks (D is a multiple of BN).
  const int slice = col0 / D;
  // The position-bias tile goes through the (now idle) LDS: every 32 consecutive
  // threads read one row's 256 bias values as whole lines (the row's position comes
  // from the row table). Each lane then reads the bias at the places of its
  // accumulators and writes its results over them: every tile position belongs to one
  // lane, which reads it before writing it, so no barrier is needed in between.
  constexpr int OLD = C::BN + 8;                     // LDS row stride of the staged tiles
  static_assert(C::BM * OLD <= SMEM, "a staged tile must fit the LDS stages");
  constexpr int CPR = C::BN / 8;                     // 16-byte chunks per tile row
  // Thread t moves the 16-byte chunk (t % CPR) of tile rows t / CPR + RSTEP_O * i.
  constexpr int RSTEP_O = C::NT / CPR;
  static_assert(C::NT % CPR == 0, "a thread keeps its chunk column");
  const int r_first = threadIdx.x / CPR, cc = (threadIdx.x % CPR) * 8;
  const bool has_bias = slice > 0 && a.pos != nullptr;   // uniform over the workgroup
  if (has_bias) {
    // a position table has fewer than 2^31 elements (checked on the host), so a
    // position's element offset is a 24 x 24-bit product
    const u16* pos = (const u16*)a.pos + (slice - 1) * D + (col0 - slice * D) + cc;
#pragma unroll
    for (int i = 0; i < C::BM * CPR / C::NT; ++i) {
      const int r = r_first + RSTEP_O * i;
      *reinterpret_cast<uint4*>(smem + r * OLD + cc) =
          *reinterpret_cast<const uint4*>(pos + __umul24((unsigned)row_pos[r], 3u * (unsigned)D));
    }
    __syncthreads();
  }
  // The finished tile goes through the LDS too: each lane writes its rounded values
  // there, then every 32 consecutive threads store 512 contiguous bytes of one row, so
  // the global writes are whole cache lines.
  // With a = X W1 - mean * colsum(W1) and y = a / sigma: SiLU(y) = y / (1 + 2^(-y log2 e))
  // = a / (sigma + sigma * 2^(a * (-log2(e) / sigma))).
  // without a bias the staged area holds stale bits: masked to +0 (integer, so NaN-safe)
  const uint32_t bias_mask = has_bias ? ~0u : 0u;
  auto silu_n = [](float a, float2 sc) {
    return a * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(a * sc.x), sc.y, sc.y));
  };
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int r = wm * C::TM + i * 32 + l32;
    const float2 sc = row_scale[r];
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2* at = reinterpret_cast<uint2*>(smem + r * OLD + wn * C::TN + j * 32 + g * 8 + hi * 4);
        uint2 bias = *at;          // read unconditionally (a select here became a branch per read)
        bias.x &= bias_mask;
        bias.y &= bias_mask;
        const float v0 = silu_n(acc[i][j][4 * g + 0], sc) + bf2f_lo(bias.x);
        const float v1 = silu_n(acc[i][j][4 * g + 1], sc) + bf2f_hi(bias.x);
        const float v2 = silu_n(acc[i][j][4 * g + 2], sc) + bf2f_lo(bias.y);
        const float v3 = silu_n(acc[i][j][4 * g + 3], sc) + bf2f_hi(bias.y);
        *at = make_uint2(pack2(v0, v1), pack2(v2, v3));
      }
    }
  }
  __syncthreads();
  // U goes to the output GEMM's operand buffer, V/Q/K to the attention's (both 3D wide);
  // new history rows' V and K are also appended to the cache. The stores are
  // non-temporal: the 4 x T x D outputs are not read again before they leave L2, and
  // through L2 they evicted W1, the layer input rows and the bias rows that the other
  // tiles of the XCD still read (reads per launch 348 -> 215 MB at the benchmark size,
  // W1 alone had been re-read for 184 MB). Each 32 lanes store whole lines, so the
  // writes stay whole.
  const int ccol = col0 - slice * D;
  u16* out = (slice == 0 ? (u16*)a.aout : (u16*)a.vqk + (slice - 1) * D) + ccol;
  u16* cache = a.cache_k == nullptr ? nullptr
               : slice == 1 ? (u16*)a.cache_v + ccol
               : slice == 3 ? (u16*)a.cache_k + ccol : nullptr;
  u16* const out0 = out + (size_t)(row0 + r_first) * 3 * D + cc;
  // Cache rows of this thread's history rows (-1: none), looked up before the stores: all
  // row-table reads in flight together, then all user-record reads, then (paged cache)
  // all page-table reads (a lookup per store would wait for dependent reads each time).
  // A paged row goes to row pos % 64 of page table[key_row + pos / 64]; an id outside
  // the pool is skipped.
  constexpr int NR = C::BM * CPR / C::NT;
  const bool append = cache != nullptr && row0 < a.Nu;   // uniform over the workgroup
  int crow[NR];
  if (append) {
    int2 q[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) q[i] = a.row_info[min(row0 + r_first + RSTEP_O * i, a.T - 1)];
#pragma unroll
    for (int i = 0; i < NR; ++i) crow[i] = row0 + r_first + RSTEP_O * i < a.Nu ? a.users[q[i].x].key_row : -1;
    if (a.pages != nullptr) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int pg = crow[i] >= 0 ? a.pages[crow[i] + (q[i].y >> 6)] : -1;
        crow[i] = (unsigned)pg < (unsigned)a.npages ? pg * kPageRows + (q[i].y & (kPageRows - 1)) : -1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) crow[i] = crow[i] >= 0 ? crow[i] + q[i].y : -1;
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r_first + RSTEP_O * i;
    const int row = row0 + r;
    if (row >= a.T) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(smem + r * OLD + cc);
    const u32x4 nv = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(out0 + (size_t)i * RSTEP_O * 3 * D));
    if (append && crow[i] >= 0) __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(cache + (size_t)crow[i] * D + cc));
  }
}

template <typename C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
void out_kernel(OutArgs a) {
  __shared__ __attribute__((aligned(16))) u16 smem[2 * C::STAGE];
  const int D = a.D, ncol = D / C::BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int row0 = (tile / ncol) * C::BM, col0 = (tile % ncol) * C::BN;
  GatedRows<C::AC, C::RSTEP> al;
  al.init((const u16*)a.aout, D, row0, threadIdx.x);
  f32x16 acc[C::MI][C::NI];
  gemm_tile<C>(al, (const u16*)a.w, 3 * D, col0, acc, smem);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv / C::WN, wn = wv % C::WN, l32 = lane & 31, hi = lane >> 5;
  // The residual tile comes into the (now idle) LDS as whole lines (every 32
  // consecutive threads read 512 contiguous bytes of one row); each lane adds its
  // accumulators to its own elements there, rounds, and writes them back in place;
  // then the tile leaves as whole lines too.
  constexpr int OLD = C::BN + 8;                     // LDS row stride of the staged tile
  static_assert(C::BM * OLD <= 2 * C::STAGE, "the staged tile must fit the LDS stages");
  constexpr int CPR = C::BN / 8;                     // 16-byte chunks per tile row
  auto xrow = [&](int row) {
    return row < a.Nu ? (const u16*)a.x_lo + (size_t)row * D : (const u16*)a.x_hi + (size_t)(row - a.Nu) * D;
  };
#pragma unroll
  for (int i = 0; i < C::BM * CPR / C::NT; ++i) {
    const int c = threadIdx.x + C::NT * i, r = c / CPR, cc = (c % CPR) * 8;
    *reinterpret_cast<uint4*>(smem + r * OLD + cc) =
        *reinterpret_cast<const uint4*>(xrow(min(row0 + r, a.T - 1)) + col0 + cc);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int r = wm * C::TM + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2* p = reinterpret_cast<uint2*>(smem + r * OLD + wn * C::TN + j * 32 + g * 8 + hi * 4);
        const uint2 xv = *p;
        const float y0 = bf2f_lo(xv.x) + acc[i][j][4 * g + 0];
        const float y1 = bf2f_hi(xv.x) + acc[i][j][4 * g + 1];
        const float y2 = bf2f_lo(xv.y) + acc[i][j][4 * g + 2];
        const float y3 = bf2f_hi(xv.y) + acc[i][j][4 * g + 3];
        *p = make_uint2(pack2(y0, y1), pack2(y2, y3));
      }
    }
  }
  __syncthreads();
  // Also the next layer's row statistics: each 16 consecutive threads hold one row's
  // 128-column group, whose {mean, M2} group_stats forms exactly as the first layer's
  // row pass does.
  static_assert(CPR % 16 == 0, "whole 128-column groups per tile row");
#pragma unroll
  for (int i = 0; i < C::BM * CPR / C::NT; ++i) {
    const int c = threadIdx.x + C::NT * i, r = c / CPR, cc = (c % CPR) * 8;
    const int row = row0 + r;
    const uint4 v = *reinterpret_cast<const uint4*>(smem + r * OLD + cc);
    if (a.st != nullptr) {
      const float2 g = group_stats(v);
      if ((c & 15) == 0 && row < a.T) a.st[(size_t)row * (D / 128) + (col0 + cc) / 128] = g;
    }
    if (row >= a.T) continue;
    u16* y = row < a.Nu ? (u16*)a.y_lo + (size_t)row * D : (u16*)a.y_hi + (size_t)(row - a.Nu) * D;
    *reinterpret_cast<uint4*>(y + col0 + cc) = v;
  }
}

// Tile shapes: the output GEMM takes the large one for big batches and the 128 x 128 one
// when the large tiles would not give every CU at least one workgroup; the projection
// takes the ring tiles below, or the 128 x 128 one for small batches.
using BigTile = Tile<256, 256, 2, 4>;
using SmallTile = Tile<128, 128, 2, 2>;
// The projection's 256 x 128 tile on 4 waves with a 3-stage ring of 32-wide K steps:
// 77 KB of LDS, so two workgroups share a CU and one's epilogue runs beside the
// other's main loop. Its 128 x 128 tile with the same ring takes 51 KB and under 170
// registers a lane, so three workgroups share a CU.
using HalfTile = Tile<256, 128, 2, 2, 32, 3>;
using QuarterTile = Tile<128, 128, 2, 2, 32, 3, 3>;

template <typename C>
long tiles_of(int T, int N) {
  return N % C::BN ? 0 : (long)((T + C::BM - 1) / C::BM) * (N / C::BN);
}

}  // namespace

hipError_t launch_uvqk_bf16(const UvqkArgs& a, hipStream_t s) {
  // A tile must lie inside one of the U, V, Q, K column blocks: D % BN == 0 (D is a
  // multiple of 128 for bfloat16 models). Half tiles (two workgroups per CU) when they
  // fill at least two rounds of 512; quarter tiles (three per CU) when they fill a round
  // of 768; otherwise 128 x 128 tiles one per CU (small batches).
  const int N = 4 * a.D;
  const int th = tiles_of<HalfTile>(a.T, N), tq = tiles_of<QuarterTile>(a.T, N);
  if (a.D % HalfTile::BN == 0 && th >= 1024)
    uvqk_kernel<HalfTile><<<th, HalfTile::NT, 0, s>>>(a);
  else if (a.D % QuarterTile::BN == 0 && tq >= 768)
    uvqk_kernel<QuarterTile><<<tq, QuarterTile::NT, 0, s>>>(a);
  else
    uvqk_kernel<SmallTile><<<tiles_of<SmallTile>(a.T, N), SmallTile::NT, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s) {
  const int N = a.D;
  if (tiles_of<BigTile>(a.T, N) >= 256)
    out_kernel<BigTile><<<tiles_of<BigTile>(a.T, N), BigTile::NT, 0, s>>>(a);
  else
    out_kernel<SmallTile><<<tiles_of<SmallTile>(a.T, N), SmallTile::NT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace hstu
