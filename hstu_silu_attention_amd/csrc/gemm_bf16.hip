// bfloat16 GEMMs of the encoder layer on gfx950: the uvqk projection (normalised
// input rows x W1, SiLU + position bias + KV-cache append in the epilogue) and the
// output GEMM ([U | O | U*O] x W2, residual in the epilogue). bf16 MFMA 32x32x16 with
// float32 accumulation.
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {
namespace {

// C[M][N] = A[M][K] * W[N][K]^T on a BM x BN tile. Four waves as 2 x 2, each owning a
// (BM/2) x (BN/2) sub-tile of (BM/64) x (BN/64) 32x32 accumulator blocks. The
// accumulators hold C^T blocks (the MFMA's A operand is a W row block), so a lane
// owns one output row and runs of 4 consecutive output columns.
//
// K advances 64 at a time through two LDS stages (rows padded to 72 elements, which
// makes the 16-byte fragment reads of 8 consecutive rows hit distinct banks). The
// next step's global loads are issued into registers before the current step's
// MFMAs and written to the other stage after them, so each step needs one barrier.
// A loaders transform rows on the way into LDS (normalisation, gating).
template <int BM, int BN>
struct Tile {
  static constexpr int BK = 64, LDK = BK + 8;
  static constexpr int TM = BM / 2, TN = BN / 2, MI = TM / 32, NI = TN / 32;
  static constexpr int AC = BM * BK / 8 / 256;  // 16-byte A chunks per thread per step
  static constexpr int BC = BN * BK / 8 / 256;  // 16-byte W chunks per thread per step
  static constexpr int STAGE = (BM + BN) * LDK;  // elements per LDS stage
};

// Thread t moves the chunks of rows t/8 + 32*i (i < AC or BC), k offset (t%8)*8.

// A rows read as stored (the normalised layer input): one base pointer, rows 32 apart.
// The buffer is padded to whole tiles, so no row needs a bounds check.
template <int AC>
struct PlainRows {
  const u16* p;
  size_t step;
  uint4 v[AC];
  __device__ __forceinline__ void init(const u16* base, int ld, int row0, int tid) {
    p = base + (size_t)(row0 + (tid >> 3)) * ld + (tid & 7) * 8;
    step = (size_t)32 * ld;
  }
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) v[i] = *reinterpret_cast<const uint4*>(p + i * step + k0);
  }
  __device__ __forceinline__ uint4 get(int i, int) const { return v[i]; }
};

// A rows of the output GEMM: [U | O | bf16(U*O)], 3D wide, built on the fly from the
// row-padded uvqk and attention-output buffers.
template <int AC>
struct GateRows {
  const u16* up;
  const u16* op;
  size_t ustep, ostep;
  uint4 u[AC], o[AC];
  int D;
  __device__ __forceinline__ void init(const OutArgs& a, int row0, int tid) {
    D = a.D;
    const int r = row0 + (tid >> 3), kc = (tid & 7) * 8;
    up = (const u16*)a.uvqk + (size_t)r * 4 * D + kc;
    op = (const u16*)a.o + (size_t)r * D + kc;
    ustep = (size_t)32 * 4 * D;
    ostep = (size_t)32 * D;
  }
  __device__ __forceinline__ void fetch(int k0) {
    if (k0 < D) {
#pragma unroll
      for (int i = 0; i < AC; ++i) u[i] = *reinterpret_cast<const uint4*>(up + i * ustep + k0);
    } else if (k0 < 2 * D) {
#pragma unroll
      for (int i = 0; i < AC; ++i) u[i] = *reinterpret_cast<const uint4*>(op + i * ostep + (k0 - D));
    } else {
#pragma unroll
      for (int i = 0; i < AC; ++i) {
        u[i] = *reinterpret_cast<const uint4*>(up + i * ustep + (k0 - 2 * D));
        o[i] = *reinterpret_cast<const uint4*>(op + i * ostep + (k0 - 2 * D));
      }
    }
  }
  __device__ __forceinline__ uint4 get(int i, int k0) const {
    if (k0 < 2 * D) return u[i];
    uint4 g;
    g.x = pack2(bf2f_lo(u[i].x) * bf2f_lo(o[i].x), bf2f_hi(u[i].x) * bf2f_hi(o[i].x));
    g.y = pack2(bf2f_lo(u[i].y) * bf2f_lo(o[i].y), bf2f_hi(u[i].y) * bf2f_hi(o[i].y));
    g.z = pack2(bf2f_lo(u[i].z) * bf2f_lo(o[i].z), bf2f_hi(u[i].z) * bf2f_hi(o[i].z));
    g.w = pack2(bf2f_lo(u[i].w) * bf2f_lo(o[i].w), bf2f_hi(u[i].w) * bf2f_hi(o[i].w));
    return g;
  }
};

// Instruction order of one k step, pinned for the scheduler (which otherwise waits
// for each fragment read right before its MFMAs): the initial fragment reads, then
// for each 16-wide sub-step but the last, the next sub-step's fragment reads
// interleaved one-to-one with this sub-step's MFMAs; the last sub-step's MFMAs are
// interleaved with the LDS writes of the next stage.
template <typename C>
__device__ __forceinline__ void schedule_step() {
  constexpr int kRead = C::MI + C::NI, kMfma = C::MI * C::NI, kWrite = C::AC + C::BC;
  constexpr unsigned MFMA = 0x008, VMEM_READ = 0x020, DS_READ = 0x100, DS_WRITE = 0x200;
  __builtin_amdgcn_sched_group_barrier(VMEM_READ, kWrite, 0);
  __builtin_amdgcn_sched_group_barrier(DS_READ, kRead, 0);
#pragma unroll
  for (int kk = 0; kk + 1 < C::BK / 16; ++kk) {
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      if (i < kRead) __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    if (i < kWrite) __builtin_amdgcn_sched_group_barrier(DS_WRITE, 1, 0);
  }
}

template <int BM, int BN, typename AL>
__device__ __forceinline__ void gemm_tile(AL& al, const u16* __restrict__ w, int K, int col0,
                                          f32x16 (&acc)[Tile<BM, BN>::MI][Tile<BM, BN>::NI], u16* smem) {
  using C = Tile<BM, BN>;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1, l32 = lane & 31, hi = lane >> 5;
  const int r0 = tid >> 3, kc = (tid & 7) * 8;
  const u16* wp = w + (size_t)(col0 + r0) * K + kc;
  uint4 rb[C::BC];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto fetch = [&](int k0) {
    al.fetch(k0);
#pragma unroll
    for (int i = 0; i < C::BC; ++i) rb[i] = *reinterpret_cast<const uint4*>(wp + (size_t)32 * i * K + k0);
  };
  auto store = [&](int stage, int k0) {
    u16* sa = smem + stage * C::STAGE;
    u16* sb = sa + BM * C::LDK;
#pragma unroll
    for (int i = 0; i < C::AC; ++i) *reinterpret_cast<uint4*>(sa + (r0 + 32 * i) * C::LDK + kc) = al.get(i, k0);
#pragma unroll
    for (int i = 0; i < C::BC; ++i) *reinterpret_cast<uint4*>(sb + (r0 + 32 * i) * C::LDK + kc) = rb[i];
  };

  const int nk = K / C::BK;
  fetch(0);
  store(0, 0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    // The last step re-fetches its own k block (never stored): every step fetches
    // unconditionally, so the prefetch registers carry nothing across iterations.
    const int kn = (t + 1 < nk ? t + 1 : t) * C::BK;
    fetch(kn);
    const u16* sa = smem + (t & 1) * C::STAGE + (wm * C::TM + l32) * C::LDK + hi * 8;
    const u16* sb = smem + (t & 1) * C::STAGE + BM * C::LDK + (wn * C::TN + l32) * C::LDK + hi * 8;
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
    // The last step stores its re-fetched block into the idle stage, which nobody
    // reads again; storing unconditionally keeps the step one basic block.
    store((t + 1) & 1, kn);
    schedule_step<C>();
    __syncthreads();
  }
}

// 256 x 256 tiles hold 256 accumulators per lane: one wave per SIMD. Saying so lets
// the scheduler keep several LDS fragment reads in flight instead of minimising
// register pressure for an occupancy it cannot reach anyway.
template <int BM> struct Occupancy { static constexpr int waves = 2; };
template <> struct Occupancy<256> { static constexpr int waves = 1; };

template <int BM, int BN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Occupancy<BM>::waves, Occupancy<BM>::waves)))
void uvqk_kernel(UvqkArgs a) {
  using C = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * C::STAGE];
  const int D = a.D, N = 4 * D, ncol = N / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int row0 = (tile / ncol) * BM, col0 = (tile % ncol) * BN;
  PlainRows<C::AC> al;
  al.init((const u16*)a.xn, D, row0, threadIdx.x);
  f32x16 acc[C::MI][C::NI];
  gemm_tile<BM, BN>(al, (const u16*)a.w, D, col0, acc, smem);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, l32 = lane & 31, hi = lane >> 5;
  const u16* pos = (const u16*)a.pos;
  u16* out = (u16*)a.uvqk;
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int row = row0 + wm * C::TM + i * 32 + l32;
    if (row >= a.T) continue;
    const int2 ri = a.row_info[row];
    const u16* prow = pos + (size_t)ri.y * 3 * D;
    const bool append = a.cache_k != nullptr && row < a.Nu;
    const size_t crow = append ? (size_t)a.users[ri.x].key_row + ri.y : 0;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + wn * C::TN + j * 32 + g * 8 + hi * 4;
        const int slice = col / D, cc = col - slice * D;
        float v0 = silu(acc[i][j][4 * g + 0]), v1 = silu(acc[i][j][4 * g + 1]);
        float v2 = silu(acc[i][j][4 * g + 2]), v3 = silu(acc[i][j][4 * g + 3]);
        if (slice > 0) {
          const uint2 bb = *reinterpret_cast<const uint2*>(prow + (slice - 1) * D + cc);
          v0 += bf2f_lo(bb.x);
          v1 += bf2f_hi(bb.x);
          v2 += bf2f_lo(bb.y);
          v3 += bf2f_hi(bb.y);
        }
        const uint2 pk = make_uint2(pack2(v0, v1), pack2(v2, v3));
        *reinterpret_cast<uint2*>(out + (size_t)row * N + col) = pk;
        if (append && (slice == 1 || slice == 3)) {
          u16* dst = (u16*)(slice == 1 ? a.cache_v : a.cache_k);
          *reinterpret_cast<uint2*>(dst + crow * D + cc) = pk;
        }
      }
      // One accumulator block at a time: keeps the scheduler from pulling every
      // accumulator out of the AGPRs at once (which would spill).
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Occupancy<BM>::waves, Occupancy<BM>::waves)))
void out_kernel(OutArgs a) {
  using C = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * C::STAGE];
  const int D = a.D, ncol = D / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int row0 = (tile / ncol) * BM, col0 = (tile % ncol) * BN;
  GateRows<C::AC> al;
  al.init(a, row0, threadIdx.x);
  f32x16 acc[C::MI][C::NI];
  gemm_tile<BM, BN>(al, (const u16*)a.w, 3 * D, col0, acc, smem);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int row = row0 + wm * C::TM + i * 32 + l32;
    if (row >= a.T) continue;
    const bool lo = row < a.Nu;
    const u16* x = lo ? (const u16*)a.x_lo + (size_t)row * D : (const u16*)a.x_hi + (size_t)(row - a.Nu) * D;
    u16* y = lo ? (u16*)a.y_lo + (size_t)row * D : (u16*)a.y_hi + (size_t)(row - a.Nu) * D;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + wn * C::TN + j * 32 + g * 8 + hi * 4;
        const uint2 xv = *reinterpret_cast<const uint2*>(x + col);
        const float y0 = bf2f_lo(xv.x) + acc[i][j][4 * g + 0];
        const float y1 = bf2f_hi(xv.x) + acc[i][j][4 * g + 1];
        const float y2 = bf2f_lo(xv.y) + acc[i][j][4 * g + 2];
        const float y3 = bf2f_hi(xv.y) + acc[i][j][4 * g + 3];
        *reinterpret_cast<uint2*>(y + col) = make_uint2(pack2(y0, y1), pack2(y2, y3));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// 256 x 256 tiles when they give at least two full rounds of workgroups over the 256
// CUs; 128 x 128 otherwise (small batches, D = 128 outputs).
bool use_big_tile(int T, int N) {
  if (N % 256) return false;
  const long tiles = (long)((T + 255) / 256) * (N / 256);
  return tiles >= 256;
}

}  // namespace

hipError_t launch_uvqk_bf16(const UvqkArgs& a, hipStream_t s) {
  const int N = 4 * a.D;
  if (use_big_tile(a.T, N))
    uvqk_kernel<256, 256><<<((a.T + 255) / 256) * (N / 256), 256, 0, s>>>(a);
  else
    uvqk_kernel<128, 128><<<((a.T + 127) / 128) * (N / 128), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s) {
  const int N = a.D;
  if (use_big_tile(a.T, N))
    out_kernel<256, 256><<<((a.T + 255) / 256) * (N / 256), 256, 0, s>>>(a);
  else
    out_kernel<128, 128><<<((a.T + 127) / 128) * (N / 128), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace hstu
