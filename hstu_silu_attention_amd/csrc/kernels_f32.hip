// float32 kernels (no intermediate rounding). These serve float32 models: plain
// LDS-tiled VALU arithmetic with float32 accumulation.
#include <hip/hip_runtime.h>

#include "hstu_internal.h"

namespace hstu {
namespace {

__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// C[M][N] = A[M][K] * W[N][K]^T on 64 x 64 tiles, K step 16, 4 x 4 outputs per thread.
constexpr int FT = 64, FK = 16;

template <typename ALoad, typename Epi>
__device__ __forceinline__ void gemm_f32(const ALoad& aload, const float* __restrict__ w, int K, int M,
                                         int ncol, const Epi& epi) {
  __shared__ float sa[FK][FT + 1];
  __shared__ float sb[FK][FT + 1];
  const int tile = blockIdx.x;
  const int row0 = (tile / ncol) * FT, col0 = (tile % ncol) * FT;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    __syncthreads();
    for (int id = tid; id < FT * FK; id += 256) {
      const int r = id / FK, k = id % FK;
      sa[k][r] = row0 + r < M ? aload(row0 + r, k0 + k) : 0.0f;
      sb[k][r] = w[(size_t)(col0 + r) * K + k0 + k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = sa[k][ty * 4 + i];
        bv[i] = sb[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) epi(row, col0 + tx * 4 + j, acc[i][j]);
  }
}

// A operands as stored: the normalised layer input, and [U | O | U*O].
struct RowLoadF {
  const float* base;
  int ld;
  __device__ __forceinline__ float operator()(int row, int k) const { return base[(size_t)row * ld + k]; }
};

__global__ __launch_bounds__(256) void uvqk_f32_kernel(UvqkArgs a) {
  const int D = a.D;
  const float* pos = (const float*)a.pos;
  auto epi = [&](int row, int col, float g) {
    const int2 ri = a.row_info[row];
    const int slice = col / D, cc = col - slice * D;
    float v = silu(g);
    if (slice > 0 && pos != nullptr) v += pos[(size_t)ri.y * 3 * D + (slice - 1) * D + cc];
    // U into the output GEMM's operand buffer, V / Q / K into the attention's
    if (slice == 0)
      ((float*)a.aout)[(size_t)row * 3 * D + cc] = v;
    else
      ((float*)a.vqk)[(size_t)row * 3 * D + (slice - 1) * D + cc] = v;
    if (a.cache_k != nullptr && row < a.Nu && (slice == 1 || slice == 3)) {
      float* dst = (float*)(slice == 1 ? a.cache_v : a.cache_k);
      const int kr = a.users[ri.x].key_row;
      if (a.pages == nullptr) {
        dst[((size_t)kr + ri.y) * D + cc] = v;
      } else {
        // paged: row pos % 64 of page table[key_row + pos / 64]; ids outside the pool skipped
        const int pg = a.pages[kr + ri.y / kPageRows];
        if ((unsigned)pg < (unsigned)a.npages) dst[((size_t)pg * kPageRows + ri.y % kPageRows) * D + cc] = v;
      }
    }
  };
  gemm_f32(RowLoadF{(const float*)a.xn, D}, (const float*)a.w, D, a.T,
           4 * D / FT, epi);
}

__global__ __launch_bounds__(256) void out_f32_kernel(OutArgs a) {
  const int D = a.D;
  auto epi = [&](int row, int col, float z) {
    if (row < a.Nu)
      ((float*)a.y_lo)[(size_t)row * D + col] = ((const float*)a.x_lo)[(size_t)row * D + col] + z;
    else
      ((float*)a.y_hi)[(size_t)(row - a.Nu) * D + col] =
          ((const float*)a.x_hi)[(size_t)(row - a.Nu) * D + col] + z;
  };
  gemm_f32(RowLoadF{(const float*)a.aout, 3 * D}, (const float*)a.w, 3 * D, a.T,
           D / FT, epi);
}

// One work item per workgroup of 64 threads; one thread per query row; key blocks of
// 32 staged in LDS.
constexpr int FBM = 64, FKB = 32;

template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float sk[FKB][DH];
  __shared__ float sv[FKB][DH];
  const AttnItem it = a.items[blockIdx.x];
  if (it.nq <= 0) return;
  const int head = it.hk >> 1, nq = it.nq;
  const bool cand = (it.hk & 1) != 0;
  const int tid = threadIdx.x;
  const int D = a.D;
  const bool qok = tid < nq;
  const size_t row = (size_t)it.rbase + tid;
  const float* vqk = (const float*)a.vqk + row * 3 * D + head * DH;  // V | Q | K of this row
  float q[DH], acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    q[e] = qok ? vqk[D + e] : 0.0f;
    acc[e] = 0.0f;
  }
  const int key_end = it.key_end;
  const int qpos = cand ? key_end : it.m + it.q0 + tid;   // candidates sit at m + n
  const float* rel = a.rel == nullptr ? nullptr : (const float*)a.rel + (size_t)head * a.max_len;
  const float* kp = (const float*)a.kbase + head * DH;
  const float* vp = (const float*)a.vbase + head * DH;
  // source row of key r: contiguous from key_row, or paged (-1: an id outside the pool)
  auto key_src = [&](int r) -> long {
    if (a.pages == nullptr) return (long)it.key_row + r;
    const int pg = a.pages[it.key_row + r / kPageRows];
    return (unsigned)pg < (unsigned)a.npages ? (long)pg * kPageRows + r % kPageRows : -1;
  };
  for (int k0 = 0; k0 < key_end; k0 += FKB) {
    __syncthreads();
    for (int id = tid; id < FKB * DH; id += 64) {
      const int key = id / DH, e = id % DH;
      const long src = k0 + key < key_end ? key_src(k0 + key) : -1;
      sk[key][e] = src >= 0 ? kp[src * a.ld + e] : 0.0f;
      sv[key][e] = src >= 0 ? vp[src * a.ld + e] : 0.0f;
    }
    __syncthreads();
    const int kn = min(FKB, key_end - k0);
    for (int j = 0; j < kn; ++j) {
      const int key = k0 + j;
      if (!cand && key > qpos) break;
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < DH; ++e) s += q[e] * sk[j][e];
      const float w = silu(s) + (rel != nullptr ? rel[qpos - key] : 0.0f);
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] += w * sv[j][e];
    }
  }
  if (!qok) return;
  if (cand) {
    const float* krow = vqk + 2 * D;
    const float* vrow = vqk;
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < DH; ++e) s += q[e] * krow[e];
    const float w = silu(s) + (rel != nullptr ? rel[0] : 0.0f);
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] += w * vrow[e];
  }
  // O into columns [D, 2D) of the output GEMM's operand row, U*O into [2D, 3D)
  float* arow = (float*)a.aout + row * 3 * D + head * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    const float o = a.inv * acc[e];
    arow[D + e] = o;
    arow[2 * D + e] = arow[e] * o;
  }
}

}  // namespace

hipError_t launch_uvqk_f32(const UvqkArgs& a, hipStream_t s) {
  uvqk_f32_kernel<<<((a.T + FT - 1) / FT) * (4 * a.D / FT), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_out_f32(const OutArgs& a, hipStream_t s) {
  out_f32_kernel<<<((a.T + FT - 1) / FT) * (a.D / FT), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(int dh, const AttnArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (dh) {
    case 32: attn_f32_kernel<32><<<grid, 64, 0, s>>>(a); break;
    case 64: attn_f32_kernel<64><<<grid, 64, 0, s>>>(a); break;
    case 128: attn_f32_kernel<128><<<grid, 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int attn_block_rows_f32() { return FBM; }

}  // namespace hstu
