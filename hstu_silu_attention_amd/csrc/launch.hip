// The jagged row planner kernel and the per-dtype launch dispatch.
#include <hip/hip_runtime.h>

#include <cstddef>

#include "hstu.h"
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {

hipError_t launch_uvqk_bf16(const UvqkArgs& a, hipStream_t s);
hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(int dh, const AttnArgs& a, int grid, hipStream_t s);
int attn_block_rows_bf16();
hipError_t launch_uvqk_f32(const UvqkArgs& a, hipStream_t s);
hipError_t launch_out_f32(const OutArgs& a, hipStream_t s);
hipError_t launch_attn_f32(int dh, const AttnArgs& a, int grid, hipStream_t s);
int attn_block_rows_f32();

namespace {

// Packed row r -> {user, absolute position}. History rows [0, Nu) belong to the user
// whose history segment holds r, at position m + (r - uoff); candidate rows
// [Nu, T) to the user whose candidate segment holds r - Nu, all at position m + n.
// The user is the last one whose segment starts at or before r (segments of empty
// users start where the next one does).
//
// The blocks past the rows' expand the planner's compact work items: workgroup w of
// the attention gets item w.
__global__ __launch_bounds__(256) void plan_rows_kernel(PlanArgs a) {
  const int row_blocks = (a.T + 255) / 256;
  if ((int)blockIdx.x >= row_blocks) {
    const int w = ((int)blockIdx.x - row_blocks) * 256 + threadIdx.x;
    if (w >= a.grid) return;
    const ItemCode ic = a.codes[w];
    AttnItem it{0, 0, 0, 0, 0, 0, 0, 0};
    if (ic.user >= 0) {
      const UserRec u = a.users[ic.user];
      const bool cand = (ic.code & 1) != 0;
      const int q0 = (ic.code >> 8) * a.bm;
      it.hk = ic.code & 0xff;
      it.q0 = q0;
      it.nq = min(a.bm, (cand ? u.c : u.n) - q0);
      it.m = u.m;
      it.rbase = (cand ? a.Nu + u.coff : u.uoff) + q0;
      it.key_end = cand ? u.m + u.n : u.m + q0 + it.nq;
      it.key_row = u.key_row;
    }
    a.items[w] = it;
    return;
  }
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.T) return;
  const bool hist = r < a.Nu;
  const int key = hist ? r : r - a.Nu;
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int start = hist ? a.users[mid].uoff : a.users[mid].coff;
    if (start <= key) lo = mid; else hi = mid - 1;
  }
  const UserRec u = a.users[lo];
  a.row_info[r] = make_int2(lo, hist ? u.m + (key - u.uoff) : u.m + u.n);
}

// The payload is read through the kernel-argument segment pointer, so indexing it by
// thread never copies the argument block into private memory.
__global__ __launch_bounds__(256) void upload_kernel(UploadArgs a) {
  const uint32_t* w = (const uint32_t*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(UploadArgs, w));
  for (int i = threadIdx.x; i < a.words; i += 256) a.dst[i] = w[i];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// 16-byte chunk <-> floats: 4 float32 or 8 bfloat16 values.
__device__ __forceinline__ void load_chunk(const float* p, float* v) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void load_chunk(const u16* p, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf2f_lo(w[e]);
    v[2 * e + 1] = bf2f_hi(w[e]);
  }
}
__device__ __forceinline__ void store_chunk(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_chunk(u16* p, const float* v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}

// One wave per row: the mean, then the mean squared deviation, each reduced across
// the wave in a fixed butterfly order (a row's result depends on that row alone),
// then the normalised row (x - mean) / sqrt(var + eps), rounded to the storage type.
template <typename T>
__global__ __launch_bounds__(256) void norm_kernel(NormArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.T) return;
  const int D = a.D, nchunk = D / VEC;
  const T* x = row < a.Nu ? (const T*)a.x_lo + (size_t)row * D : (const T*)a.x_hi + (size_t)(row - a.Nu) * D;
  T* y = (T*)a.xn + (size_t)row * D;
  float v[VEC];
  float s = 0.0f;
  for (int c = lane; c < nchunk; c += 64) {
    load_chunk(x + c * VEC, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) s += v[e];
  }
  const float mean = wave_sum(s) / (float)D;
  float q = 0.0f;
  for (int c = lane; c < nchunk; c += 64) {
    load_chunk(x + c * VEC, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) q += (v[e] - mean) * (v[e] - mean);
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)D + kNormEps);
  for (int c = lane; c < nchunk; c += 64) {
    load_chunk(x + c * VEC, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = (v[e] - mean) * rstd;
    store_chunk(y + c * VEC, v);
  }
}

// One wave per row of W1 (one output feature): the sum of its D bfloat16 values, in a
// fixed order (each lane's chunks in turn, then the wave's butterfly).
__global__ __launch_bounds__(256) void colsum_kernel(ColsumArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nrow = 4 * a.D;
  if (row >= a.L * nrow) return;
  const u16* w = (const u16*)a.w[row / nrow] + (size_t)(row % nrow) * a.D;
  float s = 0.0f;
  for (int c = lane; c < a.D / 8; c += 64) {
    float v[8];
    load_chunk(w + c * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[e];
  }
  s = wave_sum(s);
  if (lane == 0) a.cs[row] = s;
}

// One wave per row: {mean, sum of squared deviations from that mean} of each
// 128-column group (group_stats: 16 lanes of 8 values each). The output GEMM computes
// the later layers' rows with the same function on the same lane layout, so a row's
// statistics come out bit-identical whichever kernel produced them.
__global__ __launch_bounds__(256) void rowstats_kernel(const void* x_lo, const void* x_hi, int Nu, int T, int D, float2* st) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= T) return;
  const u16* x = row < Nu ? (const u16*)x_lo + (size_t)row * D : (const u16*)x_hi + (size_t)(row - Nu) * D;
  for (int c0 = 0; c0 < D / 8; c0 += 64) {          // 64 chunks = 4 groups per pass
    const int c = c0 + lane;
    // D is a multiple of 128, so a 16-lane group is either wholly inside the row or
    // wholly past it; the lanes past it feed zeros and their results are dropped
    const uint4 q = c < D / 8 ? *reinterpret_cast<const uint4*>(x + c * 8) : make_uint4(0, 0, 0, 0);
    const float2 g = group_stats(q);
    if ((lane & 15) == 0 && c < D / 8) st[(size_t)row * (D / 128) + c / 16] = g;
  }
}

}  // namespace

hipError_t launch_rowstats(const void* x_lo, const void* x_hi, int Nu, int T, int D, float2* st, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  rowstats_kernel<<<(T + 3) / 4, 256, 0, s>>>(x_lo, x_hi, Nu, T, D, st);
  return hipGetLastError();
}

hipError_t launch_colsum(const ColsumArgs& a, hipStream_t s) {
  const int rows = a.L * 4 * a.D;
  if (rows <= 0) return hipSuccess;
  colsum_kernel<<<(rows + 3) / 4, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_norm(int dtype, const NormArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int blocks = (a.T + 3) / 4;
  if (dtype == HSTU_F32)
    norm_kernel<float><<<blocks, 256, 0, s>>>(a);
  else
    norm_kernel<u16><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

int attn_block_rows(int dtype) { return dtype == HSTU_F32 ? attn_block_rows_f32() : attn_block_rows_bf16(); }

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int blocks = (a.T + 255) / 256 + (a.grid + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  plan_rows_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_upload(const UploadArgs& a, hipStream_t s) {
  if (a.words <= 0) return hipSuccess;
  if (a.words > kUploadWords) return hipErrorInvalidValue;
  upload_kernel<<<1, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_uvqk(int dtype, const UvqkArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return dtype == HSTU_F32 ? launch_uvqk_f32(a, s) : launch_uvqk_bf16(a, s);
}

hipError_t launch_attn(int dtype, int dh, const AttnArgs& a, int grid, hipStream_t s) {
  return dtype == HSTU_F32 ? launch_attn_f32(dh, a, grid, s) : launch_attn_bf16(dh, a, grid, s);
}

hipError_t launch_out(int dtype, const OutArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return dtype == HSTU_F32 ? launch_out_f32(a, s) : launch_out_bf16(a, s);
}

}  // namespace hstu
