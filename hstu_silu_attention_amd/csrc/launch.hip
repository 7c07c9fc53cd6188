// The jagged row planner kernel and the per-dtype launch dispatch.
#include <hip/hip_runtime.h>

#include "../../include/hstu.h"
#include "hstu_internal.h"

namespace hstu {

hipError_t launch_uvqk_bf16(const UvqkArgs& a, hipStream_t s);
hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(int dh, const AttnArgs& a, int ntiles, hipStream_t s);
int attn_block_rows_bf16();
hipError_t launch_uvqk_f32(const UvqkArgs& a, hipStream_t s);
hipError_t launch_out_f32(const OutArgs& a, hipStream_t s);
hipError_t launch_attn_f32(int dh, const AttnArgs& a, int ntiles, hipStream_t s);
int attn_block_rows_f32();

namespace {

// Packed row r -> {user, absolute position}. History rows [0, Nu) belong to the user
// whose history segment holds r, at position m + (r - uoff); candidate rows
// [Nu, T) to the user whose candidate segment holds r - Nu, all at position m + n.
// The user is the last one whose segment starts at or before r (segments of empty
// users start where the next one does).
__global__ __launch_bounds__(256) void plan_rows_kernel(PlanArgs a) {
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ float load_f(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// One wave per row: two passes over the row (mean, then the mean squared deviation),
// each reduced across the wave in a fixed butterfly order, so a row's statistics
// depend on that row alone.
template <typename T>
__global__ __launch_bounds__(256) void row_stats_kernel(StatsArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.T) return;
  const int D = a.D;
  const T* x = row < a.Nu ? (const T*)a.x_lo + (size_t)row * D : (const T*)a.x_hi + (size_t)(row - a.Nu) * D;
  float s = 0.0f;
  for (int k = lane; k < D; k += 64) s += load_f(x + k);
  const float mean = wave_sum(s) / (float)D;
  float q = 0.0f;
  for (int k = lane; k < D; k += 64) {
    const float d = load_f(x + k) - mean;
    q += d * d;
  }
  const float var = wave_sum(q) / (float)D;
  if (lane == 0) a.stats[row] = make_float2(mean, 1.0f / sqrtf(var + kNormEps));
}

}  // namespace

hipError_t launch_stats(int dtype, const StatsArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int blocks = (a.T + 3) / 4;
  if (dtype == HSTU_F32)
    row_stats_kernel<float><<<blocks, 256, 0, s>>>(a);
  else
    row_stats_kernel<uint16_t><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

int attn_block_rows(int dtype) { return dtype == HSTU_F32 ? attn_block_rows_f32() : attn_block_rows_bf16(); }

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  plan_rows_kernel<<<(a.T + 255) / 256, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_uvqk(int dtype, const UvqkArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return dtype == HSTU_F32 ? launch_uvqk_f32(a, s) : launch_uvqk_bf16(a, s);
}

hipError_t launch_attn(int dtype, int dh, const AttnArgs& a, int ntiles, hipStream_t s) {
  return dtype == HSTU_F32 ? launch_attn_f32(dh, a, ntiles, s) : launch_attn_bf16(dh, a, ntiles, s);
}

hipError_t launch_out(int dtype, const OutArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return dtype == HSTU_F32 ? launch_out_f32(a, s) : launch_out_bf16(a, s);
}

}  // namespace hstu
