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

}  // namespace

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
