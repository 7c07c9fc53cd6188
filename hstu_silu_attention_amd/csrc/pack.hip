// History tokens from per-event context and action embeddings (the two input forms of
// the DLRMv3 page's action-embedding paragraph, section "Model selection").
//
// Both forms are pure streaming passes: every 16-byte chunk of the output is made
// from one or two 16-byte chunks of the inputs, one thread per output chunk, so
// consecutive lanes read and write consecutive 16 bytes of one row. The interleaved
// form moves bytes unchanged; the merged form adds in float32 and rounds once to
// the storage type.
#include <hip/hip_runtime.h>

#include "hstu.h"
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kPackThreads = 256;

// Output row r of the interleaved history is row r / 2 of the context (r even) or of
// the action (r odd). `cpr` is the row length in 16-byte chunks.
__global__ __launch_bounds__(kPackThreads) void pack_interleave_kernel(
    const uint4* __restrict__ ctx, const uint4* __restrict__ act, uint4* __restrict__ out,
    int chunks, int cpr) {
  const int q = blockIdx.x * kPackThreads + threadIdx.x;
  if (q >= chunks) return;
  const int r = q / cpr, c = q - r * cpr;
  const uint4* src = (r & 1) ? act : ctx;
  out[q] = src[(r >> 1) * cpr + c];
}

// Two bfloat16 pairs -> their sums, each rounded once to bfloat16 (nearest even). The
// float32 sum of two bfloat16 values is exact unless their exponents differ by more
// than 16; then the smaller one is below half a bfloat16 unit of the larger one and
// both roundings give the larger value.
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t x, uint32_t y) {
  return pack2(bf2f_lo(x) + bf2f_lo(y), bf2f_hi(x) + bf2f_hi(y));
}

__global__ __launch_bounds__(kPackThreads) void pack_sum_bf16_kernel(
    const uint4* __restrict__ ctx, const uint4* __restrict__ act, uint4* __restrict__ out,
    int chunks) {
  const int q = blockIdx.x * kPackThreads + threadIdx.x;
  if (q >= chunks) return;
  const uint4 x = ctx[q], y = act[q];
  out[q] = make_uint4(add_bf16x2(x.x, y.x), add_bf16x2(x.y, y.y), add_bf16x2(x.z, y.z),
                      add_bf16x2(x.w, y.w));
}

__global__ __launch_bounds__(kPackThreads) void pack_sum_f32_kernel(
    const float4* __restrict__ ctx, const float4* __restrict__ act, float4* __restrict__ out,
    int chunks) {
  const int q = blockIdx.x * kPackThreads + threadIdx.x;
  if (q >= chunks) return;
  const float4 x = ctx[q], y = act[q];
  out[q] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
}

// dst[c][r] = src[r][c] on 64 x 64 tiles through LDS (rows padded by one element), so
// both the reads of src rows and the writes of dst rows are consecutive per wave.
// Elements are moved as bits. Block (bx, by, z) owns rows 64 by.. and columns 64 bx..
// of matrix z of the list: one launch moves every matrix of a list (a model's layers),
// which keeps enough workgroups in flight to hide the memory latency.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeList t) {
  const T* __restrict__ src = static_cast<const T*>(t.src[blockIdx.z]);
  T* __restrict__ dst = static_cast<T*>(t.dst[blockIdx.z]);
  const int rows = t.rows, cols = t.cols;
  __shared__ T tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ty + 4 * i, c = c0 + tx;
    if (r < rows && c < cols) tile[ty + 4 * i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty + 4 * i, r = r0 + tx;   // dst row c, column r
    if (c < cols && r < rows) dst[(size_t)c * rows + r] = tile[tx][ty + 4 * i];
  }
}

// dst[i] = float(src[i]) for a bfloat16 src: the bits move to the upper half.
__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst,
                                                         int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float((uint32_t)src[i] << 16);
}

}  // namespace

hipError_t launch_widen_bf16(const void* src, float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  widen_bf16_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(src), dst, (int)n);
  return hipGetLastError();
}

// rows * cols < 2^31 and both > 0 (checked by the caller); esize 2 or 4; 1 <=
// kTransposeList.
hipError_t launch_transpose_list(int esize, const TransposeList& t, hipStream_t s) {
  const dim3 grid((t.cols + 63) / 64, (t.rows + 63) / 64, t.count);
  if (grid.y > 65535 || t.count < 1 || t.count > kTransposeList) return hipErrorInvalidValue;
  if (esize == 2)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>(t);
  else
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>(t);
  return hipGetLastError();
}

hipError_t launch_transpose(int esize, const void* src, void* dst, int rows, int cols, hipStream_t s) {
  TransposeList t{};
  t.src[0] = src;
  t.dst[0] = dst;
  t.rows = rows;
  t.cols = cols;
  t.count = 1;
  return launch_transpose_list(esize, t, s);
}

// `chunks` counts 16-byte chunks of the output (< 2^31, checked by the caller).
hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  if (a.chunks == 0) return hipSuccess;
  const int grid = (a.chunks + kPackThreads - 1) / kPackThreads;
  if (a.interleave)
    pack_interleave_kernel<<<grid, kPackThreads, 0, s>>>((const uint4*)a.ctx, (const uint4*)a.act,
                                                         (uint4*)a.out, a.chunks, a.cpr);
  else if (a.bf16)
    pack_sum_bf16_kernel<<<grid, kPackThreads, 0, s>>>((const uint4*)a.ctx, (const uint4*)a.act,
                                                       (uint4*)a.out, a.chunks);
  else
    pack_sum_f32_kernel<<<grid, kPackThreads, 0, s>>>((const float4*)a.ctx, (const float4*)a.act,
                                                      (float4*)a.out, a.chunks);
  return hipGetLastError();
}

}  // namespace hstu
