// Candidate scoring head: a top MLP over candidate rows, then the sigmoid of each output
// (the DLRMv3 page keeps a top-layer MLP for the final prediction, section "Model
// selection"; the TorchRec tutorial page, section 1.1, takes the probability as the
// sigmoid of the top MLP's output). Hidden layers are affine maps followed by ReLU; the
// last layer gives one logit per outcome.
//
// One workgroup owns a block of candidate rows for the whole head: its activations stay
// in LDS from layer to layer, so the head reads each candidate row once and writes only
// the probabilities. Weights (at most a few hundred KB) are read from L2 by every
// workgroup.
#include <hip/hip_runtime.h>

#include "hstu.h"
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {
namespace {

// ------------------------------------------------------------------ bfloat16 (MFMA)
//
// 64 rows per workgroup, 4 waves. A hidden layer computes H^T = W X^T with 32x32x16
// MFMAs: W (output features x K) is the A operand, read from global memory 16 bytes
// per lane along K; the activations X (rows x K) are the B operand, read from LDS.
// Wave w owns output features [w N/4, (w+1) N/4) for all 64 rows. A lane then holds,
// for its row l % 32 of each 32-row half, 4 consecutive output features per group of
// 8, which it writes back to LDS as one 8-byte store after ReLU and rounding.
constexpr int kSRows = 64, kSThreads = 256, kSStride = kMaxHeadWidth + 8;  // LDS row pitch (elements)

template <int NI>
__device__ __forceinline__ void head_layer_bf16(u16* act, const u16* __restrict__ w, const u16* __restrict__ b,
                                                int K, int N) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int n0 = wv * (N / 4);
  f32x16 acc[NI][2];
#pragma unroll
  for (int j = 0; j < NI; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;
  // W fragments of one 32-wide K step: [tile j][sub-step s]
  const u16* wrow[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) wrow[j] = w + (size_t)(n0 + j * 32 + l32) * K + hi * 8;
  uint4 wf[2][NI][2];
#pragma unroll
  for (int j = 0; j < NI; ++j)
#pragma unroll
    for (int s = 0; s < 2; ++s) wf[0][j][s] = *reinterpret_cast<const uint4*>(wrow[j] + s * 16);
  const int steps = K / 32;
  for (int t = 0; t < steps; t += 2) {
    // two K steps per iteration so that the register buffers have fixed names
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int st = t + u;
      const int cur = u, nxt = u ^ 1;
      if (st + 1 < steps) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            wf[nxt][j][s] = *reinterpret_cast<const uint4*>(wrow[j] + (st + 1) * 32 + s * 16);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int k = st * 32 + s * 16 + hi * 8;
        bf16x8 xf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(act + (i * 32 + l32) * kSStride + k));
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[j][i] = mfma32(as_bf16x8(wf[cur][j][s]), xf[i], acc[j][i]);
      }
    }
  }
  __syncthreads();   // every wave has read the layer input
#pragma unroll
  for (int j = 0; j < NI; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + j * 32 + g * 8 + hi * 4;
      const float b0 = bf2f(b[n]), b1 = bf2f(b[n + 1]), b2 = bf2f(b[n + 2]), b3 = bf2f(b[n + 3]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x16& a = acc[j][i];
        const uint2 v = make_uint2(pack2(fmaxf(a[4 * g] + b0, 0.0f), fmaxf(a[4 * g + 1] + b1, 0.0f)),
                                   pack2(fmaxf(a[4 * g + 2] + b2, 0.0f), fmaxf(a[4 * g + 3] + b3, 0.0f)));
        *reinterpret_cast<uint2*>(act + (i * 32 + l32) * kSStride + n) = v;
      }
    }
  __syncthreads();   // the layer output is complete
}

// Logistic function without overflow: exp(-|z|) is at most 1.
__device__ __forceinline__ float sigmoid(float z) {
  const float e = __expf(-fabsf(z));
  return z >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}

__global__ __launch_bounds__(kSThreads, 2) void score_bf16_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) u16 act[kSRows * kSStride];
  const int row0 = blockIdx.x * kSRows;
  // the candidate rows, 16 bytes per thread and step; rows past the end read as zero
  const int cpr = a.D / 8;
  for (int q = threadIdx.x; q < kSRows * cpr; q += kSThreads) {
    const int r = q / cpr, c = q - r * cpr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < a.rows) v = *(reinterpret_cast<const uint4*>((const u16*)a.x + (size_t)(row0 + r) * a.D) + c);
    *reinterpret_cast<uint4*>(act + r * kSStride + c * 8) = v;
  }
  __syncthreads();
  int K = a.D;
  for (int l = 0; l + 1 < a.layers; ++l) {
    const int N = a.width[l];
    const u16* w = (const u16*)a.w[l];
    const u16* b = (const u16*)a.b[l];
    if (N == 512) head_layer_bf16<4>(act, w, b, K, N);
    else if (N == 256) head_layer_bf16<2>(act, w, b, K, N);
    else if (N == 384) head_layer_bf16<3>(act, w, b, K, N);
    else head_layer_bf16<1>(act, w, b, K, N);
    K = N;
  }
  // Last layer: four lanes per row, each summing a quarter of K, then a butterfly.
  const int r = threadIdx.x >> 2, p = threadIdx.x & 3;
  const int kq = K / 4;
  const u16* xr = act + r * kSStride + p * kq;
  const u16* wl = (const u16*)a.w[a.layers - 1];
  const u16* bl = (const u16*)a.b[a.layers - 1];
  for (int o = 0; o < a.outcomes; ++o) {
    const u16* wo = wl + (size_t)o * K + p * kq;
    float s = 0.0f;
    for (int k = 0; k < kq; k += 8) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xr + k);
      const uint4 wv = *reinterpret_cast<const uint4*>(wo + k);
      const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(bf2f_lo(xs[e]), bf2f_lo(ws[e]), s);
        s = fmaf(bf2f_hi(xs[e]), bf2f_hi(ws[e]), s);
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (p == 0 && row0 + r < a.rows) a.prob[(size_t)(row0 + r) * a.outcomes + o] = sigmoid(s + bf2f(bl[o]));
  }
}

// ------------------------------------------------------------------ float32 (VALU)
//
// 16 rows per workgroup; activations ping-pong between two LDS buffers. Thread t
// computes output features t and t + 256 of every row, reading its weight rows 16 bytes
// at a time and the activations as LDS broadcasts.
constexpr int kFRows = 16, kFThreads = 256;

__global__ __launch_bounds__(kFThreads) void score_f32_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) float buf[2][kFRows * kMaxHeadWidth];
  const int row0 = blockIdx.x * kFRows;
  for (int q = threadIdx.x; q < kFRows * a.D; q += kFThreads) {
    const int r = q / a.D, c = q - r * a.D;
    buf[0][r * kMaxHeadWidth + c] = row0 + r < a.rows ? ((const float*)a.x)[(size_t)(row0 + r) * a.D + c] : 0.0f;
  }
  __syncthreads();
  int K = a.D, in = 0;
  for (int l = 0; l < a.layers; ++l) {
    const bool last = l + 1 == a.layers;
    const int N = last ? a.outcomes : a.width[l];
    const float* w = (const float*)a.w[l];
    const float* b = (const float*)a.b[l];
    const float* x = buf[in];
    for (int n = threadIdx.x; n < N; n += kFThreads) {
      float acc[kFRows];
#pragma unroll
      for (int r = 0; r < kFRows; ++r) acc[r] = 0.0f;
      const float* wn = w + (size_t)n * K;
      for (int k = 0; k < K; k += 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(wn + k);
#pragma unroll
        for (int r = 0; r < kFRows; ++r) {
          const float4 x4 = *reinterpret_cast<const float4*>(x + r * kMaxHeadWidth + k);
          acc[r] = fmaf(x4.x, w4.x, acc[r]);
          acc[r] = fmaf(x4.y, w4.y, acc[r]);
          acc[r] = fmaf(x4.z, w4.z, acc[r]);
          acc[r] = fmaf(x4.w, w4.w, acc[r]);
        }
      }
      const float bn = b[n];
#pragma unroll
      for (int r = 0; r < kFRows; ++r) {
        if (last) {
          if (row0 + r < a.rows) a.prob[(size_t)(row0 + r) * a.outcomes + n] = sigmoid(acc[r] + bn);
        } else {
          buf[in ^ 1][r * kMaxHeadWidth + n] = fmaxf(acc[r] + bn, 0.0f);
        }
      }
    }
    __syncthreads();
    in ^= 1;
    K = N;
  }
}

}  // namespace

int score_rows_per_block(int dtype) { return dtype == HSTU_BF16 ? kSRows : kFRows; }

hipError_t launch_score(int dtype, const ScoreArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    score_bf16_kernel<<<(a.rows + kSRows - 1) / kSRows, kSThreads, 0, s>>>(a);
  } else {
    score_f32_kernel<<<(a.rows + kFRows - 1) / kFRows, kFThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace hstu
