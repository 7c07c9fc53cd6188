// Device helpers shared by the bfloat16 kernels (gfx950).
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_bf16, wave64): for
// D = A*B + C with A 32 x 16, B 16 x 32, lane l supplies A[l%32][8*(l/32) .. +8] and
// B[8*(l/32) .. +8][l%32]; it receives D[8*i + 4*(l/32) + j][l%32] in accumulator
// element 4*i + j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float bf2f_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Two floats -> two bfloat16 (hardware round to nearest even), packed low first.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float round_bf(float a) { return (float)(__bf16)a; }

// SiLU(x) = x / (1 + 2^(-x*log2(e))) with the hardware exp2 and reciprocal. For
// x -> -inf the exponential overflows to +inf and the result is -0; no NaN arises.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Sum over each group of 16 consecutive lanes, every lane of the group receiving it, by
// DPP lane moves (no LDS round trip). Lanes pair as i ^ 1, then i ^ 2; after these every
// lane of a quad holds the quad's sum, so the mirror within 8 (lane 7 - i) and within 16
// (lane 15 - i) add the neighbouring quad, then the neighbouring 8: the additions group
// the values exactly as the xor butterfly 1, 2, 4, 8 does. All 64 lanes must be active.
__device__ __forceinline__ float sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));    // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));    // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));   // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));   // row_mirror
  return v;
}

// Statistics of one row's 128-column group held by 16 consecutive lanes, 8 bfloat16
// values (one 16-byte chunk) each: {mean, M2} with M2 the sum of squared deviations
// from that mean, both float32 and every lane receiving them. Two passes over the
// values in registers: the deviations are taken from the group's own mean, so M2
// carries no cancellation however large the mean is against the spread. All 64 lanes
// must be active.
__device__ __forceinline__ float2 group_stats(uint4 q) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += bf2f_lo(w[e]) + bf2f_hi(w[e]);
  const float mean = sum16(s) * (1.0f / 128.0f);
  float d2 = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = bf2f_lo(w[e]) - mean, b = bf2f_hi(w[e]) - mean;
    d2 = __builtin_fmaf(a, a, __builtin_fmaf(b, b, d2));
  }
  return make_float2(mean, sum16(d2));
}

// Mean and variance of a whole row from its groups' {mean, M2}: the groups are merged
// one at a time by the pairwise update of Chan, Golub and LeVeque (1979): merging n
// values (mean ma, M2 Ma) with 128 more (mb, Mb) gives mean ma + d * 128 / (n + 128) and
// M2 Ma + Mb + d^2 * n * 128 / (n + 128), with d = mb - ma. Returns {mean, M2 / D}.
// One step of that merge: {mean, M2} of groups 0..i-1 and group i's {mean, M2}.
__device__ __forceinline__ void merge_group_step(float& mean, float& m2, float2 b, int i) {
  const float d = b.x - mean, f = 1.0f / (float)(i + 1);   // 128 / (n + 128) with n = 128 i
  mean = __builtin_fmaf(d, f, mean);
  m2 += b.y + d * d * (128.0f * (float)i * f);
}
__device__ __forceinline__ float2 merge_group_stats(const float2* g, int groups) {
  float mean = g[0].x, m2 = g[0].y;
  for (int i = 1; i < groups; ++i) merge_group_step(mean, m2, g[i], i);
  return make_float2(mean, m2 / (float)(128 * groups));
}

// Workgroup -> tile order that keeps neighbouring tiles on one XCD. Workgroups are
// dealt to the 8 XCDs round-robin; giving each XCD a contiguous run of tiles keeps
// tiles that share operand blocks inside one XCD's L2.
__device__ __forceinline__ int xcd_swizzle(int wg, int nwg) {
  const int per = nwg / 8, rem = nwg % 8;
  const int xcd = wg % 8, local = wg / 8;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

}  // namespace hstu
