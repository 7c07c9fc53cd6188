// bfloat16 kernels for gfx950 (CDNA4): bf16 MFMA (v_mfma_f32_32x32x16_bf16) with
// float32 accumulation, 64-wide wavefronts, LDS-staged tiles.
//
// Rounding to bfloat16 (hardware round-to-nearest-even conversion) happens exactly
// at: the normalised layer input; U, V, Q, K after the position bias; each attention weight SiLU(q.k); each
// attention output; the gate U*O; and X + Z.
//
// MFMA operand layout used throughout (32x32x16, wave64): for D = A*B + C with A
// 32xK16, B K16x32, lane l supplies A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32];
// it receives D[8*i + 4*(l/32) + j][l%32] in accumulator element 4*i + j.
#include <hip/hip_runtime.h>

#include "hstu_internal.h"

namespace hstu {
namespace {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float bf2f_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float round_bf(float a) { return (float)(__bf16)a; }

// SiLU(x) = x / (1 + 2^(-x*log2(e))): the hardware exp2 and reciprocal. For x -> -inf
// the exponential overflows to +inf and the result is -0; no NaN arises.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup -> tile order that keeps neighbouring tiles on one XCD. Workgroups are
// dealt to the 8 XCDs round-robin; giving each XCD a contiguous run of tiles keeps
// the tiles that share an A row block inside one XCD's L2.
__device__ __forceinline__ int xcd_swizzle(int wg, int nwg) {
  const int per = nwg / 8, rem = nwg % 8;
  const int xcd = wg % 8, local = wg / 8;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// ------------------------------------------------------------------ GEMM core
// C[M][N] = A[M][K] * W[N][K]^T on a 128 x 128 tile, K step 64, 256 threads as 2 x 2
// waves of 64 x 64. Accumulators hold C^T blocks (MFMA A operand = W rows), so a lane
// owns one output row and runs of 4 consecutive output columns.
constexpr int GM = 128, GN = 128, GK = 64, GLD = GK + 8;

struct GemmSmem {
  u16 a[GM * GLD];
  u16 b[GN * GLD];
};

template <typename ALoad>
__device__ __forceinline__ void gemm_core(const ALoad& aload, const u16* __restrict__ w, int K,
                                          int row0, int col0, f32x16 (&acc)[2][2], GemmSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1, l32 = lane & 31, hi = lane >> 5;
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 3, kc = (id & 7) * 8;
      ra[i] = aload(row0 + r, k0 + kc);
      rb[i] = *reinterpret_cast<const uint4*>(w + (size_t)(col0 + r) * K + k0 + kc);
    }
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  gload(0);
  for (int k0 = 0; k0 < K; k0 += GK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 3, kc = (id & 7) * 8;
      *reinterpret_cast<uint4*>(&sm.a[r * GLD + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&sm.b[r * GLD + kc]) = rb[i];
    }
    __syncthreads();
    if (k0 + GK < K) gload(k0 + GK);
#pragma unroll
    for (int kk = 0; kk < GK / 16; ++kk) {
      bf16x8 af[2], bw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.a[(wm * 64 + i * 32 + l32) * GLD + kk * 16 + hi * 8]));
        bw[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.b[(wn * 64 + i * 32 + l32) * GLD + kk * 16 + hi * 8]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(bw[j], af[i], acc[i][j]);
    }
  }
}

// A rows of the projection: the normalised layer input bf16((x - mean) * rstd),
// history rows then candidate rows.
struct XLoad {
  const u16* lo;
  const u16* hi;
  const float2* stats;
  int Nu, T, D;
  __device__ __forceinline__ uint4 operator()(int row, int k) const {
    if (row >= T) return make_uint4(0, 0, 0, 0);
    const u16* p = row < Nu ? lo + (size_t)row * D : hi + (size_t)(row - Nu) * D;
    const uint4 v = *reinterpret_cast<const uint4*>(p + k);
    const float2 st = stats[row];
    uint4 r;
    r.x = pack2((bf2f_lo(v.x) - st.x) * st.y, (bf2f_hi(v.x) - st.x) * st.y);
    r.y = pack2((bf2f_lo(v.y) - st.x) * st.y, (bf2f_hi(v.y) - st.x) * st.y);
    r.z = pack2((bf2f_lo(v.z) - st.x) * st.y, (bf2f_hi(v.z) - st.x) * st.y);
    r.w = pack2((bf2f_lo(v.w) - st.x) * st.y, (bf2f_hi(v.w) - st.x) * st.y);
    return r;
  }
};

// A rows of the output GEMM: [U | O | bf16(U*O)], 3D wide, built on the fly.
struct GateLoad {
  const u16* uvqk;
  const u16* o;
  int T, D;
  __device__ __forceinline__ uint4 operator()(int row, int k) const {
    if (row >= T) return make_uint4(0, 0, 0, 0);
    const u16* urow = uvqk + (size_t)row * 4 * D;
    const u16* orow = o + (size_t)row * D;
    if (k < D) return *reinterpret_cast<const uint4*>(urow + k);
    if (k < 2 * D) return *reinterpret_cast<const uint4*>(orow + (k - D));
    const uint4 u = *reinterpret_cast<const uint4*>(urow + (k - 2 * D));
    const uint4 v = *reinterpret_cast<const uint4*>(orow + (k - 2 * D));
    uint4 g;
    g.x = pack2(bf2f_lo(u.x) * bf2f_lo(v.x), bf2f_hi(u.x) * bf2f_hi(v.x));
    g.y = pack2(bf2f_lo(u.y) * bf2f_lo(v.y), bf2f_hi(u.y) * bf2f_hi(v.y));
    g.z = pack2(bf2f_lo(u.z) * bf2f_lo(v.z), bf2f_hi(u.z) * bf2f_hi(v.z));
    g.w = pack2(bf2f_lo(u.w) * bf2f_lo(v.w), bf2f_hi(u.w) * bf2f_hi(v.w));
    return g;
  }
};

__global__ __launch_bounds__(256) void uvqk_kernel(UvqkArgs a) {
  __shared__ GemmSmem sm;
  const int D = a.D, N = 4 * D, ncol = N / GN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int row0 = (tile / ncol) * GM, col0 = (tile % ncol) * GN;
  f32x16 acc[2][2];
  XLoad ld{(const u16*)a.x_lo, (const u16*)a.x_hi, a.stats, a.Nu, a.T, D};
  gemm_core(ld, (const u16*)a.w, D, row0, col0, acc, sm);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, l32 = lane & 31, hi = lane >> 5;
  const u16* pos = (const u16*)a.pos;
  u16* out = (u16*)a.uvqk;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = row0 + wm * 64 + i * 32 + l32;
    if (row >= a.T) continue;
    const int2 ri = a.row_info[row];
    const u16* prow = pos + (size_t)ri.y * 3 * D;
    const bool append = a.cache_k != nullptr && row < a.Nu;
    const size_t crow = append ? (size_t)a.users[ri.x].key_row + ri.y : 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + wn * 64 + j * 32 + g * 8 + hi * 4;
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
    }
  }
}

__global__ __launch_bounds__(256) void out_kernel(OutArgs a) {
  __shared__ GemmSmem sm;
  const int D = a.D, ncol = D / GN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int row0 = (tile / ncol) * GM, col0 = (tile % ncol) * GN;
  f32x16 acc[2][2];
  GateLoad ld{(const u16*)a.uvqk, (const u16*)a.o, a.T, D};
  gemm_core(ld, (const u16*)a.w, 3 * D, row0, col0, acc, sm);

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = row0 + wm * 64 + i * 32 + l32;
    if (row >= a.T) continue;
    const bool lo = row < a.Nu;
    const u16* x = lo ? (const u16*)a.x_lo + (size_t)row * D : (const u16*)a.x_hi + (size_t)(row - a.Nu) * D;
    u16* y = lo ? (u16*)a.y_lo + (size_t)row * D : (u16*)a.y_hi + (size_t)(row - a.Nu) * D;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + wn * 64 + j * 32 + g * 8 + hi * 4;
        const uint2 xv = *reinterpret_cast<const uint2*>(x + col);
        const float y0 = bf2f_lo(xv.x) + acc[i][j][4 * g + 0];
        const float y1 = bf2f_hi(xv.x) + acc[i][j][4 * g + 1];
        const float y2 = bf2f_lo(xv.y) + acc[i][j][4 * g + 2];
        const float y3 = bf2f_hi(xv.y) + acc[i][j][4 * g + 3];
        *reinterpret_cast<uint2*>(y + col) = make_uint2(pack2(y0, y1), pack2(y2, y3));
      }
    }
  }
}

// ------------------------------------------------------------------ attention
// One work item = (user, head, up to 128 query rows of one kind). Four waves own
// 32 query rows each; key blocks of 64 are staged in LDS (K row-major, V
// transposed). Per 32-key half: S^T = K Q^T (queries along lanes), mask + SiLU +
// bf16, then O^T += V^T A^T with the key order permuted identically on both operands.
// No softmax: partial sums over key blocks simply add; the 1/max_len scale is
// applied once to the float32 accumulator.
constexpr int ABM = 128, AKB = 64;

template <int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int KLD = DH + 8, VLD = AKB + 8;
  __shared__ __attribute__((aligned(16))) u16 sK[AKB * KLD];
  __shared__ __attribute__((aligned(16))) u16 sVt[DH * VLD];

  const int4 t = a.tiles[blockIdx.x];
  const UserRec u = a.users[t.x];
  const int head = t.y >> 1, q0 = t.z, nq = t.w;
  const bool cand = (t.y & 1) != 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int D = a.D;
  const size_t ld4 = 4 * (size_t)D;
  const int qloc = wv * 32 + l32;
  const bool qok = qloc < nq;
  const int qi = q0 + qloc;
  const size_t row = cand ? (size_t)a.Nu + u.coff + qi : (size_t)u.uoff + qi;
  const u16* uvqk = (const u16*)a.uvqk;

  bf16x8 qf[DH / 16];
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk)
    qf[kk] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(uvqk + row * ld4 + 2 * D + head * DH + kk * 16 + hi * 8)
                           : make_uint4(0, 0, 0, 0));

  const int key_end = cand ? u.m + u.n : u.m + q0 + nq;  // keys [0, key_end)
  const int qpos = u.m + qi;                             // history row: keys <= qpos
  f32x16 oacc[DH / 32];
#pragma unroll
  for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[mb][e] = 0.0f;

  const u16* kp = (const u16*)a.kbase + (size_t)u.key_row * a.ld + head * DH;
  const u16* vp = (const u16*)a.vbase + (size_t)u.key_row * a.ld + head * DH;

  for (int k0 = 0; k0 < key_end; k0 += AKB) {
    __syncthreads();
    for (int id = tid; id < AKB * DH / 8; id += 256) {
      const int key = id / (DH / 8), c8 = (id % (DH / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k0 + key < key_end) v = *reinterpret_cast<const uint4*>(kp + (size_t)(k0 + key) * a.ld + c8);
      *reinterpret_cast<uint4*>(&sK[key * KLD + c8]) = v;
    }
    for (int id = tid; id < AKB * DH / 8; id += 256) {
      const int key = id % AKB, c8 = (id / AKB) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k0 + key < key_end) v = *reinterpret_cast<const uint4*>(vp + (size_t)(k0 + key) * a.ld + c8);
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(c8 + 2 * e) * VLD + key] = (u16)(wds[e] & 0xffffu);
        sVt[(c8 + 2 * e + 1) * VLD + key] = (u16)(wds[e] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4*>(&sK[(kh * 32 + l32) * KLD + kk * 16 + hi * 8]));
        s = mfma32(kf, qf[kk], s);
      }
      // s[4*i + j] = q(row l32) . k(key k0 + kh*32 + 8*i + 4*hi + j)
      bf16x8 af[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kh * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
        const bool ok = key < key_end && (cand || key <= qpos);
        af[e >> 3][e & 7] = (__bf16)(ok ? silu(s[e]) : 0.0f);
      }
      // B operand chunk c, element e <-> key kh*32 + (2c + e/4)*8 + 4*hi + e%4; the
      // V^T operand reads the same keys for its dh row.
#pragma unroll
      for (int mb = 0; mb < DH / 32; ++mb) {
        const u16* vrow = &sVt[(mb * 32 + l32) * VLD + kh * 32 + hi * 4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint2 p0 = *reinterpret_cast<const uint2*>(vrow + (2 * c) * 8);
          const uint2 p1 = *reinterpret_cast<const uint2*>(vrow + (2 * c + 1) * 8);
          oacc[mb] = mfma32(as_bf16x8(make_uint4(p0.x, p0.y, p1.x, p1.y)), af[c], oacc[mb]);
        }
      }
    }
  }

  if (cand) {
    // the candidate's own key and value: a_self = bf16(SiLU(q . k_self))
    const u16* krow = uvqk + row * ld4 + 3 * D + head * DH;
    const u16* vrow = uvqk + row * ld4 + 1 * D + head * DH;
    float part = 0.0f;
    if (qok) {
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + kk * 16 + hi * 8);
        const uint32_t wds[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part += (float)qf[kk][2 * e] * bf2f_lo(wds[e]);
          part += (float)qf[kk][2 * e + 1] * bf2f_hi(wds[e]);
        }
      }
    }
    const float dot = part + __shfl_xor(part, 32);
    const float as = qok ? round_bf(silu(dot)) : 0.0f;
    if (qok) {
#pragma unroll
      for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 vv = *reinterpret_cast<const uint2*>(vrow + mb * 32 + i * 8 + hi * 4);
          oacc[mb][4 * i + 0] += as * bf2f_lo(vv.x);
          oacc[mb][4 * i + 1] += as * bf2f_hi(vv.x);
          oacc[mb][4 * i + 2] += as * bf2f_lo(vv.y);
          oacc[mb][4 * i + 3] += as * bf2f_hi(vv.y);
        }
    }
  }
  if (qok) {
    u16* orow = (u16*)a.o + row * D + head * DH;
#pragma unroll
    for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 pk = make_uint2(pack2(a.inv * oacc[mb][4 * i + 0], a.inv * oacc[mb][4 * i + 1]),
                                    pack2(a.inv * oacc[mb][4 * i + 2], a.inv * oacc[mb][4 * i + 3]));
        *reinterpret_cast<uint2*>(orow + mb * 32 + i * 8 + hi * 4) = pk;
      }
  }
}

}  // namespace

hipError_t launch_uvqk_bf16(const UvqkArgs& a, hipStream_t s) {
  const int tiles = ((a.T + GM - 1) / GM) * (4 * a.D / GN);
  uvqk_kernel<<<tiles, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s) {
  const int tiles = ((a.T + GM - 1) / GM) * (a.D / GN);
  out_kernel<<<tiles, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(int dh, const AttnArgs& a, int ntiles, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  if (dh == 64)
    attn_kernel<64><<<ntiles, 256, 0, s>>>(a);
  else if (dh == 128)
    attn_kernel<128><<<ntiles, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int attn_block_rows_bf16() { return ABM; }

}  // namespace hstu
